"""LookupDrafter: the drafting hot path for one batch of requests, as an object.

It owns what the C entry points leave to the caller -- the lookup and decode
workspaces, the per-request scheduler state, optional acceptance telemetry,
an optional incremental index and the sampled-verification workspace -- and
exposes the path's calls on device tensors.  Everything runs in the HIP
library (liblcd.so) on the current torch stream; nothing here computes.

    d = LookupDrafter(B=64, max_len=40_000, device="cuda:0")
    out = d.step(hist, row_off, lens, cap, model_draft, target)      # one decode step
    m, e, draft = d.propose(hist, row_off, lens)                      # lookup only
"""

from __future__ import annotations

from typing import Optional

from . import (DRAFT_STRIDE, LookupIndex, Params, alloc_decode_workspace, alloc_rejection_workspace,
               alloc_telemetry, alloc_workspace, default_params, fuse_verify_block, lookup_decode_step,
               lookup_propose, rejection_accept, telemetry_reduce)


class LookupDrafter:
    """Drafting state for B requests whose histories are at most ``max_len``
    tokens long (the launch bound of the lookup; rows may be ragged).

    telemetry: keep per-request acceptance counters (updated by every step).
    index_cap: per-row capacities (host array) to answer lookups from the
    incremental n-gram index instead of scanning (build it with build_index).
    """

    def __init__(self, B: int, max_len: int, device, params: Optional[Params] = None,
                 telemetry: bool = False, index_cap=None):
        import torch
        self.B = int(B)
        self.max_len = int(max_len)
        self.device = torch.device(device)
        self.params = params or default_params()
        dev = self.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.ws = alloc_workspace(self.B, dev)
        self.decode_ws = alloc_decode_workspace(self.B, self.max_len, dev, self.params)
        self.state = torch.zeros((self.B, 3), **i32)
        self.match_len = torch.empty(self.B, **i32)
        self.match_end = torch.empty(self.B, **i32)
        self.draft = torch.empty((self.B, DRAFT_STRIDE), **i32)
        self.block = torch.empty((self.B, DRAFT_STRIDE), **i32)
        self.block_len = torch.empty(self.B, **i32)
        self.accept = torch.empty(self.B, **i32)
        self.long_next = torch.empty(self.B, **i32)
        self.lens_next = torch.empty(self.B, **i32)
        self.telemetry = alloc_telemetry(self.B, dev) if telemetry else None
        self.index = LookupIndex(index_cap, dev, self.params) if index_cap is not None else None
        self._rej_ws = None
        self._rej_vocab = None

    # -- lookup ------------------------------------------------------------
    def build_index(self, hist, row_off, lens):
        """Index the rows' current histories (only with index_cap)."""
        if self.index is None:
            raise RuntimeError("LookupDrafter was created without index_cap")
        self.index.build(hist, row_off, lens, self.max_len)

    def propose(self, hist, row_off, lens):
        """Longest-suffix lookup and 15-token draft of every request: returns
        (match_len, match_end, draft), device tensors owned by the drafter."""
        if self.index is not None:
            self.index.propose(hist, row_off, lens, self.match_len, self.match_end, self.draft)
        else:
            lookup_propose(hist, row_off, lens, self.max_len, self.ws, self.match_len,
                           self.match_end, self.draft, self.params)
        return self.match_len, self.match_end, self.draft

    def fuse(self, model_draft, model_mask=None):
        """Verify block of the last proposal under each request's current mode."""
        fuse_verify_block(self.draft, self.match_len, model_draft, self.state[:, 0].contiguous(),
                          self.block, self.block_len, self.params, model_mask=model_mask)
        return self.block, self.block_len

    # -- whole greedy step ---------------------------------------------------
    def step(self, hist, row_off, lens, cap, model_draft, target, append: bool = True,
             separate: bool = False):
        """One greedy decode step in one kernel (lookup, fusion, acceptance,
        append, scheduler update; telemetry when enabled): lookup_decode_step,
        or lookup_index_decode_step with the index.  ``separate`` runs the
        index path as its four entry points instead (same outputs).  ``lens``
        is updated in place: lookup_decode_step writes the new lengths to the
        drafter's second length array, which is then copied into ``lens`` on
        the same stream (callers that alternate two arrays themselves call
        lookup_decode_step directly)."""
        if self.index is not None and not separate:
            self.index.decode_step(hist, row_off, lens, cap, model_draft, target, self.state,
                                   self.match_len, self.match_end, self.draft, self.block,
                                   self.block_len, self.accept, self.long_next, append,
                                   telemetry=self.telemetry)
        elif self.index is not None:
            from . import greedy_accept, lookup_schedule_step, telemetry_update
            self.propose(hist, row_off, lens)
            long_used = self.state[:, 0].clone()
            fuse_verify_block(self.draft, self.match_len, model_draft, long_used, self.block,
                              self.block_len, self.params)
            if append:
                greedy_accept(self.block, self.block_len, target, self.accept, hist=hist,
                              row_off=row_off, lens=lens, cap=cap)
            else:
                greedy_accept(self.block, self.block_len, target, self.accept)
            lookup_schedule_step(self.state, self.match_len, self.accept, self.block_len,
                                 self.long_next, self.params)
            if self.telemetry is not None:
                telemetry_update(self.telemetry, self.match_len, self.draft, model_draft, long_used,
                                 self.block_len, self.accept, self.long_next, self.params)
        else:
            lookup_decode_step(hist, row_off, lens, cap, self.max_len, model_draft, target,
                               self.state, self.decode_ws, self.match_len, self.match_end,
                               self.draft, self.block, self.block_len, self.accept,
                               self.long_next, append, self.params, telemetry=self.telemetry,
                               lens_out=self.lens_next if append else None)
            if append:
                lens.copy_(self.lens_next)
        return dict(match_len=self.match_len, match_end=self.match_end, draft=self.draft,
                    block=self.block, block_len=self.block_len, accept=self.accept,
                    long_next=self.long_next)

    # -- sampled verification ------------------------------------------------
    def verify_sampled(self, target_probs, u_accept, u_sample, emitted, model_mask=None,
                       model_probs=None, hist=None, row_off=None, lens=None, cap=None):
        """Rejection-sampling verification of the current block (point-mass
        lookup slots); writes self.accept and `emitted` [B,16]."""
        V = int(target_probs.shape[2])
        if self._rej_ws is None or self._rej_vocab != V:
            self._rej_ws = alloc_rejection_workspace(self.B, V, self.device)
            self._rej_vocab = V
        rejection_accept(self.block, self.block_len, target_probs, u_accept, u_sample, self._rej_ws,
                         self.accept, emitted, model_mask=model_mask, model_probs=model_probs,
                         hist=hist, row_off=row_off, lens=lens, cap=cap)
        return self.accept

    # -- diagnostics -----------------------------------------------------------
    def telemetry_totals(self, class_id, K: int):
        """Per-class totals of the acceptance counters: int64 [K,32]."""
        if self.telemetry is None:
            raise RuntimeError("LookupDrafter was created without telemetry")
        return telemetry_reduce(self.telemetry, class_id, K)
