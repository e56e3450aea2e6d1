"""Decode-step simulation used by the tests.

One step, for every request of a workload: lookup on the current history,
fusion with the draft model's proposal under the current block mode, greedy
acceptance against the target's argmax tokens (which appends the emitted
tokens to the history), then the scheduler update that picks the next step's
mode.  The truth stream plays the target model, so the emitted stream must
equal it whatever the drafts are.

``simulate_oracle`` drives the CPU oracle on host arrays; ``simulate_gpu``
drives the HIP library through its Python binding on device tensors.  Both take
their per-step inputs from the workload generator only.
"""

from __future__ import annotations

import numpy as np

from context_lookup_drafting_amd.workloads import Workload, pack_rows, N_TARGET


def _extra(steps):
    return N_TARGET * (steps + 1)


def simulate_oracle(w: Workload, steps: int, params=None, record: bool = True):
    import oracle
    params = params or oracle.default_params()
    flat, row_off, lens, cap = pack_rows(w.hists, extra=_extra(steps))
    B = w.B
    state = np.zeros((B, 3), np.int32)
    long_mode = np.zeros(B, np.int32)
    tele = np.zeros((B, 32), np.uint32)
    pos = np.zeros(B, np.int64)
    recs = []
    emitted = [[] for _ in range(B)]
    for t in range(steps):
        m, e, d = oracle.lookup_propose(flat, row_off, lens, params)
        q, tgt = w.step_inputs(pos, t)
        blk, bl = oracle.fuse_verify_block(d, m, q, long_mode, params)
        acc = oracle.greedy_accept(blk, bl, tgt, flat, row_off, lens, cap)
        long_used = long_mode.copy()
        long_mode = oracle.lookup_schedule_step(state, m, acc, bl, params)
        oracle.telemetry_update(tele, m, d, q, long_used, bl, acc, long_mode, params)
        for r in range(B):
            if acc[r] >= 0:
                emitted[r].extend(tgt[r, :acc[r] + 1].tolist())
        pos = pos + np.maximum(acc, 0) + 1
        if record:
            recs.append(dict(m=m, e=e, d=d, q=q, tgt=tgt, long=long_used, block=blk,
                             blk=bl, acc=acc, state=state.copy(), long_next=long_mode.copy()))
    return dict(recs=recs, emitted=emitted, lens=lens, flat=flat, row_off=row_off, tele=tele)


def simulate_gpu(w: Workload, steps: int, params=None, record: bool = True, device="cuda:0",
                 index: bool = False, fp_bits: int = 0):
    """The decode loop through the four separate entry points; with ``index``
    the lookup comes from lookup_index_propose (built once from the prompts,
    updated by every call) instead of lookup_propose."""
    import torch
    import context_lookup_drafting_amd as lcd
    params = params or lcd.default_params()
    flat, row_off, lens, cap = pack_rows(w.hists, extra=_extra(steps))
    B = w.B
    dev = torch.device(device)
    h_d = torch.from_numpy(flat).to(dev)
    ro_d = torch.from_numpy(row_off).to(dev)
    len_d = torch.from_numpy(lens.copy()).to(dev)
    cap_d = torch.from_numpy(cap).to(dev)
    ws = lcd.alloc_workspace(B, dev)
    state = torch.zeros((B, 3), dtype=torch.int32, device=dev)
    long_mode = torch.zeros(B, dtype=torch.int32, device=dev)
    m = torch.empty(B, dtype=torch.int32, device=dev)
    e = torch.empty(B, dtype=torch.int32, device=dev)
    d = torch.empty((B, 15), dtype=torch.int32, device=dev)
    block = torch.empty((B, 15), dtype=torch.int32, device=dev)
    bl = torch.empty(B, dtype=torch.int32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    long_next = torch.empty(B, dtype=torch.int32, device=dev)
    tele = lcd.alloc_telemetry(B, dev)
    pos = np.zeros(B, np.int64)
    recs = []
    emitted = [[] for _ in range(B)]
    max_len = int(lens.max()) + _extra(steps) if B else 0
    idx = None
    if index:
        idx = lcd.LookupIndex(cap, dev, params, fp_bits=fp_bits)
        idx.build(h_d, ro_d, len_d, max_len)
    for t in range(steps):
        if idx is not None:
            idx.propose(h_d, ro_d, len_d, m, e, d)
        else:
            lcd.lookup_propose(h_d, ro_d, len_d, max_len, ws, m, e, d, params)
        q, tgt = w.step_inputs(pos, t)
        q_d = torch.from_numpy(q).to(dev)
        tgt_d = torch.from_numpy(tgt).to(dev)
        lcd.fuse_verify_block(d, m, q_d, long_mode, block, bl, params)
        lcd.greedy_accept(block, bl, tgt_d, acc, hist=h_d, row_off=ro_d, lens=len_d, cap=cap_d)
        long_used = long_mode.clone()
        lcd.lookup_schedule_step(state, m, acc, bl, long_next, params)
        lcd.telemetry_update(tele, m, d, q_d, long_used, bl, acc, long_next, params)
        long_mode.copy_(long_next)
        acc_h = acc.cpu().numpy()
        for r in range(B):
            if acc_h[r] >= 0:
                emitted[r].extend(tgt[r, :acc_h[r] + 1].tolist())
        pos = pos + np.maximum(acc_h, 0) + 1
        if record:
            recs.append(dict(m=m.cpu().numpy(), e=e.cpu().numpy(), d=d.cpu().numpy(), q=q,
                             tgt=tgt, long=long_used.cpu().numpy(), block=block.cpu().numpy(),
                             blk=bl.cpu().numpy(), acc=acc_h, state=state.cpu().numpy(),
                             long_next=long_next.cpu().numpy()))
    torch.cuda.synchronize()
    return dict(recs=recs, emitted=emitted, lens=len_d.cpu().numpy(), flat=h_d.cpu().numpy(),
                row_off=row_off, ws=ws, tele=tele.cpu().numpy().view(np.uint32),
                indexed_len=None if idx is None else idx.indexed_len.cpu().numpy())


def simulate_gpu_fused(w: Workload, steps: int, params=None, record: bool = True, device="cuda:0"):
    """Same decode loop through the fused lookup_decode_step entry point (the
    block mode of each step comes from the scheduler state itself)."""
    from context_lookup_drafting_amd.decode_sim import run_fused
    res = run_fused(w, steps, params, device, record)
    res.pop("tele_d")
    return res


def simulate_gpu_index_fused(w: Workload, steps: int, params=None, record: bool = True,
                             device="cuda:0", fp_bits: int = 0, separate_every: int = 0,
                             rebuild_at=()):
    """The decode loop through lookup_index_decode_step: one kernel per step,
    the lookup answered from the index (built once from the prompts) and the
    step's appended tokens indexed by the next call.  With separate_every = k,
    every k-th step goes through the four entry points instead (the index
    propose, then fusion, the appending greedy accept and the scheduler), so
    the next call finds histories grown behind its back; before each step in
    rebuild_at the index is built again from the current histories."""
    import torch
    import context_lookup_drafting_amd as lcd
    params = params or lcd.default_params()
    flat, row_off, lens, cap = pack_rows(w.hists, extra=_extra(steps))
    B = w.B
    dev = torch.device(device)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h_d, ro_d, len_d, cap_d = t(flat), t(row_off), t(lens.copy()), t(cap)
    state = torch.zeros((B, 3), dtype=torch.int32, device=dev)
    mk = lambda *s: torch.empty(s, dtype=torch.int32, device=dev)
    m, e, d, block, bl, acc, long_next = mk(B), mk(B), mk(B, 15), mk(B, 15), mk(B), mk(B), mk(B)
    tele = lcd.alloc_telemetry(B, dev)
    max_len = int(lens.max()) + _extra(steps) if B else 0
    idx = lcd.LookupIndex(cap, dev, params, fp_bits=fp_bits)
    idx.build(h_d, ro_d, len_d, max_len)
    pos = np.zeros(B, np.int64)
    recs = []
    emitted = [[] for _ in range(B)]
    for step in range(steps):
        q, tgt = w.step_inputs(pos, step)
        long_used = state[:, 0].clone()
        if step in rebuild_at:
            idx.build(h_d, ro_d, len_d, max_len)
        if separate_every and step % separate_every == separate_every - 1:
            q_d, tgt_d = t(q), t(tgt)
            idx.propose(h_d, ro_d, len_d, m, e, d)
            lcd.fuse_verify_block(d, m, q_d, long_used, block, bl, params)
            lcd.greedy_accept(block, bl, tgt_d, acc, hist=h_d, row_off=ro_d, lens=len_d, cap=cap_d)
            lcd.lookup_schedule_step(state, m, acc, bl, long_next, params)
            lcd.telemetry_update(tele, m, d, q_d, long_used, bl, acc, long_next, params)
        else:
            idx.decode_step(h_d, ro_d, len_d, cap_d, t(q), t(tgt), state, m, e, d, block, bl, acc,
                            long_next, True, telemetry=tele)
        acc_h = acc.cpu().numpy()
        for r in range(B):
            if acc_h[r] >= 0:
                emitted[r].extend(tgt[r, :acc_h[r] + 1].tolist())
        pos = pos + np.maximum(acc_h, 0) + 1
        if record:
            recs.append(dict(m=m.cpu().numpy(), e=e.cpu().numpy(), d=d.cpu().numpy(), q=q,
                             tgt=tgt, long=long_used.cpu().numpy(), block=block.cpu().numpy(),
                             blk=bl.cpu().numpy(), acc=acc_h, state=state.cpu().numpy(),
                             long_next=long_next.cpu().numpy()))
    torch.cuda.synchronize()
    return dict(recs=recs, emitted=emitted, lens=len_d.cpu().numpy(), flat=h_d.cpu().numpy(),
                row_off=row_off, tele=tele.cpu().numpy().view(np.uint32),
                indexed_len=idx.indexed_len.cpu().numpy())
