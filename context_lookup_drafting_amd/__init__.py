"""Context-lookup drafting for speculative decoding on AMD Instinct MI355X.

A thin ctypes binding over ``liblcd.so`` (HIP kernels for gfx950, C ABI in
``include/lcd.h``).  The functions below only check and marshal arguments: every
step of the hot path runs in the library's kernels, asynchronously on the
current torch stream.  There is no CPU fallback; a missing or unloadable
library raises.

Entry points (same names as the C ABI):
  lookup_propose(hist, row_off, lens, max_len, workspace, match_len, match_end, draft, params)
  lookup_decode_step(hist, row_off, lens, cap, max_len, model_draft, target, state, workspace,
                     match_len, match_end, draft, block, block_len, accept, long_next, append, params,
                     lens_out=...)
  fuse_verify_block(draft, match_len, model_draft, long_mode, block, block_len, params,
                    model_mask=None)
  greedy_accept(block, block_len, target, accept, hist=None, row_off=None, lens=None, cap=None)
  rejection_accept(block, block_len, target_probs, u_accept, u_sample, workspace, accept, emitted,
                   model_mask=None, model_probs=None, hist=None, row_off=None, lens=None, cap=None)
  LookupIndex(cap, device, params).build(hist, row_off, lens, max_len)
  LookupIndex.propose(hist, row_off, lens, match_len, match_end, draft)
  LookupIndex.decode_step(hist, row_off, lens, cap, model_draft, target, state, match_len,
                          match_end, draft, block, block_len, accept, long_next, append, telemetry)
                                          (lookup_index_plan / _build / _propose)
  lookup_schedule_step(state, match_len, accept, block_len, long_next, params)
"""

from __future__ import annotations

import ctypes
import os

PAD = -1
DRAFT_STRIDE = 15
Q_STRIDE = 7
TARGET_STRIDE = 16
MAX_SUFFIX = 16

LCD_OK = 0
LCD_EINVAL = -1
LCD_EHIP = -2

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblcd.so")


class LCDError(RuntimeError):
    def __init__(self, fn: str, code: int):
        what = {LCD_EINVAL: "invalid argument", LCD_EHIP: "HIP launch error"}.get(code, "error")
        super().__init__(f"{fn} returned {code} ({what})")
        self.code = code


class Params(ctypes.Structure):
    """Mirror of ``lcd_params`` (include/lcd.h)."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "l_min", "l_max", "k_max", "n_head", "n_block", "head_full", "head_agree",
        "agree_n", "tail_min", "entry_steps", "sticky", "near_full_slack", "scan_wgs",
        "scan_balance", "merge_polls", "index_load")]

    def __repr__(self):
        return "Params(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_lib = None


def load():
    """Load liblcd.so once; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} "
                               "(run python -m context_lookup_drafting_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        pp = ctypes.POINTER(Params)
        L.lcd_default_params.argtypes = [pp]
        L.lcd_default_params.restype = None
        L.lcd_check_params.argtypes = [pp]
        L.lcd_check_params.restype = ctypes.c_int
        L.lcd_workspace_bytes.argtypes = [i32]
        L.lcd_workspace_bytes.restype = ctypes.c_size_t
        L.lookup_propose.argtypes = [P, P, P, i32, i32, pp, P, P, P, P, P]
        L.lookup_propose_timed.argtypes = [P, P, P, i32, i32, pp, P, P, P, P, P, P, P]
        L.fuse_verify_block.argtypes = [P, P, P, P, i32, pp, P, P, P, P]
        L.lcd_decode_step_workspace_bytes.argtypes = [i32, i32, pp]
        L.lcd_decode_step_workspace_bytes.restype = ctypes.c_size_t
        dec = [P, P, P, P, P, i32, i32, P, P, P, pp, P, ctypes.c_size_t, P, P, P, P, P, P, P, P, i32,
               P]
        L.lookup_decode_step.argtypes = dec
        L.lookup_decode_step_timed.argtypes = dec + [P, P]
        L.lookup_decode_step_noalloc.argtypes = dec[:11] + dec[13:]
        L.greedy_accept.argtypes = [P, P, P, i32, P, P, P, P, P, P]
        L.lookup_schedule_step.argtypes = [P, P, P, P, i32, pp, P, P]
        L.lookup_telemetry_update.argtypes = [P, P, P, P, P, P, P, P, i32, pp, P]
        L.lookup_telemetry_reduce.argtypes = [P, P, i32, i32, P, P]
        L.rejection_accept_workspace_bytes.argtypes = [i32, i32]
        L.rejection_accept_workspace_bytes.restype = ctypes.c_size_t
        L.lookup_launch_shape.argtypes = [i32, i32, pp, P, P, P]
        L.lookup_launch_shape.restype = ctypes.c_int
        L.lookup_scan_occupancy.argtypes = [i32, P]
        L.lcd_read_probe.argtypes = [P, ctypes.c_int64, i32, i32, P, P, P, P]
        L.lcd_read_probe.restype = ctypes.c_int
        L.lcd_empty_probe.argtypes = [i32, P, P, P]
        L.lcd_empty_probe.restype = ctypes.c_int
        L.lookup_index_plan.argtypes = [P, i32, pp, P, P]
        L.lookup_index_plan.restype = ctypes.c_int64
        L.lookup_index_build.argtypes = [P, P, P, i32, pp, i32, P, P, P, ctypes.c_size_t, P, P, i32, P]
        L.lookup_index_propose.argtypes = [P, P, P, i32, pp, i32, P, P, P, P, P, P, P, P]
        L.lookup_index_propose_timed.argtypes = [P, P, P, i32, pp, i32, P, P, P, P, P, P, P, P, P, P]
        idec = [P, P, P, P, i32, pp, i32, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, i32, P]
        L.lookup_index_decode_step.argtypes = idec
        L.lookup_index_decode_step_timed.argtypes = idec + [P, P]
        rej = [P, P, P, P, P, i32, P, P, i32, i32, i32, P, ctypes.c_size_t, P, P, P, P, P, P, P]
        L.rejection_accept.argtypes = rej
        L.rejection_accept_timed.argtypes = rej + [P, P]
        for f in (L.lookup_propose, L.lookup_propose_timed, L.fuse_verify_block,
                  L.greedy_accept, L.lookup_schedule_step, L.lookup_decode_step,
                  L.lookup_decode_step_timed, L.lookup_decode_step_noalloc,
                  L.lookup_telemetry_update,
                  L.lookup_telemetry_reduce, L.rejection_accept, L.rejection_accept_timed,
                  L.lookup_index_build, L.lookup_index_propose, L.lookup_index_propose_timed,
                  L.lookup_index_decode_step, L.lookup_index_decode_step_timed):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def default_params(**overrides) -> Params:
    p = Params()
    load().lcd_default_params(ctypes.byref(p))
    for k, v in overrides.items():
        if not hasattr(p, k):
            raise KeyError(k)
        setattr(p, k, int(v))
    return p


def check_params(p: Params) -> bool:
    return load().lcd_check_params(ctypes.byref(p)) == LCD_OK


def workspace_bytes(B: int) -> int:
    return int(load().lcd_workspace_bytes(int(B)))


def alloc_workspace(B: int, device):
    """Zero-filled lookup workspace for B requests (then kept valid by every
    call: counts and gathered slots back at zero, a per-request call epoch)."""
    import torch
    n = max(workspace_bytes(B), 16)
    return torch.zeros(n // 8, dtype=torch.int64, device=device)


# ---------------------------------------------------------------------------
# argument marshalling
# ---------------------------------------------------------------------------

def _dev(t, name, dtype, numel=None, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn, rc):
    if rc != LCD_OK:
        raise LCDError(fn, rc)


def _propose_args(hist, row_off, lens, max_len, workspace, match_len, match_end, draft, p):
    import torch
    B = lens.numel()
    dev = lens.device
    if workspace.numel() * workspace.element_size() < workspace_bytes(B):
        raise ValueError("workspace too small")
    return (
        _dev(hist, "hist", torch.int32, device=dev),
        _dev(row_off, "row_off", torch.int64, B, dev),
        _dev(lens, "lens", torch.int32, B, dev),
        ctypes.c_int32(B), ctypes.c_int32(int(max_len)), ctypes.byref(p),
        _dev(workspace, "workspace", workspace.dtype, device=dev),
        _dev(match_len, "match_len", torch.int32, B, dev),
        _dev(match_end, "match_end", torch.int32, B, dev),
        _dev(draft, "draft", torch.int32, B * DRAFT_STRIDE, dev),
        _stream(dev),
    )


def lookup_propose(hist, row_off, lens, max_len, workspace, match_len, match_end, draft,
                   params: Params | None = None):
    """Longest-suffix / latest-occurrence lookup and 15-token draft for every
    request (include/lcd.h, lookup_propose)."""
    p = params or default_params()
    args = _propose_args(hist, row_off, lens, max_len, workspace, match_len, match_end, draft, p)
    _check("lookup_propose", load().lookup_propose(*args))


def lookup_propose_timed(hist, row_off, lens, max_len, workspace, match_len, match_end, draft,
                         ev_start, ev_stop, params: Params | None = None):
    """lookup_propose with GPU-stamped start/stop events (raw hipEvent_t handles
    as ints, either may be 0) around its scan kernel, for profiling."""
    p = params or default_params()
    args = _propose_args(hist, row_off, lens, max_len, workspace, match_len, match_end, draft, p)
    _check("lookup_propose_timed", load().lookup_propose_timed(
        *args, ctypes.c_void_p(ev_start or None), ctypes.c_void_p(ev_stop or None)))


def fuse_verify_block(draft, match_len, model_draft, long_mode, block, block_len,
                      params: Params | None = None, model_mask=None):
    """Verify block of every request; ``model_mask`` (int32 [B], optional)
    gets bit i set for each slot keeping the draft model's token."""
    import torch
    p = params or default_params()
    B = match_len.numel()
    dev = match_len.device
    _check("fuse_verify_block", load().fuse_verify_block(
        _dev(draft, "draft", torch.int32, B * DRAFT_STRIDE, dev),
        _dev(match_len, "match_len", torch.int32, B, dev),
        _dev(model_draft, "model_draft", torch.int32, B * Q_STRIDE, dev),
        _dev(long_mode, "long_mode", torch.int32, B, dev),
        ctypes.c_int32(B), ctypes.byref(p),
        _dev(block, "block", torch.int32, B * DRAFT_STRIDE, dev),
        _dev(block_len, "block_len", torch.int32, B, dev),
        ctypes.c_void_p(None) if model_mask is None
        else _dev(model_mask, "model_mask", torch.int32, B, dev),
        _stream(dev)))


def greedy_accept(block, block_len, target, accept, hist=None, row_off=None, lens=None, cap=None):
    import torch
    B = block_len.numel()
    dev = block_len.device
    if hist is None:
        h = ro = ln = cp = ctypes.c_void_p(None)
    else:
        h = _dev(hist, "hist", torch.int32, device=dev)
        ro = _dev(row_off, "row_off", torch.int64, B, dev)
        ln = _dev(lens, "lens", torch.int32, B, dev)
        cp = _dev(cap, "cap", torch.int32, B, dev)
    _check("greedy_accept", load().greedy_accept(
        _dev(block, "block", torch.int32, B * DRAFT_STRIDE, dev),
        _dev(block_len, "block_len", torch.int32, B, dev),
        _dev(target, "target", torch.int32, B * TARGET_STRIDE, dev),
        ctypes.c_int32(B),
        _dev(accept, "accept", torch.int32, B, dev),
        h, ro, ln, cp, _stream(dev)))


def lookup_schedule_step(state, match_len, accept, block_len, long_next,
                         params: Params | None = None):
    """``state`` is an int32 [B,3] device tensor {long_mode, streak, down}."""
    import torch
    p = params or default_params()
    B = match_len.numel()
    dev = match_len.device
    _check("lookup_schedule_step", load().lookup_schedule_step(
        _dev(state, "state", torch.int32, 3 * B, dev),
        _dev(match_len, "match_len", torch.int32, B, dev),
        _dev(accept, "accept", torch.int32, B, dev),
        _dev(block_len, "block_len", torch.int32, B, dev),
        ctypes.c_int32(B), ctypes.byref(p),
        _dev(long_next, "long_next", torch.int32, B, dev),
        _stream(dev)))


def decode_step_workspace_bytes(B: int, max_len: int, params: Params | None = None) -> int:
    p = params or default_params()
    return int(load().lcd_decode_step_workspace_bytes(int(B), int(max_len), ctypes.byref(p)))


def alloc_decode_workspace(B: int, max_len: int, device, params: Params | None = None):
    """Zero-filled workspace for lookup_decode_step (then kept valid by every
    call, as lookup_propose's)."""
    import torch
    n = max(decode_step_workspace_bytes(B, max_len, params), 16)
    return torch.zeros((n + 7) // 8, dtype=torch.int64, device=device)


def _decode_args(hist, row_off, lens, cap, max_len, model_draft, target, state, workspace,
                 match_len, match_end, draft, block, block_len, accept, long_next, append, p,
                 telemetry=None, lens_out=None):
    import torch
    B = lens.numel()
    dev = lens.device
    nul = ctypes.c_void_p(None)
    if append and lens_out is None:
        raise ValueError("lookup_decode_step: append needs lens_out, a second length array "
                         "(the launch reads lens and writes the new lengths to lens_out)")
    return (
        _dev(hist, "hist", torch.int32, device=dev),
        _dev(row_off, "row_off", torch.int64, B, dev),
        _dev(lens, "lens", torch.int32, B, dev),
        _dev(lens_out, "lens_out", torch.int32, B, dev) if lens_out is not None else nul,
        _dev(cap, "cap", torch.int32, B, dev) if cap is not None else nul,
        ctypes.c_int32(B), ctypes.c_int32(int(max_len)),
        _dev(model_draft, "model_draft", torch.int32, B * Q_STRIDE, dev),
        _dev(target, "target", torch.int32, B * TARGET_STRIDE, dev),
        _dev(state, "state", torch.int32, 3 * B, dev),
        ctypes.byref(p),
        _dev(workspace, "workspace", workspace.dtype, device=dev),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        _dev(match_len, "match_len", torch.int32, B, dev),
        _dev(match_end, "match_end", torch.int32, B, dev),
        _dev(draft, "draft", torch.int32, B * DRAFT_STRIDE, dev),
        _dev(block, "block", torch.int32, B * DRAFT_STRIDE, dev),
        _dev(block_len, "block_len", torch.int32, B, dev),
        _dev(accept, "accept", torch.int32, B, dev),
        _dev(long_next, "long_next", torch.int32, B, dev) if long_next is not None else nul,
        (_dev(telemetry, "telemetry", torch.int32, B * TELE_WORDS, dev)
         if telemetry is not None else nul),
        ctypes.c_int32(1 if append else 0),
        _stream(dev),
    )


def lookup_decode_step(hist, row_off, lens, cap, max_len, model_draft, target, state, workspace,
                       match_len, match_end, draft, block, block_len, accept, long_next=None,
                       append=True, params: Params | None = None, telemetry=None, lens_out=None):
    """One whole decode step (lookup, fusion under state's current mode, greedy
    accept with optional append, scheduler update, optional telemetry) in one
    kernel.  ``lens`` is only read; with ``append`` the lengths after the step
    go to ``lens_out`` (int32 [B], not overlapping ``lens``; a decode loop
    alternates the two).  ``telemetry``: int32 [B,32] counter rows (from
    alloc_telemetry)."""
    p = params or default_params()
    _check("lookup_decode_step", load().lookup_decode_step(*_decode_args(
        hist, row_off, lens, cap, max_len, model_draft, target, state, workspace, match_len,
        match_end, draft, block, block_len, accept, long_next, append, p, telemetry, lens_out)))


def lookup_decode_step_timed(hist, row_off, lens, cap, max_len, model_draft, target, state,
                             workspace, match_len, match_end, draft, block, block_len, accept,
                             ev_start, ev_stop, long_next=None, append=True,
                             params: Params | None = None, telemetry=None, lens_out=None):
    """lookup_decode_step with GPU-stamped events around its scan kernel."""
    p = params or default_params()
    _check("lookup_decode_step_timed", load().lookup_decode_step_timed(*_decode_args(
        hist, row_off, lens, cap, max_len, model_draft, target, state, workspace, match_len,
        match_end, draft, block, block_len, accept, long_next, append, p, telemetry, lens_out),
        ctypes.c_void_p(ev_start or None), ctypes.c_void_p(ev_stop or None)))


NOALLOC_MAX_B = 1024


def lookup_decode_step_noalloc(hist, row_off, lens, cap, max_len, model_draft, target, state,
                               match_len, match_end, draft, block, block_len, accept,
                               long_next=None, append=True, params: Params | None = None,
                               telemetry=None, lens_out=None):
    """lookup_decode_step without a workspace argument: the library's static
    per-GPU array serves as the workspace (at most NOALLOC_MAX_B requests;
    calls that overlap on one GPU race)."""
    import torch
    p = params or default_params()
    dummy = torch.empty(0, dtype=torch.int64, device=lens.device)
    a = _decode_args(hist, row_off, lens, cap, max_len, model_draft, target, state, dummy,
                     match_len, match_end, draft, block, block_len, accept, long_next, append, p,
                     telemetry, lens_out)
    _check("lookup_decode_step_noalloc", load().lookup_decode_step_noalloc(*(a[:11] + a[13:])))


TELE_WORDS = 32
TELE_FIELDS = ("steps", "hits", "head_lookup", "tail_lookup", "long_steps", "entries", "exits",
               "emitted", "failed_append")
TELE_HIST = 9


def alloc_telemetry(B: int, device):
    """Zeroed telemetry rows: int32 [B,32] (the library treats them as uint32)."""
    import torch
    return torch.zeros((B, TELE_WORDS), dtype=torch.int32, device=device)


def telemetry_update(telemetry, match_len, draft, model_draft, long_mode, block_len, accept,
                     long_next, params: Params | None = None):
    """Adds one step (the separate calls' outputs) to the telemetry rows."""
    import torch
    p = params or default_params()
    B = match_len.numel()
    dev = match_len.device
    _check("lookup_telemetry_update", load().lookup_telemetry_update(
        _dev(telemetry, "telemetry", torch.int32, B * TELE_WORDS, dev),
        _dev(match_len, "match_len", torch.int32, B, dev),
        _dev(draft, "draft", torch.int32, B * DRAFT_STRIDE, dev),
        _dev(model_draft, "model_draft", torch.int32, B * Q_STRIDE, dev),
        _dev(long_mode, "long_mode", torch.int32, B, dev),
        _dev(block_len, "block_len", torch.int32, B, dev),
        _dev(accept, "accept", torch.int32, B, dev),
        _dev(long_next, "long_next", torch.int32, B, dev),
        ctypes.c_int32(B), ctypes.byref(p), _stream(dev)))


def telemetry_reduce(telemetry, class_id, K: int):
    """Per-class totals of the telemetry rows: int64 [K,32] (uint64 values)."""
    import torch
    B = class_id.numel()
    dev = class_id.device
    out = torch.empty((K, TELE_WORDS), dtype=torch.int64, device=dev)
    _check("lookup_telemetry_reduce", load().lookup_telemetry_reduce(
        _dev(telemetry, "telemetry", torch.int32, B * TELE_WORDS, dev),
        _dev(class_id, "class_id", torch.int32, B, dev), ctypes.c_int32(B), ctypes.c_int32(K),
        _dev(out, "out", torch.int64, K * TELE_WORDS, dev), _stream(dev)))
    return out


SAMPLE_MAX_VOCAB = 1 << 22


def rejection_accept_workspace_bytes(B: int, V: int) -> int:
    return int(load().rejection_accept_workspace_bytes(int(B), int(V)))


def alloc_rejection_workspace(B: int, V: int, device):
    """Zero-filled rejection_accept workspace (then kept valid by every call)."""
    import torch
    n = max(rejection_accept_workspace_bytes(B, V), 16)
    return torch.zeros((n + 7) // 8, dtype=torch.int64, device=device)


def _rejection_args(block, block_len, target_probs, u_accept, u_sample, workspace, accept,
                    emitted, model_mask, model_probs, hist, row_off, lens, cap, wg_units,
                    merge_polls=0):
    import torch
    B = block_len.numel()
    dev = block_len.device
    if target_probs.dim() != 3 or target_probs.shape[0] != B or target_probs.shape[1] != TARGET_STRIDE:
        raise ValueError("target_probs must be [B, 16, V]")
    V = target_probs.shape[2]
    if model_probs is not None and tuple(model_probs.shape) != (B, Q_STRIDE, V):
        raise ValueError("model_probs must be [B, 7, V]")
    if workspace.numel() * workspace.element_size() < rejection_accept_workspace_bytes(B, V):
        raise ValueError("workspace too small")
    none = ctypes.c_void_p(None)
    if hist is None:
        h = ro = ln = cp = none
    else:
        h = _dev(hist, "hist", torch.int32, device=dev)
        ro = _dev(row_off, "row_off", torch.int64, B, dev)
        ln = _dev(lens, "lens", torch.int32, B, dev)
        cp = _dev(cap, "cap", torch.int32, B, dev)
    return (
        _dev(block, "block", torch.int32, B * DRAFT_STRIDE, dev),
        _dev(block_len, "block_len", torch.int32, B, dev),
        none if model_mask is None else _dev(model_mask, "model_mask", torch.int32, B, dev),
        _dev(target_probs, "target_probs", torch.float32, B * TARGET_STRIDE * V, dev),
        none if model_probs is None
        else _dev(model_probs, "model_probs", torch.float32, B * Q_STRIDE * V, dev),
        ctypes.c_int32(V),
        _dev(u_accept, "u_accept", torch.float64, B * DRAFT_STRIDE, dev),
        _dev(u_sample, "u_sample", torch.int64, B, dev),
        ctypes.c_int32(B), ctypes.c_int32(int(wg_units)), ctypes.c_int32(int(merge_polls)),
        _dev(workspace, "workspace", workspace.dtype, device=dev),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        _dev(accept, "accept", torch.int32, B, dev),
        _dev(emitted, "emitted", torch.int32, B * TARGET_STRIDE, dev),
        h, ro, ln, cp, _stream(dev),
    )


def rejection_accept(block, block_len, target_probs, u_accept, u_sample, workspace, accept,
                     emitted, model_mask=None, model_probs=None, hist=None, row_off=None,
                     lens=None, cap=None, wg_units: int = 0, merge_polls: int = 0):
    """Sampled verification with point-mass lookup proposals (include/lcd.h,
    rejection_accept).  target_probs float32 [B,16,V], model_probs float32
    [B,7,V] or None, u_accept float64 [B,15], u_sample int64 [B] (the bits of
    uniform 64-bit words), model_mask int32 [B] or None; writes accept int32
    [B] and emitted int32 [B,16]; appends when ``hist`` is given.
    ``merge_polls`` is a diagnostic bound of the gathering's wait."""
    args = _rejection_args(block, block_len, target_probs, u_accept, u_sample, workspace, accept,
                           emitted, model_mask, model_probs, hist, row_off, lens, cap, wg_units,
                           merge_polls)
    _check("rejection_accept", load().rejection_accept(*args))


def rejection_accept_timed(block, block_len, target_probs, u_accept, u_sample, workspace, accept,
                           emitted, ev_start, ev_stop, model_mask=None, model_probs=None,
                           wg_units: int = 0):
    """rejection_accept with GPU-stamped start/stop events, for profiling."""
    args = _rejection_args(block, block_len, target_probs, u_accept, u_sample, workspace, accept,
                           emitted, model_mask, model_probs, None, None, None, None, wg_units)
    _check("rejection_accept_timed", load().rejection_accept_timed(
        *args, ctypes.c_void_p(ev_start or None), ctypes.c_void_p(ev_stop or None)))


class LookupIndex:
    """Device n-gram index of a batch (include/lcd.h, lookup_index_*): the
    lookup of lookup_propose without scanning the histories.  ``cap`` are the
    rows' capacities (the longest each history may grow to)."""

    def __init__(self, cap, device, params: Params | None = None, fp_bits: int = 0):
        import numpy as np
        import torch
        self.p = params or default_params()
        self.fp_bits = int(fp_bits)
        cap = np.ascontiguousarray(cap, dtype=np.int32)
        self.B = len(cap)
        off = np.zeros(max(self.B, 1), np.int64)
        slots = np.zeros(max(self.B, 1), np.int32)
        nbytes = int(load().lookup_index_plan(cap.ctypes.data_as(ctypes.c_void_p), self.B,
                                                ctypes.byref(self.p),
                                                off.ctypes.data_as(ctypes.c_void_p),
                                                slots.ctypes.data_as(ctypes.c_void_p)))
        if nbytes < 0:
            raise LCDError("lookup_index_plan", nbytes)
        self.device = torch.device(device)
        self.table_bytes = max(nbytes, 8)
        # zeroed: empty tables and no cached tokens until build() indexes the rows
        self.tables = torch.zeros(self.table_bytes // 8, dtype=torch.int64, device=self.device)
        self.table_off = torch.from_numpy(off[:self.B].copy()).to(self.device)
        self.table_slots = torch.from_numpy(slots[:self.B].copy()).to(self.device)
        self.indexed_len = torch.zeros(self.B, dtype=torch.int32, device=self.device)
        self._scratch = torch.zeros(max(self.B, 1), dtype=torch.int32, device=self.device)

    def build(self, hist, row_off, lens, max_len: int):
        import torch
        B, dev = self.B, self.device
        _check("lookup_index_build", load().lookup_index_build(
            _dev(hist, "hist", torch.int32, device=dev),
            _dev(row_off, "row_off", torch.int64, B, dev),
            _dev(lens, "lens", torch.int32, B, dev), ctypes.c_int32(B), ctypes.byref(self.p),
            ctypes.c_int32(self.fp_bits), _dev(self.table_off, "table_off", torch.int64, B, dev),
            _dev(self.table_slots, "table_slots", torch.int32, B, dev),
            ctypes.c_void_p(self.tables.data_ptr()), ctypes.c_size_t(self.table_bytes),
            _dev(self.indexed_len, "indexed_len", torch.int32, B, dev),
            ctypes.c_void_p(self._scratch.data_ptr()), ctypes.c_int32(int(max_len)), _stream(dev)))

    def propose(self, hist, row_off, lens, match_len, match_end, draft, events=None):
        """``events``: optional (start, stop) raw hipEvent_t handles stamped by
        the GPU around the kernel (profiling)."""
        import torch
        B, dev = self.B, self.device
        L = load()
        fn = L.lookup_index_propose if events is None else L.lookup_index_propose_timed
        extra = () if events is None else (ctypes.c_void_p(events[0] or None),
                                           ctypes.c_void_p(events[1] or None))
        _check("lookup_index_propose", fn(
            _dev(hist, "hist", torch.int32, device=dev),
            _dev(row_off, "row_off", torch.int64, B, dev),
            _dev(lens, "lens", torch.int32, B, dev), ctypes.c_int32(B), ctypes.byref(self.p),
            ctypes.c_int32(self.fp_bits), _dev(self.table_off, "table_off", torch.int64, B, dev),
            _dev(self.table_slots, "table_slots", torch.int32, B, dev),
            ctypes.c_void_p(self.tables.data_ptr()),
            _dev(self.indexed_len, "indexed_len", torch.int32, B, dev),
            _dev(match_len, "match_len", torch.int32, B, dev),
            _dev(match_end, "match_end", torch.int32, B, dev),
            _dev(draft, "draft", torch.int32, B * DRAFT_STRIDE, dev), _stream(dev), *extra))

    def decode_step(self, hist, row_off, lens, cap, model_draft, target, state, match_len,
                    match_end, draft, block, block_len, accept, long_next=None, append=True,
                    telemetry=None, events=None):
        """One whole decode step through the index in one kernel
        (lookup_index_decode_step): the outputs of decode_step's four calls.
        ``events`` as for propose."""
        import torch
        B, dev = self.B, self.device
        L = load()
        fn = L.lookup_index_decode_step if events is None else L.lookup_index_decode_step_timed
        extra = () if events is None else (ctypes.c_void_p(events[0] or None),
                                           ctypes.c_void_p(events[1] or None))
        nul = ctypes.c_void_p(None)
        _check("lookup_index_decode_step", fn(
            _dev(hist, "hist", torch.int32, device=dev),
            _dev(row_off, "row_off", torch.int64, B, dev),
            _dev(lens, "lens", torch.int32, B, dev),
            _dev(cap, "cap", torch.int32, B, dev) if cap is not None else nul,
            ctypes.c_int32(B), ctypes.byref(self.p), ctypes.c_int32(self.fp_bits),
            _dev(self.table_off, "table_off", torch.int64, B, dev),
            _dev(self.table_slots, "table_slots", torch.int32, B, dev),
            ctypes.c_void_p(self.tables.data_ptr()),
            _dev(self.indexed_len, "indexed_len", torch.int32, B, dev),
            _dev(model_draft, "model_draft", torch.int32, B * Q_STRIDE, dev),
            _dev(target, "target", torch.int32, B * TARGET_STRIDE, dev),
            _dev(state, "state", torch.int32, 3 * B, dev),
            _dev(match_len, "match_len", torch.int32, B, dev),
            _dev(match_end, "match_end", torch.int32, B, dev),
            _dev(draft, "draft", torch.int32, B * DRAFT_STRIDE, dev),
            _dev(block, "block", torch.int32, B * DRAFT_STRIDE, dev),
            _dev(block_len, "block_len", torch.int32, B, dev),
            _dev(accept, "accept", torch.int32, B, dev),
            _dev(long_next, "long_next", torch.int32, B, dev) if long_next is not None else nul,
            (_dev(telemetry, "telemetry", torch.int32, B * TELE_WORDS, dev)
             if telemetry is not None else nul),
            ctypes.c_int32(1 if append else 0), _stream(dev), *extra))


def launch_shape(B: int, max_len: int, params: Params | None = None, lens=None):
    """(workgroups per launch, chunk length) of the scan; ``lens`` (host array)
    is needed with scan_balance = 1."""
    import numpy as np
    p = params or default_params()
    wgs, chunk = ctypes.c_int32(), ctypes.c_int32()
    lh = None if lens is None else np.ascontiguousarray(lens, dtype=np.int32)
    _check("lookup_launch_shape", load().lookup_launch_shape(
        ctypes.c_int32(B), ctypes.c_int32(max_len), ctypes.byref(p),
        None if lh is None else lh.ctypes.data_as(ctypes.c_void_p), ctypes.byref(wgs),
        ctypes.byref(chunk)))
    return wgs.value, chunk.value


def scan_occupancy(waves: int) -> int:
    """Workgroups of the `waves`-wave scan kernel (4 or 16) one CU holds at once."""
    n = ctypes.c_int32()
    _check("lookup_scan_occupancy", load().lookup_scan_occupancy(ctypes.c_int32(waves), ctypes.byref(n)))
    return n.value


PROBE_VARIANTS = {"contig4": 0, "contig8": 1, "interleave4": 2, "interleave8": 3,
                  "interleave16": 4}
PROBE_NT = 8                       # or-ed in: non-temporal loads ("...-nt" names)
PROBE_VARIANTS.update({k + "-nt": v | PROBE_NT for k, v in list(PROBE_VARIANTS.items())})


def read_probe(buf, nbytes: int, blocks: int, out, ev_start=None, ev_stop=None,
               variant: str = "contig4"):
    """Plain streaming read of the first `nbytes` of a device tensor
    (measurement); ``out`` is int32 [blocks]."""
    import torch
    dev = buf.device
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("read beyond the buffer")
    _check("lcd_read_probe", load().lcd_read_probe(
        ctypes.c_void_p(buf.data_ptr()), ctypes.c_int64(int(nbytes)), ctypes.c_int32(int(blocks)),
        ctypes.c_int32(PROBE_VARIANTS[variant]), _dev(out, "out", torch.int32, int(blocks), dev),
        _stream(dev), ctypes.c_void_p(ev_start or None), ctypes.c_void_p(ev_stop or None)))


def empty_probe(blocks: int, device, ev_start=None, ev_stop=None):
    """A kernel of `blocks` workgroups that does nothing (launch floor)."""
    _check("lcd_empty_probe", load().lcd_empty_probe(
        ctypes.c_int32(int(blocks)), _stream(device), ctypes.c_void_p(ev_start or None),
        ctypes.c_void_p(ev_stop or None)))


from .drafter import LookupDrafter  # noqa: E402  (the stateful wrapper over the calls above)
