"""CPU oracle for context-lookup drafting (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liblcd_oracle.so`` (built from
``lcd_oracle.c`` by :func:`build`) with numpy arrays; it shares nothing with the
HIP library or its Python binding.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lcd_oracle.c")
_BENCH_SRC = os.path.join(_HERE, "lcd_oracle_bench.c")   # the CPU-baseline timing harness
_LIB = os.path.join(_HERE, "liblcd_oracle.so")

PAD = -1
DRAFT_STRIDE = 15
Q_STRIDE = 7
TARGET_STRIDE = 16


class OracleParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "l_min", "l_max", "k_max", "n_head", "n_block", "head_full", "head_agree",
        "agree_n", "tail_min", "entry_steps", "sticky", "near_full_slack")]


def default_params(**kw) -> OracleParams:
    """The article's settings: suffixes of 4..12 tokens, 15 drafted tokens, a
    7-slot draft-model head, head thresholds 8 (or 6 with 2 agreeing slots),
    tail threshold 4, two-step entry and a sticky exit of 3."""
    v = dict(l_min=4, l_max=12, k_max=15, n_head=7, n_block=15, head_full=8,
             head_agree=6, agree_n=2, tail_min=4, entry_steps=2, sticky=3,
             near_full_slack=1)
    v.update(kw)
    return OracleParams(**v)


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
           _SRC, _BENCH_SRC, "-o", _LIB + ".tmp"]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"oracle library missing: {_LIB} (run oracle.build())")
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        pp = ctypes.POINTER(OracleParams)
        L.oracle_lookup_propose.argtypes = [P, P, P, i32, pp, P, P, P]
        L.oracle_fuse_verify_block.argtypes = [P, P, P, P, i32, pp, P, P, P]
        L.oracle_greedy_accept.argtypes = [P, P, P, i32, P, P, P, P, P]
        L.oracle_lookup_schedule_step.argtypes = [P, P, P, P, i32, pp, P]
        L.oracle_telemetry_update.argtypes = [P, P, P, P, P, P, P, P, i32, pp]
        L.oracle_telemetry_reduce.argtypes = [P, P, i32, i32, P]
        L.oracle_rejection_accept.argtypes = [P, P, P, P, P, i32, P, P, i32, P, P, P, P, P, P]
        L.oracle_bench_steps.argtypes = [P, P, P, i32, P, P, pp, i32, ctypes.c_double, i32, P, P,
                                         P, P]
        L.oracle_bench_rejection.argtypes = [P, P, P, P, P, i32, P, P, i32, i32, ctypes.c_double,
                                             i32, P, P, P, P]
        for f in (L.oracle_lookup_propose, L.oracle_fuse_verify_block,
                  L.oracle_greedy_accept, L.oracle_lookup_schedule_step,
                  L.oracle_telemetry_update, L.oracle_telemetry_reduce,
                  L.oracle_rejection_accept, L.oracle_bench_steps, L.oracle_bench_rejection):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    a = np.ascontiguousarray(a, dtype=dt)
    return a


def lookup_propose(hist, row_off, lens, params=None):
    """Returns (match_len [B], match_end [B], draft [B,15]) for host arrays."""
    params = params or default_params()
    hist = _c(hist, np.int32)
    row_off = _c(row_off, np.int64)
    lens = _c(lens, np.int32)
    B = len(lens)
    m = np.zeros(B, np.int32)
    e = np.zeros(B, np.int32)
    d = np.zeros((B, DRAFT_STRIDE), np.int32)
    if B:
        lib().oracle_lookup_propose(_ptr(hist), _ptr(row_off), _ptr(lens), B,
                                    ctypes.byref(params), _ptr(m), _ptr(e), _ptr(d))
    return m, e, d


def lookup_one(h, params=None):
    """Lookup for a single history array."""
    h = _c(h, np.int32)
    buf = h if h.size else np.zeros(1, np.int32)
    m, e, d = lookup_propose(buf, np.zeros(1, np.int64), np.array([h.size], np.int32), params)
    return int(m[0]), int(e[0]), d[0]


def fuse_verify_block(draft, match_len, q, long_mode, params=None, with_mask=False):
    """Returns (block [B,15], block_len [B]) and, with ``with_mask``, the
    uint32 [B] mask of slots holding the draft model's own token."""
    params = params or default_params()
    draft = _c(draft, np.int32).reshape(-1, DRAFT_STRIDE)
    match_len = _c(match_len, np.int32)
    q = _c(q, np.int32).reshape(-1, Q_STRIDE)
    long_mode = _c(long_mode, np.int32)
    B = len(match_len)
    blk = np.zeros((B, DRAFT_STRIDE), np.int32)
    bl = np.zeros(B, np.int32)
    mask = np.zeros(B, np.uint32) if with_mask else None
    if B:
        lib().oracle_fuse_verify_block(_ptr(draft), _ptr(match_len), _ptr(q), _ptr(long_mode),
                                       B, ctypes.byref(params), _ptr(blk), _ptr(bl), _ptr(mask))
    return (blk, bl, mask) if with_mask else (blk, bl)


def greedy_accept(block, block_len, target, hist=None, row_off=None, lens=None, cap=None):
    """Returns accept [B]; when ``hist`` is given the accepted tokens are
    appended in place (``hist`` and ``lens`` are modified)."""
    block = _c(block, np.int32).reshape(-1, DRAFT_STRIDE)
    block_len = _c(block_len, np.int32)
    target = _c(target, np.int32).reshape(-1, TARGET_STRIDE)
    B = len(block_len)
    acc = np.zeros(B, np.int32)
    if hist is not None:
        for a in (hist, lens):
            assert a.dtype == np.int32 and a.flags.c_contiguous
        row_off = _c(row_off, np.int64)
        cap = _c(cap, np.int32)
    if B:
        lib().oracle_greedy_accept(_ptr(block), _ptr(block_len), _ptr(target), B, _ptr(acc),
                                   _ptr(hist), _ptr(row_off), _ptr(lens), _ptr(cap))
    return acc


def lookup_schedule_step(state, match_len, accept, block_len, params=None):
    """``state`` is an int32 [B,3] array {long_mode, streak, down}, updated in
    place.  Returns long_next [B]."""
    params = params or default_params()
    assert state.dtype == np.int32 and state.flags.c_contiguous
    match_len = _c(match_len, np.int32)
    accept = _c(accept, np.int32)
    block_len = _c(block_len, np.int32)
    B = len(match_len)
    ln = np.zeros(B, np.int32)
    if B:
        lib().oracle_lookup_schedule_step(_ptr(state), _ptr(match_len), _ptr(accept),
                                          _ptr(block_len), B, ctypes.byref(params), _ptr(ln))
    return ln


TELE_WORDS = 32
TELE_FIELDS = ("steps", "hits", "head_lookup", "tail_lookup", "long_steps", "entries", "exits",
               "emitted", "failed_append")


def telemetry_update(tele, match_len, draft, q, long_mode, block_len, accept, long_next,
                     params=None):
    """Adds one step to the per-request counters ``tele`` (uint32 [B,32], in place)."""
    params = params or default_params()
    assert tele.dtype == np.uint32 and tele.flags.c_contiguous
    match_len = _c(match_len, np.int32)
    B = len(match_len)
    if B:
        lib().oracle_telemetry_update(
            _ptr(tele), _ptr(match_len), _ptr(_c(draft, np.int32).reshape(-1, DRAFT_STRIDE)),
            _ptr(_c(q, np.int32).reshape(-1, Q_STRIDE)), _ptr(_c(long_mode, np.int32)),
            _ptr(_c(block_len, np.int32)), _ptr(_c(accept, np.int32)),
            _ptr(_c(long_next, np.int32)), B, ctypes.byref(params))
    return tele


def telemetry_reduce(tele, class_id, K):
    """Per-class totals: uint64 [K,32]."""
    tele = _c(tele, np.uint32).reshape(-1, TELE_WORDS)
    class_id = _c(class_id, np.int32)
    out = np.zeros((K, TELE_WORDS), np.uint64)
    lib().oracle_telemetry_reduce(_ptr(tele), _ptr(class_id), len(class_id), K, _ptr(out))
    return out


def rejection_accept(block, block_len, target_probs, u_accept, u_sample, model_mask=None,
                     model_probs=None, hist=None, row_off=None, lens=None, cap=None):
    """Sampled verification with point-mass lookup proposals.

    target_probs float32 [B,16,V]; model_probs float32 [B,7,V] or None;
    u_accept float64 [B,15]; u_sample uint64 [B]; model_mask uint32 [B] or None.
    Returns (accept [B], emitted [B,16]); when ``hist`` is given the emitted
    tokens are appended in place (``hist`` and ``lens`` are modified)."""
    block = _c(block, np.int32).reshape(-1, DRAFT_STRIDE)
    block_len = _c(block_len, np.int32)
    B = len(block_len)
    tp = _c(target_probs, np.float32).reshape(B, TARGET_STRIDE, -1)
    V = tp.shape[2]
    assert V < (1 << 23)
    mp = None if model_probs is None else _c(model_probs, np.float32).reshape(B, Q_STRIDE, V)
    mm = None if model_mask is None else _c(model_mask, np.uint32)
    ua = _c(u_accept, np.float64).reshape(B, DRAFT_STRIDE)
    us = _c(u_sample, np.uint64).reshape(B)
    acc = np.zeros(B, np.int32)
    em = np.full((B, TARGET_STRIDE), PAD, np.int32)
    if hist is not None:
        for a in (hist, lens):
            assert a.dtype == np.int32 and a.flags.c_contiguous
        row_off = _c(row_off, np.int64)
        cap = _c(cap, np.int32)
    if B:
        lib().oracle_rejection_accept(_ptr(block), _ptr(block_len), _ptr(mm), _ptr(tp), _ptr(mp),
                                      V, _ptr(ua), _ptr(us), B, _ptr(acc), _ptr(em), _ptr(hist),
                                      _ptr(row_off), _ptr(lens), _ptr(cap))
    return acc, em


def bench_steps(hist, row_off, lens, q, target, params=None, nthreads=1, min_seconds=1.0,
                max_steps=1 << 30):
    """Times whole decode steps of the batch (lookup, fusion, greedy accept,
    scheduler per request; no append) with the oracle's own functions on
    `nthreads` native threads (lcd_oracle_bench.c).  Returns (steps, wall
    seconds, process CPU seconds, checksum)."""
    params = params or default_params()
    hist = _c(hist, np.int32)
    row_off = _c(row_off, np.int64)
    lens = _c(lens, np.int32)
    q = _c(q, np.int32)
    target = _c(target, np.int32)
    steps = ctypes.c_int64()
    wall = ctypes.c_double()
    cpu = ctypes.c_double()
    chk = ctypes.c_int64()
    rc = lib().oracle_bench_steps(_ptr(hist), _ptr(row_off), _ptr(lens), len(lens), _ptr(q),
                                  _ptr(target), ctypes.byref(params), int(nthreads),
                                  float(min_seconds), int(max_steps), ctypes.byref(steps),
                                  ctypes.byref(wall), ctypes.byref(cpu), ctypes.byref(chk))
    if rc != 0:
        raise RuntimeError("oracle_bench_steps failed")
    return steps.value, wall.value, cpu.value, chk.value


def bench_rejection(block, block_len, target_probs, u_accept, u_sample, model_mask=None,
                    model_probs=None, nthreads=1, min_seconds=1.0, max_steps=1 << 30):
    """Times whole sampled-verification steps of the batch (the oracle's
    rejection_accept on every request, no append) on `nthreads` native threads
    (lcd_oracle_bench.c).  Returns (steps, wall seconds, process CPU seconds,
    checksum: the sum of every accepted count and emitted token per step)."""
    block = _c(block, np.int32).reshape(-1, DRAFT_STRIDE)
    block_len = _c(block_len, np.int32)
    B = len(block_len)
    tp = _c(target_probs, np.float32).reshape(B, TARGET_STRIDE, -1)
    V = tp.shape[2]
    mp = None if model_probs is None else _c(model_probs, np.float32).reshape(B, Q_STRIDE, V)
    mm = None if model_mask is None else _c(model_mask, np.uint32)
    ua = _c(u_accept, np.float64).reshape(B, DRAFT_STRIDE)
    us = _c(u_sample, np.uint64).reshape(B)
    steps = ctypes.c_int64()
    wall = ctypes.c_double()
    cpu = ctypes.c_double()
    chk = ctypes.c_int64()
    rc = lib().oracle_bench_rejection(_ptr(block), _ptr(block_len), _ptr(mm), _ptr(tp), _ptr(mp), V,
                                      _ptr(ua), _ptr(us), B, int(nthreads), float(min_seconds),
                                      int(max_steps), ctypes.byref(steps), ctypes.byref(wall),
                                      ctypes.byref(cpu), ctypes.byref(chk))
    if rc != 0:
        raise RuntimeError("oracle_bench_rejection failed")
    return steps.value, wall.value, cpu.value, chk.value
