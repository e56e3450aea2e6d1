"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/lcd.h declares, and rejects misuse before launching."""

import ctypes
import os
import re

import numpy as np
import pytest

import context_lookup_drafting_amd as lcd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "lcd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|void|size_t|int64_t)\s+\**\s*(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"lookup_propose", "fuse_verify_block", "greedy_accept",
            "lookup_schedule_step"} <= set(names)
    L = lcd.load()
    for n in names:
        assert hasattr(L, n), n


def test_default_params_are_the_articles_values():
    p = lcd.default_params()
    assert (p.l_min, p.l_max, p.k_max) == (4, 12, 15)
    assert (p.n_head, p.n_block) == (7, 15)
    assert (p.head_full, p.head_agree, p.agree_n, p.tail_min) == (8, 6, 2, 4)
    assert (p.entry_steps, p.sticky, p.near_full_slack, p.scan_wgs) == (2, 3, 1, 0)
    assert p.scan_balance == 0 and p.merge_polls == 0 and p.index_load == 3
    assert lcd.check_params(p)


@pytest.mark.parametrize("bad", [
    dict(l_min=0), dict(l_min=5, l_max=4), dict(l_max=17), dict(k_max=-1), dict(k_max=16),
    dict(n_head=0), dict(n_head=8, n_block=15), dict(n_block=6), dict(n_block=16),
    dict(head_full=0), dict(head_agree=0), dict(agree_n=-1), dict(agree_n=8),
    dict(tail_min=0), dict(entry_steps=0), dict(sticky=-1), dict(near_full_slack=-1),
    dict(scan_wgs=-1), dict(scan_balance=2), dict(scan_balance=-1), dict(merge_polls=-2),
    dict(index_load=1), dict(index_load=17),
])
def test_param_ranges_rejected(bad):
    assert not lcd.check_params(lcd.default_params(**bad))


def test_workspace_bytes():
    assert lcd.workspace_bytes(0) == 0
    assert lcd.workspace_bytes(64) == 64 * 8208      # LCD_WORKSPACE_PER_REQUEST


def _P(v):
    return ctypes.c_void_p(v)


def test_entry_points_reject_misuse_without_launching():
    L = lcd.load()
    p = lcd.default_params()
    pp = ctypes.byref(p)
    s = _P(None)
    fake = 0x10000          # never dereferenced: validation fails first
    # B < 0
    assert L.lookup_propose(_P(fake), _P(fake), _P(fake), -1, 10, pp, _P(fake),
                            _P(fake), _P(fake), _P(fake), s) == lcd.LCD_EINVAL
    # NULL arrays with B > 0
    assert L.lookup_propose(None, _P(fake), _P(fake), 4, 10, pp, _P(fake),
                            _P(fake), _P(fake), _P(fake), s) == lcd.LCD_EINVAL
    assert L.lookup_propose(_P(fake), _P(fake), _P(fake), 4, 10, pp, None,
                            _P(fake), _P(fake), _P(fake), s) == lcd.LCD_EINVAL
    # misaligned history / workspace
    assert L.lookup_propose(_P(fake + 4), _P(fake), _P(fake), 4, 10, pp, _P(fake),
                            _P(fake), _P(fake), _P(fake), s) == lcd.LCD_EINVAL
    assert L.lookup_propose(_P(fake), _P(fake), _P(fake), 4, 10, pp, _P(fake + 8),
                            _P(fake), _P(fake), _P(fake), s) == lcd.LCD_EINVAL
    # negative max_len, bad params
    assert L.lookup_propose(_P(fake), _P(fake), _P(fake), 4, -1, pp, _P(fake),
                            _P(fake), _P(fake), _P(fake), s) == lcd.LCD_EINVAL
    bad = lcd.default_params(l_max=20)
    assert L.lookup_propose(_P(fake), _P(fake), _P(fake), 4, 10, ctypes.byref(bad), _P(fake),
                            _P(fake), _P(fake), _P(fake), s) == lcd.LCD_EINVAL
    assert L.lookup_propose(_P(fake), _P(fake), _P(fake), 4, 10, None, _P(fake),
                            _P(fake), _P(fake), _P(fake), s) == lcd.LCD_EINVAL
    assert L.fuse_verify_block(None, _P(fake), _P(fake), _P(fake), 3, pp, _P(fake), _P(fake),
                               None, s) == lcd.LCD_EINVAL
    assert L.greedy_accept(_P(fake), _P(fake), _P(fake), 3, None, None, None, None, None,
                           s) == lcd.LCD_EINVAL
    # appending needs row offsets, lengths and capacities
    assert L.greedy_accept(_P(fake), _P(fake), _P(fake), 3, _P(fake), _P(fake), None, _P(fake),
                           _P(fake), s) == lcd.LCD_EINVAL
    assert L.lookup_schedule_step(_P(fake), _P(fake), _P(fake), None, 3, pp, _P(fake),
                                  s) == lcd.LCD_EINVAL


def test_empty_batch_is_a_noop():
    L = lcd.load()
    p = lcd.default_params()
    pp = ctypes.byref(p)
    assert L.lookup_propose(None, None, None, 0, 0, pp, None, None, None, None, None) == lcd.LCD_OK
    assert L.fuse_verify_block(None, None, None, None, 0, pp, None, None, None, None) == lcd.LCD_OK
    assert L.rejection_accept(None, None, None, None, None, 64, None, None, 0, 0, 0, None, 0, None,
                              None, None, None, None, None, None) == lcd.LCD_OK
    assert L.greedy_accept(None, None, None, 0, None, None, None, None, None, None) == lcd.LCD_OK
    assert L.lookup_schedule_step(None, None, None, None, 0, pp, None, None) == lcd.LCD_OK


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(lcd, "LIB_PATH", "/nonexistent/liblcd.so")
    monkeypatch.setattr(lcd, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        lcd.load()


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        lcd.lookup_propose(x, torch.zeros(4, dtype=torch.int64), x, 4,
                           torch.zeros(4 * 8208 // 8, dtype=torch.int64),
                           x, x, torch.zeros(60, dtype=torch.int32))


def test_decode_step_rejects_misuse_without_launching():
    L = lcd.load()
    p = lcd.default_params()
    pp = ctypes.byref(p)
    f = 0x10000
    need = lcd.decode_step_workspace_bytes(8, 1000)
    assert need == 8 * 8208           # LCD_WORKSPACE_PER_REQUEST

    lo = 0x20000

    def call(B=8, max_len=1000, cap=f, ws=f, ws_bytes=need, append=1, hist=f, prm=pp, ln=f,
             ln_out=lo):
        P = _P
        return L.lookup_decode_step(P(hist), P(f), P(ln), P(ln_out), P(cap), B, max_len, P(f),
                                    P(f), P(f), prm, P(ws), ws_bytes, P(f), P(f), P(f), P(f), P(f),
                                    P(f), None, None, append, None)
    assert call(B=0, hist=None, ln=None, cap=None, ws=None, ws_bytes=0) == lcd.LCD_OK
    assert call(B=-1) == lcd.LCD_EINVAL
    assert call(ws_bytes=need - 8) == lcd.LCD_EINVAL          # workspace too small
    assert call(cap=None) == lcd.LCD_EINVAL                   # append needs capacities
    assert call(ln_out=None) == lcd.LCD_EINVAL                # ... and a second length array
    assert call(ln_out=f) == lcd.LCD_EINVAL                   # that is not the one read
    assert call(ln_out=f + 4 * 7) == lcd.LCD_EINVAL           # nor overlaps it
    assert call(ln_out=f - 4 * 7) == lcd.LCD_EINVAL
    assert call(hist=f + 4) == lcd.LCD_EINVAL                 # misaligned history
    assert call(ws=None) == lcd.LCD_EINVAL
    assert call(max_len=-5) == lcd.LCD_EINVAL
    bad = lcd.default_params(k_max=16)
    assert call(prm=ctypes.byref(bad)) == lcd.LCD_EINVAL
    bad = lcd.default_params(merge_polls=-2)
    assert call(prm=ctypes.byref(bad)) == lcd.LCD_EINVAL


def test_noalloc_step_rejects_misuse_without_launching():
    L = lcd.load()
    p = lcd.default_params()
    f = ctypes.c_void_p(0x10000)

    def call(B, prm=p):
        return L.lookup_decode_step_noalloc(f, f, f, f, f, B, 100, f, f, f, ctypes.byref(prm), f, f,
                                            f, f, f, f, f, None, 1, None)
    assert call(lcd.NOALLOC_MAX_B + 1) == lcd.LCD_EINVAL       # more than the static array holds
    assert call(-1) == lcd.LCD_EINVAL
    assert call(0) == lcd.LCD_OK
    assert call(0, lcd.default_params(k_max=16)) == lcd.LCD_EINVAL


def test_binding_needs_a_second_length_array_to_append():
    import torch
    x = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="lens_out"):
        lcd.lookup_decode_step(x, x, x, x, 4, x, x, x, x, x, x, x, x, x, x, append=True)


def test_same_launch_append_would_move_the_chunk_plan():
    """Why the fused step reads its lengths from an array it never writes: the
    launch derives every workgroup's (row, chunk) and whether it takes part
    from the rows' lengths, so a workgroup that started after another had
    appended a row's emitted tokens would work from another plan.  Shown with
    the host-compiled launch rule over a 256-step decode of 256 rows of
    1k-262k tokens (log-uniform), each step appending 1-16 tokens per row:
    token-balanced chunks (3000 workgroups), where one row's append can change
    the batch's chunk length or that row's chunk count (which moves every later
    row's workgroups), and equal chunks (4096 workgroups), where it can make
    one more chunk of the row take part (c * T < n - 1)."""
    rng = np.random.Generator(np.random.PCG64(5))
    lens = np.floor(np.exp(rng.uniform(np.log(1024), np.log(262144), 256))).astype(np.int64)
    B = len(lens)
    bal = lcd.default_params(scan_balance=1, scan_wgs=3000)
    eq = lcd.default_params(scan_wgs=4096)
    chunks = lambda n, T: np.maximum((n - 1 + T - 1) // T, 1)
    moved_bal = moved_eq = 0
    for _ in range(256):
        grow = rng.integers(1, 17, B)
        _, T0 = lcd.launch_shape(B, int(lens.max()), bal, lens)
        _, Te = lcd.launch_shape(B, int(lens.max()), eq, None)
        step_bal = step_eq = False
        for r in range(B):
            grown = lens.copy()
            grown[r] += grow[r]
            _, T1 = lcd.launch_shape(B, int(grown.max()), bal, grown)
            step_bal |= T1 != T0 or chunks(grown[r], T1) != chunks(lens[r], T0)
            # equal chunks are sized from the launch's max_len, so only the
            # participation test sees the append
            step_eq |= chunks(grown[r], Te) != chunks(lens[r], Te)
        moved_bal += step_bal
        moved_eq += step_eq
        lens += grow
    assert moved_bal > 0 and moved_eq > 0


def test_telemetry_entry_points_reject_misuse_without_launching():
    L = lcd.load()
    p = lcd.default_params()
    pp = ctypes.byref(p)
    f = 0x10000
    P = _P
    assert L.lookup_telemetry_update(None, None, None, None, None, None, None, None, 0, pp, None) == lcd.LCD_OK
    assert L.lookup_telemetry_update(P(f), P(f), P(f), P(f), P(f), P(f), P(f), P(f), -1, pp, None) == lcd.LCD_EINVAL
    assert L.lookup_telemetry_update(None, P(f), P(f), P(f), P(f), P(f), P(f), P(f), 4, pp, None) == lcd.LCD_EINVAL
    assert L.lookup_telemetry_update(P(f), P(f), P(f), P(f), P(f), P(f), P(f), P(f), 4, None, None) == lcd.LCD_EINVAL
    assert L.lookup_telemetry_reduce(P(f), P(f), 4, 0, None, None) == lcd.LCD_OK        # K = 0: no-op
    assert L.lookup_telemetry_reduce(P(f), P(f), 4, -1, P(f), None) == lcd.LCD_EINVAL
    assert L.lookup_telemetry_reduce(None, P(f), 4, 2, P(f), None) == lcd.LCD_EINVAL
    assert L.lookup_telemetry_reduce(P(f), P(f), 4, 2, None, None) == lcd.LCD_EINVAL


def test_rejection_accept_rejects_misuse_without_launching():
    """Host-checkable misuse returns LCD_EINVAL before any launch (the fake
    device pointers are never dereferenced)."""
    L = lcd.load()
    fake = 0x1000                      # 16-byte aligned, never touched
    s = None
    need = lcd.rejection_accept_workspace_bytes(3, 64)
    assert need == 3 * 8 * (2 + 1)
    assert lcd.rejection_accept_workspace_bytes(3, 1 << 20) == 3 * 8 * (2 + 1024)
    assert lcd.rejection_accept_workspace_bytes(0, 64) == 0

    def call(B=3, V=64, wg=0, ws_bytes=need, tp=fake, mp=None, ua=fake, hist=None, ro=None,
             ln=None, cp=None, ws=fake, block=fake, polls=0):
        return L.rejection_accept(_P(block), _P(fake), None, _P(tp), _P(mp) if mp else None, V,
                                  _P(ua), _P(fake), B, wg, polls, _P(ws), ws_bytes, _P(fake),
                                  _P(fake), _P(hist) if hist else None, _P(ro) if ro else None,
                                  _P(ln) if ln else None, _P(cp) if cp else None, s)

    assert call(V=62) == lcd.LCD_EINVAL                    # not a multiple of 4
    assert call(V=0) == lcd.LCD_EINVAL
    assert call(V=lcd.SAMPLE_MAX_VOCAB + 4) == lcd.LCD_EINVAL
    assert call(B=-1) == lcd.LCD_EINVAL
    assert call(wg=-1) == lcd.LCD_EINVAL
    assert call(wg=257) == lcd.LCD_EINVAL                   # at most 256 units per workgroup
    assert call(polls=-2) == lcd.LCD_EINVAL
    assert call(ws_bytes=need - 8) == lcd.LCD_EINVAL        # workspace too small
    assert call(tp=fake + 4) == lcd.LCD_EINVAL              # target rows not 16-byte aligned
    assert call(mp=fake + 8) == lcd.LCD_EINVAL
    assert call(ws=fake + 4) == lcd.LCD_EINVAL
    assert call(ua=0) == lcd.LCD_EINVAL
    assert call(block=0) == lcd.LCD_EINVAL
    assert call(hist=fake, ro=fake, ln=None, cp=fake) == lcd.LCD_EINVAL   # append needs len


def test_index_plan_sizes_tables_on_the_host():
    """lookup_index_plan runs on the host: tables of exactly index_load slots
    per indexed length and token of capacity (at least 16), laid out back to
    back after 256 bytes of token cache per request: 8 x 3 x 9 = 216 bytes per
    token of capacity at the defaults, 144 with index_load = 2."""
    L = lcd.load()
    cap = np.array([0, 1, 100, 25_000, 262_144], np.int32)
    for load in (3, 2, 4, 16):
        p = lcd.default_params(index_load=load)
        off = np.zeros(5, np.int64)
        slots = np.zeros(5, np.int32)
        total = L.lookup_index_plan(cap.ctypes.data_as(ctypes.c_void_p), 5, ctypes.byref(p),
                                    off.ctypes.data_as(ctypes.c_void_p),
                                    slots.ctypes.data_as(ctypes.c_void_p))
        nL = p.l_max - p.l_min + 1
        want = np.maximum(load * nL * np.maximum(cap.astype(np.int64), 1), 16)
        assert slots.tolist() == want.tolist()
        # 32 words of token cache per request first, then the tables
        assert off.tolist() == (32 * 5 + np.concatenate([[0], np.cumsum(want)[:-1]])).tolist()
        assert total == 8 * (32 * 5 + int(want.sum()))
        # bytes per token of capacity, past the token caches and the 16-slot minimum
        assert 8 * int(want[2:].sum()) == 8 * load * nL * int(cap[2:].sum())
    bits = np.zeros(5, np.int32)
    off = np.zeros(5, np.int64)
    p = lcd.default_params()
    # misuse
    bad_cap = np.array([5, -1], np.int32)
    assert L.lookup_index_plan(bad_cap.ctypes.data_as(ctypes.c_void_p), 2, ctypes.byref(p),
                               off.ctypes.data_as(ctypes.c_void_p),
                               bits.ctypes.data_as(ctypes.c_void_p)) == lcd.LCD_EINVAL
    bad = lcd.default_params(l_max=20)
    assert L.lookup_index_plan(cap.ctypes.data_as(ctypes.c_void_p), 5, ctypes.byref(bad),
                               off.ctypes.data_as(ctypes.c_void_p),
                               bits.ctypes.data_as(ctypes.c_void_p)) == lcd.LCD_EINVAL
    assert L.lookup_index_plan(None, 0, ctypes.byref(p), None, None) == 0


def test_index_entry_points_reject_misuse_without_launching():
    L = lcd.load()
    p = lcd.default_params()
    pp = ctypes.byref(p)
    f = _P(0x1000)
    s = None
    # build: fingerprint bits out of range, missing scratch, misaligned tables
    assert L.lookup_index_build(f, f, f, 3, pp, 32, f, f, f, 64, f, f, 10, s) == lcd.LCD_EINVAL
    assert L.lookup_index_build(f, f, f, 3, pp, 0, f, f, f, 64, f, None, 10, s) == lcd.LCD_EINVAL
    assert L.lookup_index_build(f, f, f, 3, pp, 0, f, f, _P(0x1004), 64, f, f, 10, s) == lcd.LCD_EINVAL
    assert L.lookup_index_build(f, f, f, 3, pp, 0, f, f, f, 64, f, f, -1, s) == lcd.LCD_EINVAL
    assert L.lookup_index_build(None, None, None, 0, pp, 0, None, None, None, 0, None, None, 0,
                                s) == lcd.LCD_OK
    # propose
    assert L.lookup_index_propose(f, f, f, 3, pp, -1, f, f, f, f, f, f, f, s) == lcd.LCD_EINVAL
    assert L.lookup_index_propose(f, f, f, 3, pp, 0, f, f, f, None, f, f, f, s) == lcd.LCD_EINVAL
    bad = lcd.default_params(l_min=0)
    assert L.lookup_index_propose(f, f, f, 3, ctypes.byref(bad), 0, f, f, f, f, f, f, f,
                                  s) == lcd.LCD_EINVAL
    assert L.lookup_index_propose(None, None, None, 0, pp, 0, None, None, None, None, None, None,
                                  None, s) == lcd.LCD_OK
    # the whole step through the index: the propose checks plus the step's own
    # (hist, row_off, len, cap, B, p, fp_bits, table_off, table_slots, tables,
    #  indexed_len, model_draft, target, state, match_len, match_end, draft,
    #  block, block_len, accept, long_next, telemetry, append, stream)
    step = lambda *a: L.lookup_index_decode_step(*a)
    ok = [f, f, f, f, 3, pp, 0, f, f, f, f, f, f, f, f, f, f, f, f, f, None, None, 1, s]
    for i, v in ((6, 32), (9, _P(0x1004)), (10, None), (11, None), (12, None), (13, None),
                 (17, None), (18, None), (19, None), (3, None)):
        args = list(ok)
        args[i] = v
        assert step(*args) == lcd.LCD_EINVAL, i
    args = list(ok)
    args[5] = ctypes.byref(bad)
    assert step(*args) == lcd.LCD_EINVAL
    args = list(ok)
    args[4] = -1
    assert step(*args) == lcd.LCD_EINVAL
    args = [None] * 24
    args[4], args[5], args[6], args[22] = 0, pp, 0, 1
    assert step(*args) == lcd.LCD_OK                  # B = 0: nothing to do


def test_launch_shape_query():
    """Equal chunks per row without lengths; token-balanced chunks need the
    rows' lengths (host) and cover every row's candidate ends within the grid."""
    p = lcd.default_params()
    assert lcd.launch_shape(64, 25_000, p) == (256, 6400)
    # fewer than 32 rows of 6k+ tokens: one workgroup per ~12k tokens of the
    # longest row, at most 256 in all
    assert lcd.launch_shape(16, 8_192, p) == (16, 8192)
    assert lcd.launch_shape(1, 5_999, p) == (3, 2048)          # 4-wave launch below 6k
    assert lcd.launch_shape(1, 25_000, p) == (2, 12544)
    assert lcd.launch_shape(1, 150_000, p) == (12, 12544)
    assert lcd.launch_shape(16, 150_000, p) == (192, 12544)
    assert lcd.launch_shape(31, 262_144, p) == (248, 32768)
    # 16-wave workgroups (one per CU) never exceed the 256 CUs
    for B in range(1, 129):
        for n in (16_384, 25_000, 150_000, 262_144):
            assert lcd.launch_shape(B, n, p)[0] <= 256, (B, n)
    assert lcd.launch_shape(100, 150_000, p)[0] == 200
    # 32-128 rows of 8k-16k tokens: 16-wave from 1.2M tokens in all
    assert lcd.launch_shape(100, 14_000, p) == (200, 7168)
    assert lcd.launch_shape(100, 12_000, p) == (200, 6144)    # 1.2M exactly
    assert lcd.launch_shape(100, 11_999, p)[0] == 300         # 4-wave below 1.2M
    pb = lcd.default_params(scan_balance=1)
    with pytest.raises(lcd.LCDError):
        lcd.launch_shape(256, 262_144, pb)
    lens = np.array([1024 * (1 + (r % 7)) for r in range(255)] + [262_144], np.int32)
    wgs, T = lcd.launch_shape(256, 262_144, pb, lens)
    assert T % 256 == 0
    chunks = sum(max(1, -(-(int(n) - 1) // T)) for n in lens)
    assert chunks <= wgs and max(-(-(int(n) - 1) // T) for n in lens) <= 64
    # over the balanced limit the equal-chunk shape is used
    big = np.full(1100, 100, np.int32)
    assert lcd.launch_shape(1100, 100, pb, big) == lcd.launch_shape(1100, 100, p)


def test_automatic_grids_of_large_batches():
    """Batches past the 16-wave shapes get about one 4-wave workgroup per 12k
    tokens of B x max_len, at most 4 dispatch rounds of the 7 x 256 resident
    workgroups (chunks of ~12k tokens of the longest row where that fits),
    unless 32768-token chunks of the longest row need more; the token-balanced
    default stays within one round; explicit scan_wgs and one-chunk-per-row
    batches are left alone."""
    p = lcd.default_params()
    assert lcd.launch_shape(256, 262_144, p) == (22 * 256, 12_032)   # 262,143 ends in 22 chunks
    assert lcd.launch_shape(256, 53_600, p) == (1024, 13_568)
    assert lcd.launch_shape(200, 150_000, p) == (2600, 11_776)
    for B, n in ((200, 262_144), (300, 150_000), (512, 100_000)):
        wgs, T = lcd.launch_shape(B, n, p)
        assert wgs % B == 0 and T % 256 == 0 and abs(T - 12_000) <= 1_000, (B, n, T)
    assert lcd.launch_shape(512, 262_144, p) == (4 * 7 * 256, 18_944)  # the 4-round cap
    assert lcd.launch_shape(1024, 262_144, p) == (8 * 1024, 32_768)   # 32k-token chunks at most
    assert lcd.launch_shape(1024, 1 << 20, p) == (32 * 1024, 32_768)
    assert lcd.launch_shape(256, 262_144, lcd.default_params(scan_wgs=2048))[0] == 2048
    assert lcd.launch_shape(2000, 262_144, p)[0] == 2000 * 8
    assert lcd.launch_shape(2000, 1000, p) == (2000, 1024)
    pb = lcd.default_params(scan_balance=1)
    assert lcd.launch_shape(512, 4096, pb, np.full(512, 4096, np.int32))[0] == 1792
    with pytest.raises(lcd.LCDError):
        lcd.scan_occupancy(8)
