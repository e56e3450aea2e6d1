"""GPU <-> oracle parity, bit-exact, through the C ABI (via the binding).

Every comparison is element by element on the same seeded inputs: match
lengths, match ends, drafts, fused blocks, block lengths, accept counts,
appended histories, scheduler states and next modes.
"""

import numpy as np
import pytest

import oracle
from context_lookup_drafting_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _lcd():
    import context_lookup_drafting_amd as lcd
    return lcd


def lookup_ws_clean(ws, B):
    """Every arrival count, pad word and slot of a lookup workspace for B
    requests is zero (each header word keeps the request's call epoch in its
    upper half)."""
    words = 8208 // 8                     # LCD_WORKSPACE_PER_REQUEST
    w = ws.cpu().numpy()[: B * words].reshape(B, words)
    return bool((w[:, 0] & 0xFFFFFFFF == 0).all() and (w[:, 1:] == 0).all())


def _oparams(p):
    """Oracle parameters with the same values as a binding Params."""
    return oracle.default_params(**{n: getattr(p, n) for n, _ in oracle.OracleParams._fields_})


def gpu_lookup(flat, row_off, lens, params=None, max_len=None, device="cuda:0", ws=None):
    import torch
    lcd = _lcd()
    p = params or lcd.default_params()
    B = len(lens)
    dev = torch.device(device)
    h = torch.from_numpy(np.ascontiguousarray(flat, dtype=np.int32)).to(dev)
    ro = torch.from_numpy(np.ascontiguousarray(row_off, dtype=np.int64)).to(dev)
    ln = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to(dev)
    own_ws = ws is None
    if own_ws:
        ws = lcd.alloc_workspace(B, dev)
    m = torch.full((B,), 77, dtype=torch.int32, device=dev)
    e = torch.full((B,), 77, dtype=torch.int32, device=dev)
    d = torch.full((B, 15), 77, dtype=torch.int32, device=dev)
    if max_len is None:
        max_len = int(lens.max()) if B else 0
    lcd.lookup_propose(h, ro, ln, max_len, ws, m, e, d, p)
    torch.cuda.synchronize()
    if own_ws:
        assert lookup_ws_clean(ws, B), "workspace not left clean"
    return m.cpu().numpy(), e.cpu().numpy(), d.cpu().numpy()


def assert_lookup_parity(flat, row_off, lens, params=None, **kw):
    lcd = _lcd()
    p = params or lcd.default_params()
    m, e, d = gpu_lookup(flat, row_off, lens, p, **kw)
    om, oe, od = oracle.lookup_propose(flat, row_off, lens, _oparams(p))
    bad = np.nonzero((m != om) | (e != oe) | np.any(d != od, axis=1))[0]
    assert bad.size == 0, (f"{bad.size} requests differ; first r={bad[0]}: gpu m={m[bad[0]]} "
                           f"e={e[bad[0]]} oracle m={om[bad[0]]} e={oe[bad[0]]} n={lens[bad[0]]}")
    return m, e, d


def gpu_fuse_accept(draft, m, q, long_mode, target, params=None):
    import torch
    lcd = _lcd()
    p = params or lcd.default_params()
    dev = torch.device("cuda:0")
    B = len(m)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    blk = torch.empty((B, 15), dtype=torch.int32, device=dev)
    bl = torch.empty(B, dtype=torch.int32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    mask = torch.full((B,), -7, dtype=torch.int32, device=dev)
    lcd.fuse_verify_block(t(draft), t(m), t(q), t(long_mode), blk, bl, p, model_mask=mask)
    lcd.greedy_accept(blk, bl, t(target), acc)
    torch.cuda.synchronize()
    return blk.cpu().numpy(), bl.cpu().numpy(), acc.cpu().numpy(), mask.cpu().numpy().view(np.uint32)


def assert_step_parity(w, d, m, long_mode, params=None):
    lcd = _lcd()
    p = params or lcd.default_params()
    q, tgt = w.step_inputs(np.zeros(w.B, np.int64), 0)
    blk, bl, acc, mask = gpu_fuse_accept(d, m, q, long_mode, tgt, p)
    oblk, obl, omask = oracle.fuse_verify_block(d, m, q, long_mode, _oparams(p), with_mask=True)
    oacc = oracle.greedy_accept(oblk, obl, tgt)
    np.testing.assert_array_equal(mask, omask)
    np.testing.assert_array_equal(blk, oblk)
    np.testing.assert_array_equal(bl, obl)
    np.testing.assert_array_equal(acc, oacc)
    return acc


# ---------------------------------------------------------------------------
# configs
# ---------------------------------------------------------------------------

def test_config1_single_and_every_prefix(gpu):
    w = wl.config1()
    flat, ro, ln, cap = wl.pack_rows(w.hists)
    m, e, d = assert_lookup_parity(flat, ro, ln)
    assert m[0] == 12 and 2048 - 1 - e[0] == 5
    for lg in (0, 1):
        acc = assert_step_parity(w, d, m, np.array([lg], np.int32))
        j = int(w.note.split()[-1])
        assert acc[0] == (min(j, 7) if lg == 0 else min(j, 15))
    # every prefix length 1..2048 as one ragged, tightly packed batch
    flat, ro, ln = wl.pack_csr(wl.prefix_batch(w.hists[0]))
    assert_lookup_parity(flat, ro, ln)


def test_config4_full_batch(gpu):
    w = wl.config4()
    flat, ro, ln, cap = wl.pack_rows(w.hists)
    m, e, d = assert_lookup_parity(flat, ro, ln)
    for lg in (0, 1):
        assert_step_parity(w, d, m, np.full(w.B, lg, np.int32))


def test_config5_ragged_batch(gpu):
    w = wl.config5()
    flat, ro, ln = wl.pack_csr(w.hists)             # unaligned CSR rows
    m, e, d = assert_lookup_parity(flat, ro, ln)
    for lg in (0, 1):
        assert_step_parity(w, d, m, np.full(w.B, lg, np.int32))
    flat, ro, ln, cap = wl.pack_rows(w.hists)       # padded rows
    assert_lookup_parity(flat, ro, ln)


def _compare_sims(a, b):
    assert len(a["recs"]) == len(b["recs"])
    for t, (ra, rb) in enumerate(zip(a["recs"], b["recs"])):
        for k in ("m", "e", "d", "long", "block", "blk", "acc", "state", "long_next"):
            if not np.array_equal(ra[k], rb[k]):
                bad = np.nonzero(np.any(np.asarray(ra[k]).reshape(len(ra["m"]), -1)
                                        != np.asarray(rb[k]).reshape(len(rb["m"]), -1), axis=1))[0]
                raise AssertionError(f"step {t}: field {k} differs for requests {bad[:8]}")
    np.testing.assert_array_equal(a["lens"], b["lens"])
    np.testing.assert_array_equal(a["flat"], b["flat"])
    if "tele" in a and "tele" in b:                    # acceptance telemetry rows
        np.testing.assert_array_equal(a["tele"], b["tele"])


def test_config2_simulation_200_steps(gpu):
    from simulate import simulate_gpu, simulate_oracle
    w = wl.config2()
    g = simulate_gpu(w, 200)
    o = simulate_oracle(w, 200)
    _compare_sims(g, o)
    em = g["emitted"][0]
    assert em == w.truths[0][:len(em)].tolist()
    assert lookup_ws_clean(g["ws"], w.B)


def test_config3_simulation_256_steps(gpu):
    from simulate import simulate_gpu, simulate_oracle
    w = wl.config3()
    g = simulate_gpu(w, 256)
    o = simulate_oracle(w, 256)
    _compare_sims(g, o)
    for r in range(w.B):
        em = g["emitted"][r]
        assert em == w.truths[r][:len(em)].tolist()


# ---------------------------------------------------------------------------
# exhaustive tiny vocabularies as one huge ragged batch
# ---------------------------------------------------------------------------

def test_exhaustive_tiny_vocab_batches(gpu):
    for alphabet, n_max in ((3, 12), (2, 18)):
        hs = []
        for n in range(0, n_max + 1):
            X = wl.all_strings(alphabet, n)
            hs.extend(list(X))
        flat, ro, ln = wl.pack_csr(hs)
        assert_lookup_parity(flat, ro, ln)


# ---------------------------------------------------------------------------
# edge cases, parameters, launch shapes
# ---------------------------------------------------------------------------

def _stress_batch(seed=11, B=300):
    rng = np.random.Generator(np.random.PCG64(seed))
    hs = []
    for k in range(B):
        kind = k % 6
        n = int(rng.integers(0, 3000))
        if kind == 0:
            h = rng.integers(0, int(rng.integers(2, 5)), n)
        elif kind == 1:
            h = rng.integers(0, 50_000, n)
            if n > 64:
                L = int(rng.integers(4, 40))
                s = int(rng.integers(0, n - 2 * L))
                h[n - L:] = h[s:s + L]
        elif kind == 2:
            h = rng.integers(0, 50_000, n)
            P = int(rng.integers(1, 17))
            run = int(rng.integers(0, n + 1))
            h[n - run:] = np.resize(rng.integers(0, 50_000, max(P, 1)), run)
        elif kind == 3:
            h = np.full(n, 5)
        elif kind == 4:
            h = rng.choice(np.array([-1, 0, 2**31 - 1, -2**31, 7]), n)
        else:
            n = int(rng.integers(0, 20))
            h = rng.integers(0, 3, n)
        hs.append(h.astype(np.int32))
    return hs


@pytest.mark.parametrize("prm", [
    dict(), dict(l_min=1, l_max=1), dict(l_min=1, l_max=16), dict(l_min=2, l_max=5, k_max=7),
    dict(l_min=3, l_max=16), dict(l_min=4, l_max=16, k_max=0), dict(l_min=12, l_max=12),
    dict(l_min=6, l_max=9, k_max=3),
])
def test_stress_params(gpu, prm):
    lcd = _lcd()
    p = lcd.default_params(**prm)
    hs = _stress_batch()
    flat, ro, ln = wl.pack_csr(hs)
    assert_lookup_parity(flat, ro, ln, p)


@pytest.mark.parametrize("wgs", [1, 2, 3, 7, 64, 257, 968, 1000, 3872, 4096])
def test_launch_shapes_do_not_change_results(gpu, wgs):
    """121 rows: 120 of up to 3,000 tokens and one of 25,000, so most chunks of
    most rows are empty; 968 and 3,872 workgroups give 8 and 32 chunks per row
    (the chunk order within a row is rotated by the row)."""
    lcd = _lcd()
    hs = _stress_batch(seed=5, B=120) + [wl.config2().hists[0]]
    flat, ro, ln = wl.pack_csr(hs)
    assert_lookup_parity(flat, ro, ln, lcd.default_params(scan_wgs=wgs))
    assert_lookup_parity(flat, ro, ln, lcd.default_params(scan_wgs=wgs), max_len=0)


def test_automatic_grid_is_resident(gpu):
    """The token-balanced launch rule assumes 7 resident 4-wave workgroups per
    CU on a 256-CU part; the runtime's occupancy for the compiled kernels must
    allow at least that (a kernel change that costs registers would break it)."""
    import numpy as np
    import torch
    lcd = _lcd()
    assert torch.cuda.get_device_properties(0).multi_processor_count == 256
    assert lcd.scan_occupancy(4) >= 7
    assert lcd.scan_occupancy(16) >= 1
    pb = lcd.default_params(scan_balance=1)
    lens = np.full(512, 262_144, np.int32)
    assert lcd.launch_shape(512, 262_144, pb, lens)[0] == 7 * 256 <= lcd.scan_occupancy(4) * 256


def test_match_across_workgroup_boundaries(gpu):
    """Rows split over many workgroups with the winning occurrence straddling
    range boundaries at every offset."""
    lcd = _lcd()
    rng = np.random.Generator(np.random.PCG64(21))
    hs = []
    for off in range(0, 40):
        n = 4096
        h = rng.integers(0, 1 << 20, n).astype(np.int32)
        L = 12
        end = 256 * 7 + off - 6          # occurrence ends near a 256-token tile edge
        h[n - L:] = h[end - L + 1:end + 1]
        hs.append(h)
    flat, ro, ln = wl.pack_csr(hs)
    for wgs in (40 * 16, 40 * 8, 40 * 3):
        m, e, d = assert_lookup_parity(flat, ro, ln, lcd.default_params(scan_wgs=wgs))
        assert np.all(m == 12)


@pytest.mark.parametrize("k", [4, 5])
def test_small_batches_of_long_rows(gpu, k):
    """Batches of 1-100 rows of 16k+ tokens (16-wave workgroups: one per ~12k
    tokens of the longest row below 32 rows, at most one per CU from 32):
    lookup, and the fused step on the same rows, equal the oracle's."""
    import torch
    lcd = _lcd()
    w = wl.make_config(k)
    order = np.argsort([-len(h) for h in w.hists], kind="stable")
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    op = _oparams(lcd.default_params())
    for B in (1, 7, 16, 31, 37, 100):
        sel = order[np.arange(B) % len(order)]
        hs = [w.hists[i] for i in sel]
        flat, ro, ln, cap = wl.pack_rows(hs, extra=16)
        assert lcd.launch_shape(B, int(ln.max()))[0] >= B
        m, e, d = assert_lookup_parity(flat, ro, ln)
        q, tgt = w.step_inputs(np.zeros(w.B, np.int64), 0)
        q, tgt = q[sel], tgt[sel]
        h_d, ln_d = t(flat), t(ln.copy())
        dr = lcd.LookupDrafter(B, int(ln.max()), dev)
        out = dr.step(h_d, t(ro), ln_d, t(cap), t(q), t(tgt))
        torch.cuda.synchronize()
        oblk, obl = oracle.fuse_verify_block(d, m, q, np.zeros(B, np.int32), op)
        o_flat, o_ln = flat.copy(), ln.copy()
        oacc = oracle.greedy_accept(oblk, obl, tgt, o_flat, ro, o_ln, cap)
        np.testing.assert_array_equal(out["match_len"].cpu().numpy(), m)
        np.testing.assert_array_equal(out["match_end"].cpu().numpy(), e)
        np.testing.assert_array_equal(out["block"].cpu().numpy(), oblk)
        np.testing.assert_array_equal(out["accept"].cpu().numpy(), oacc)
        np.testing.assert_array_equal(h_d.cpu().numpy(), o_flat)
        np.testing.assert_array_equal(ln_d.cpu().numpy(), o_ln)


def test_small_batch_rows_longer_than_max_len(gpu):
    """16-wave launches of 1-3 rows sized from a max_len below the rows' true
    lengths (each workgroup then takes every cpr-th chunk), and rows on both
    sides of the 6k- and 16k-token thresholds of the 16-wave launches."""
    lcd = _lcd()
    w = wl.config4()
    hs = [w.hists[i] for i in range(3)]
    for B in (1, 3):
        flat, ro, ln, cap = wl.pack_rows(hs[:B])
        for ml in (16_384, 20_000, 30_000, 70_000):
            assert lcd.launch_shape(B, ml)[1] < int(ln.max())
            assert_lookup_parity(flat, ro, ln, max_len=ml)
    for n in (5_999, 6_000, 8_192, 16_383, 16_384, 16_385, 24_577):
        flat, ro, ln = wl.pack_csr([h[-n:] for h in hs])
        assert_lookup_parity(flat, ro, ln)
    # 32-128 rows of 8k-16k tokens, on both sides of 1.2M tokens in all
    for B, n in ((64, 14_000), (100, 14_000), (128, 9_500)):
        flat, ro, ln = wl.pack_csr([w.hists[i % w.B][-n:] for i in range(B)])
        assert_lookup_parity(flat, ro, ln)


def test_match_across_long_chunk_boundaries(gpu):
    """One 40k-token row cut into 16-wave chunks, with the winning occurrence
    ending at every offset around a chunk edge."""
    lcd = _lcd()
    rng = np.random.Generator(np.random.PCG64(23))
    n = 40_000
    wgs, T = lcd.launch_shape(1, n)
    assert wgs >= 2
    for edge in (T, 2 * T):
        hs = []
        for off in range(-13, 14):
            h = rng.integers(0, 1 << 20, n).astype(np.int32)
            L = 12
            end = edge + off
            h[n - L:] = h[end - L + 1:end + 1]
            hs.append(h)
        for h in hs:
            flat, ro, ln = wl.pack_csr([h])
            m, e, d = assert_lookup_parity(flat, ro, ln)
            assert m[0] == 12


def test_empty_and_tiny_rows(gpu):
    hs = [np.zeros(0, np.int32), np.array([1], np.int32), np.array([1, 1], np.int32),
          np.array([2, 2, 2, 2], np.int32), np.array([2, 2, 2, 2, 2], np.int32),
          np.zeros(0, np.int32)] + [np.full(k, 3, np.int32) for k in range(0, 30)]
    flat, ro, ln = wl.pack_csr(hs)
    assert_lookup_parity(flat, ro, ln)
    ln2 = ln.copy()
    ln2[3] = -5                                      # negative length reads as empty
    m, e, d = gpu_lookup(flat, ro, ln2)
    assert m[3] == 0 and e[3] == -1 and np.all(d[3] == -1)


def test_repeatable_and_workspace_reuse(gpu):
    import torch
    lcd = _lcd()
    w = wl.config3(steps=1)
    flat, ro, ln, cap = wl.pack_rows(w.hists)
    ws = lcd.alloc_workspace(w.B, "cuda:0")
    ref = gpu_lookup(flat, ro, ln, ws=ws)
    for _ in range(20):
        out = gpu_lookup(flat, ro, ln, ws=ws)
        for a, b in zip(ref, out):
            np.testing.assert_array_equal(a, b)
    assert lookup_ws_clean(ws, w.B)


def test_large_batch_split_launches(gpu):
    """B above the per-launch limit is split into several launches."""
    rng = np.random.Generator(np.random.PCG64(9))
    hs = [rng.integers(0, 4, int(rng.integers(0, 60))).astype(np.int32) for _ in range(2500)]
    flat, ro, ln = wl.pack_csr(hs)
    assert_lookup_parity(flat, ro, ln)


def test_schedule_parity_random(gpu):
    import torch
    lcd = _lcd()
    rng = np.random.Generator(np.random.PCG64(4))
    B = 1000
    p = lcd.default_params()
    dev = torch.device("cuda:0")
    st_h = np.zeros((B, 3), np.int32)
    st_d = torch.zeros((B, 3), dtype=torch.int32, device=dev)
    ln_d = torch.empty(B, dtype=torch.int32, device=dev)
    for t in range(60):
        m = rng.integers(0, 13, B).astype(np.int32)
        blk = np.where(st_h[:, 0] == 1, 15, 7).astype(np.int32)
        a = np.minimum(rng.integers(-1, 17, B), blk).astype(np.int32)
        tt = lambda x: torch.from_numpy(x).to(dev)
        lcd.lookup_schedule_step(st_d, tt(m), tt(a), tt(blk), ln_d, p)
        o = oracle.lookup_schedule_step(st_h, m, a, blk, _oparams(p))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(st_d.cpu().numpy(), st_h)
        np.testing.assert_array_equal(ln_d.cpu().numpy(), o)


def test_fuse_accept_parity_random(gpu):
    lcd = _lcd()
    rng = np.random.Generator(np.random.PCG64(8))
    B = 2000
    for prm in (dict(), dict(n_head=5, n_block=11, k_max=9, agree_n=3, head_full=10),
                dict(n_block=7), dict(agree_n=0, head_agree=4)):
        p = lcd.default_params(**prm)
        m = rng.integers(0, 13, B).astype(np.int32)
        d = rng.integers(0, 3, (B, 15)).astype(np.int32)
        d[m == 0] = -1
        q = rng.integers(0, 3, (B, 7)).astype(np.int32)
        lg = rng.integers(0, 2, B).astype(np.int32)
        tgt = rng.integers(0, 3, (B, 16)).astype(np.int32)
        blk, bl, acc, mask = gpu_fuse_accept(d, m, q, lg, tgt, p)
        oblk, obl, omask = oracle.fuse_verify_block(d, m, q, lg, _oparams(p), with_mask=True)
        np.testing.assert_array_equal(mask, omask)
        np.testing.assert_array_equal(blk, oblk)
        np.testing.assert_array_equal(bl, obl)
        np.testing.assert_array_equal(acc, oracle.greedy_accept(oblk, obl, tgt))


def test_accept_append_capacity_parity(gpu):
    import torch
    lcd = _lcd()
    rng = np.random.Generator(np.random.PCG64(12))
    B = 300
    hs = [rng.integers(0, 9, int(rng.integers(0, 40))).astype(np.int32) for _ in range(B)]
    flat, ro, ln, cap = wl.pack_rows(hs, extra=int(0))
    cap = np.minimum(cap, ln + rng.integers(0, 20, B)).astype(np.int32)
    blk = rng.integers(0, 2, (B, 15)).astype(np.int32)
    bl = rng.choice(np.array([7, 15], np.int32), B)
    tgt = rng.integers(0, 2, (B, 16)).astype(np.int32)
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h_d, ln_d, acc_d = t(flat), t(ln), torch.empty(B, dtype=torch.int32, device=dev)
    lcd.greedy_accept(t(blk), t(bl), t(tgt), acc_d, hist=h_d, row_off=t(ro), lens=ln_d, cap=t(cap))
    o_flat, o_ln = flat.copy(), ln.copy()
    oacc = oracle.greedy_accept(blk, bl, tgt, o_flat, ro, o_ln, cap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc_d.cpu().numpy(), oacc)
    np.testing.assert_array_equal(ln_d.cpu().numpy(), o_ln)
    np.testing.assert_array_equal(h_d.cpu().numpy(), o_flat)
    assert (oacc == -1).any() and (oacc >= 0).any()


def test_telemetry_reduce_matches_oracle(gpu):
    import torch
    import context_lookup_drafting_amd as lcd
    rng = np.random.Generator(np.random.PCG64(11))
    for B, K in ((0, 3), (1, 1), (300, 5), (4096, 2)):
        tele = rng.integers(0, 2**32, (B, 32), dtype=np.uint64).astype(np.uint32)
        cls = rng.integers(-1, K + 1, B).astype(np.int32)
        got = lcd.telemetry_reduce(torch.from_numpy(tele.view(np.int32)).cuda(),
                                   torch.from_numpy(cls).cuda(), K)
        want = oracle.telemetry_reduce(tele, cls, K)
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint64), want)


def test_telemetry_per_class_config3(gpu):
    """Per-class totals of a 256-step config-3 decode through the fused step
    equal the oracle's; the copy-mode class hits and accepts far more."""
    import torch
    import context_lookup_drafting_amd as lcd
    from simulate import simulate_gpu_fused, simulate_oracle
    w = wl.config3()
    g = simulate_gpu_fused(w, 256)
    o = simulate_oracle(w, 256)
    np.testing.assert_array_equal(g["tele"], o["tele"])
    cls = w.class_ids
    got = lcd.telemetry_reduce(torch.from_numpy(g["tele"].view(np.int32)).cuda(),
                               torch.from_numpy(cls).cuda(), 2).cpu().numpy().view(np.uint64)
    np.testing.assert_array_equal(got, oracle.telemetry_reduce(o["tele"], cls, 2))
    copy, plain = got[0].astype(np.float64), got[1].astype(np.float64)
    assert copy[1] / copy[0] > 0.4 and plain[1] / plain[0] < 0.05         # hit rates
    assert copy[7] / copy[0] > 1.5 * (plain[7] / plain[0])                # tokens per step
    assert copy[4] > 0 and plain[4] == 0                                  # long-block steps


def test_decode_replay_report_config3(gpu):
    """The package's decode replay emits exactly the target's stream and its
    per-class report is the oracle's per-class totals, restated."""
    from context_lookup_drafting_amd.decode_sim import run_fused, summarise
    from simulate import simulate_oracle
    w = wl.config3()
    steps = 96
    g = run_fused(w, steps, record=False)
    for r in range(w.B):
        em = g["emitted"][r]
        assert em == w.truths[r][:len(em)].tolist()
    rep = summarise(g["tele_d"], w.class_ids, w.CLASS_NAMES)
    tot = oracle.telemetry_reduce(simulate_oracle(w, steps)["tele"], w.class_ids, 2)
    for k, name in enumerate(w.CLASS_NAMES):
        t = tot[k].astype(np.int64)
        c = rep[name]
        assert c["requests"] == int((w.class_ids == k).sum())
        assert c["steps"] == t[0] == c["requests"] * steps
        assert c["hit_rate"] == round(t[1] / t[0], 4)
        assert c["tokens_per_step"] == round(t[7] / t[0], 3)
        assert c["long_entries"] == t[5] and c["long_exits"] == t[6]
        assert c["accepted_hist"] == t[9:25].tolist()


# ---------------------------------------------------------------------------
# token-balanced chunks (scan_balance = 1): same results, other launch shape
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", [3, 4, 5])
def test_balanced_scan_configs(gpu, k):
    lcd = _lcd()
    w = wl.make_config(k)
    flat, ro, ln, cap = wl.pack_rows(w.hists)
    for wgs in (0, 1, 3000):
        assert_lookup_parity(flat, ro, ln, lcd.default_params(scan_balance=1, scan_wgs=wgs))


def test_balanced_scan_stress_and_edges(gpu):
    """Ragged stress rows, empty and tiny rows, rows longer than max_len, and
    a batch over the balanced limit (which falls back to equal chunks)."""
    lcd = _lcd()
    p = lcd.default_params(scan_balance=1)
    hs = _stress_batch(seed=17, B=300)
    flat, ro, ln = wl.pack_csr(hs)
    assert_lookup_parity(flat, ro, ln, p)
    assert_lookup_parity(flat, ro, ln, p, max_len=0)          # rows longer than max_len
    hs2 = [np.zeros(0, np.int32), np.array([1], np.int32)] + [np.full(k, 3, np.int32) for k in range(30)]
    flat2, ro2, ln2 = wl.pack_csr(hs2)
    assert_lookup_parity(flat2, ro2, ln2, p)
    big = _stress_batch(seed=19, B=1100)                      # B > 1024
    flat3, ro3, ln3 = wl.pack_csr(big)
    assert_lookup_parity(flat3, ro3, ln3, p)


def test_balanced_scan_batches_at_the_limit(gpu):
    """Token-balanced chunks at 1,024 rows (all 16 groups of 64 lengths per
    lane present), 1,023 and 961 rows (the last group partial), each with one
    50k-token row among short ones: every length load of a lane is in flight at
    once and rows past the batch are masked."""
    lcd = _lcd()
    p = lcd.default_params(scan_balance=1)
    long_row = wl.config4(B=1, n=50_000).hists[0]
    for B in (1024, 1023, 961):
        hs = _stress_batch(seed=23 + B, B=B - 1) + [long_row]
        flat, ro, ln = wl.pack_csr(hs)
        assert lcd.launch_shape(B, int(ln.max()), p, ln)[0] >= B
        assert_lookup_parity(flat, ro, ln, p)


def test_balanced_fused_simulation(gpu):
    """The fused decode step with token-balanced chunks: 128 steps of config 3
    equal the oracle's simulation."""
    lcd = _lcd()
    from context_lookup_drafting_amd.decode_sim import run_fused
    from simulate import simulate_oracle
    w = wl.config3()
    g = run_fused(w, 128, params=lcd.default_params(scan_balance=1), record=True)
    g.pop("tele_d")
    _compare_sims(g, simulate_oracle(w, 128))


def test_balanced_fused_step_ragged(gpu):
    """One fused step over the ragged 256-request batch, both launch modes."""
    import torch
    lcd = _lcd()
    w = wl.config5()
    flat, ro, ln, cap = wl.pack_rows(w.hists, extra=16)
    q, tgt = w.step_inputs(np.zeros(w.B, np.int64), 0)
    outs = []
    for bal in (0, 1):
        p = lcd.default_params(scan_balance=bal)
        dev = torch.device("cuda:0")
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        h_d, ln_d = t(flat), t(ln.copy())
        dr = lcd.LookupDrafter(w.B, int(ln.max()), dev, p)
        out = dr.step(h_d, t(ro), ln_d, t(cap), t(q), t(tgt))
        torch.cuda.synchronize()
        outs.append([out[k].cpu().numpy() for k in ("match_len", "match_end", "draft", "block",
                                                    "accept")] + [h_d.cpu().numpy(), ln_d.cpu().numpy()])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
    om, oe, od = oracle.lookup_propose(flat, ro, ln, _oparams(lcd.default_params()))
    np.testing.assert_array_equal(outs[1][0], om)
    np.testing.assert_array_equal(outs[1][1], oe)
