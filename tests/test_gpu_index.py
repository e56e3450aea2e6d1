"""GPU <-> oracle parity of the incremental n-gram index (lookup_index_*).

The index is another way to compute the lookup, so its reference is the
oracle's lookup itself: match length, match end and draft must equal it bit
for bit on every input -- full-size configurations, whole decode simulations
whose histories grow every step, exhaustive tiny vocabularies, the stress
batches, other suffix-length ranges, histories that grow by many tokens at
once, and the slow paths (fingerprint collisions forced by using 1-3
fingerprint bits, and histories that got shorter than the index).
"""

import numpy as np
import pytest

import oracle
from context_lookup_drafting_amd import workloads as wl
from test_gpu_parity import _compare_sims, _oparams, _stress_batch

pytestmark = pytest.mark.gpu


def index_lookup(flat, row_off, lens, params=None, fp_bits=0, cap=None, idx=None):
    """Builds an index over the rows (unless given one) and proposes once."""
    import torch
    import context_lookup_drafting_amd as lcd
    p = params or lcd.default_params()
    dev = torch.device("cuda:0")
    B = len(lens)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)
    h, ro, ln = t(flat, np.int32), t(row_off, np.int64), t(lens, np.int32)
    if idx is None:
        idx = lcd.LookupIndex(np.maximum(lens, 0) if cap is None else cap, dev, p, fp_bits=fp_bits)
        idx.build(h, ro, ln, int(max(lens.max(), 0)) if B else 0)
    m = torch.full((B,), 77, dtype=torch.int32, device=dev)
    e = torch.full((B,), 77, dtype=torch.int32, device=dev)
    d = torch.full((B, 15), 77, dtype=torch.int32, device=dev)
    idx.propose(h, ro, ln, m, e, d)
    torch.cuda.synchronize()
    return m.cpu().numpy(), e.cpu().numpy(), d.cpu().numpy(), idx


def assert_index_parity(flat, row_off, lens, params=None, fp_bits=0, cap=None):
    import context_lookup_drafting_amd as lcd
    p = params or lcd.default_params()
    m, e, d, idx = index_lookup(flat, row_off, lens, p, fp_bits, cap)
    om, oe, od = oracle.lookup_propose(flat, row_off, lens, _oparams(p))
    bad = np.nonzero((m != om) | (e != oe) | np.any(d != od, axis=1))[0]
    assert bad.size == 0, (f"{bad.size} requests differ; first r={bad[0]}: gpu m={m[bad[0]]} "
                           f"e={e[bad[0]]} oracle m={om[bad[0]]} e={oe[bad[0]]} n={lens[bad[0]]}")
    return m, e, d, idx


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_full_size_configs(gpu, k):
    w = wl.make_config(k)
    flat, ro, ln, cap = wl.pack_rows(w.hists)
    m, _, _, idx = assert_index_parity(flat, ro, ln, cap=cap)
    assert (idx.indexed_len.cpu().numpy() == ln).all()


@pytest.mark.parametrize("k", [2, 3])
def test_decode_simulation_through_the_index(gpu, k):
    """Whole decode loops (200 / 256 steps) with the lookup answered from the
    index, updated by every call as the histories grow: every step equals the
    oracle's simulation."""
    from simulate import simulate_gpu, simulate_oracle
    w = wl.make_config(k)
    steps = 200 if k == 2 else 256
    g = simulate_gpu(w, steps, index=True)
    o = simulate_oracle(w, steps)
    _compare_sims(g, o)
    # the index covers the history as of the last propose; the last step's
    # acceptance then appended its 1..16 tokens
    gap = g["lens"] - g["indexed_len"]
    assert ((gap >= 0) & (gap <= 16)).all()


def test_decode_simulation_with_collisions(gpu):
    """Two fingerprint bits: collisions at every turn, answered by the exact
    slow path; the decode is still the oracle's."""
    from simulate import simulate_gpu, simulate_oracle
    w = wl.config3()
    g = simulate_gpu(w, 48, index=True, fp_bits=2)
    o = simulate_oracle(w, 48)
    _compare_sims(g, o)


def test_exhaustive_tiny_vocab_batches(gpu):
    for alphabet, n_max in ((3, 10), (2, 14)):
        hs = []
        for n in range(0, n_max + 1):
            hs.extend(list(wl.all_strings(alphabet, n)))
        flat, ro, ln = wl.pack_csr(hs)
        assert_index_parity(flat, ro, ln)


@pytest.mark.parametrize("prm", [
    dict(), dict(l_min=1, l_max=1), dict(l_min=2, l_max=5, k_max=7), dict(l_min=3, l_max=16),
    dict(l_min=4, l_max=16, k_max=0), dict(l_min=12, l_max=12), dict(l_min=6, l_max=9, k_max=3),
])
def test_stress_params(gpu, prm):
    import context_lookup_drafting_amd as lcd
    flat, ro, ln = wl.pack_csr(_stress_batch())
    assert_index_parity(flat, ro, ln, lcd.default_params(**prm))


@pytest.mark.parametrize("fp_bits", [1, 2, 3])
def test_forced_fingerprint_collisions(gpu, fp_bits):
    import context_lookup_drafting_amd as lcd
    flat, ro, ln = wl.pack_csr(_stress_batch(seed=13, B=120))
    assert_index_parity(flat, ro, ln, fp_bits=fp_bits)
    assert_index_parity(flat, ro, ln, lcd.default_params(l_min=2, l_max=7), fp_bits=fp_bits)
    assert_index_parity(flat, ro, ln, lcd.default_params(index_load=2), fp_bits=fp_bits)


@pytest.mark.parametrize("k", [3, 5])
def test_densest_tables_full_size(gpu, k):
    """index_load = 2 (144 bytes per token of capacity): the full-size
    batches, with the tables half full at capacity."""
    import context_lookup_drafting_amd as lcd
    w = wl.make_config(k)
    flat, ro, ln, cap = wl.pack_rows(w.hists)
    assert_index_parity(flat, ro, ln, lcd.default_params(index_load=2), cap=ln.copy())


@pytest.mark.parametrize("prm", [dict(), dict(l_min=1, l_max=16), dict(index_load=2)])
def test_growth_by_many_tokens_and_shrinking(gpu, prm):
    """Histories grow by 0..3000 tokens between two proposes (the propose
    indexes all of them: many rounds of 64 positions, up to 1,024 queued
    entries each with 16 lengths); then some rows shrink below the index
    (answered by scans, rows marked stale), and grow again."""
    import torch
    import context_lookup_drafting_amd as lcd
    rng = np.random.Generator(np.random.PCG64(31))
    B = 64
    full = [rng.integers(0, int(rng.integers(2, 200)), int(rng.integers(0, 6000))).astype(np.int32)
            for _ in range(B)]
    for r in range(0, B, 5):                              # planted long repeats
        n = len(full[r])
        if n > 200:
            full[r][n - 40:] = full[r][50:90]
    flat, ro, ln_full, cap = wl.pack_rows(full)
    start = np.array([int(rng.integers(0, len(h) + 1)) for h in full], np.int32)
    p = lcd.default_params(**prm)
    dev = torch.device("cuda:0")
    idx = lcd.LookupIndex(cap, dev, p)
    h_d = torch.from_numpy(flat).to(dev)
    ro_d = torch.from_numpy(ro).to(dev)
    idx.build(h_d, ro_d, torch.from_numpy(start).to(dev), int(start.max()))

    def check(lens):
        m, e, d, _ = index_lookup(flat, ro, lens, p, idx=idx)
        om, oe, od = oracle.lookup_propose(flat, ro, lens, _oparams(p))
        np.testing.assert_array_equal(m, om)
        np.testing.assert_array_equal(e, oe)
        np.testing.assert_array_equal(d, od)

    check(start)
    mid = np.minimum(start + rng.integers(0, 3000, B), ln_full).astype(np.int32)
    check(mid)
    check(ln_full)
    assert (idx.indexed_len.cpu().numpy() == ln_full).all()
    shrunk = ln_full.copy()
    shrunk[::3] = shrunk[::3] // 2
    check(shrunk)
    il = idx.indexed_len.cpu().numpy()
    assert (il[::3][ln_full[::3] > shrunk[::3]] == -1).all()
    check(ln_full)                                        # stale rows keep answering by scans


def test_empty_negative_and_tiny_rows(gpu):
    hs = [np.zeros(0, np.int32), np.array([1], np.int32), np.array([1, 1], np.int32),
          np.array([2, 2, 2, 2], np.int32), np.array([2, 2, 2, 2, 2], np.int32),
          np.zeros(0, np.int32)] + [np.full(k, 3, np.int32) for k in range(0, 30)]
    flat, ro, ln = wl.pack_csr(hs)
    assert_index_parity(flat, ro, ln)
    ln2 = ln.copy()
    ln2[3] = -5
    m, e, d, _ = index_lookup(flat, ro, ln2)
    assert m[3] == 0 and e[3] == -1 and np.all(d[3] == -1)


def test_drafter_with_index_matches_the_oracle_decode(gpu):
    """LookupDrafter answering from the index (build once, propose every
    step): the whole 128-step decode and its telemetry equal the oracle's."""
    from context_lookup_drafting_amd.decode_sim import run_fused
    from simulate import simulate_oracle
    w = wl.config3()
    g = run_fused(w, 128, record=True, index=True)
    g.pop("tele_d")
    o = simulate_oracle(w, 128)
    _compare_sims(g, o)
