"""GPU <-> oracle parity of sampled verification (rejection_accept), bit-exact.

The accepted count and every emitted token are integers, and both sides take
each decision in the same arithmetic (fp32 probabilities, fp64 acceptance
test, integer weights floor(w * 2^40) with an exact total), so the bar is
equality, element by element, on the same seeded inputs: the full-size
sampled batch (64 requests over a 248,320-entry vocabulary), ragged
vocabularies that end inside a 1024-float unit, every launch shape, the exact
enumeration grids whose law the oracle pins prove lossless, the draw's word
boundaries, the edge cases, special float values and the append.
"""

import numpy as np
import pytest

import oracle
from context_lookup_drafting_amd import workloads as wl
from test_oracle_sampling import boundary_batch, edge_batch, model_grid_batch, point_mass_grid_batch

pytestmark = pytest.mark.gpu


def rejection_ws_clean(ws, B):
    """Every arrival count, pad word and unit sum of a rejection_accept
    workspace for B requests is zero (each header word keeps the request's
    call epoch in its upper half)."""
    w = ws.cpu().numpy().reshape(B, -1)
    return bool((w[:, 0] & 0xFFFFFFFF == 0).all() and (w[:, 1:] == 0).all())


def gpu_rejection(blk, bl, tp, ua, us, mask=None, mp=None, wg_units=0, ws=None, hist=None,
                  row_off=None, lens=None, cap=None):
    import torch
    import context_lookup_drafting_amd as lcd
    dev = torch.device("cuda:0")
    B = len(bl)
    V = tp.shape[2]
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)
    own_ws = ws is None
    if own_ws:
        ws = lcd.alloc_rejection_workspace(B, V, dev)
    acc = torch.full((B,), 77, dtype=torch.int32, device=dev)
    em = torch.full((B, 16), 77, dtype=torch.int32, device=dev)
    kw = {}
    if hist is not None:
        kw = dict(hist=hist, row_off=t(row_off, np.int64), lens=lens, cap=t(cap, np.int32))
    lcd.rejection_accept(t(blk, np.int32), t(bl, np.int32), t(tp, np.float32), t(ua, np.float64),
                         t(np.asarray(us, np.uint64).view(np.int64), np.int64), ws, acc, em,
                         model_mask=None if mask is None else t(np.asarray(mask, np.uint32).view(np.int32), np.int32),
                         model_probs=None if mp is None else t(mp, np.float32), wg_units=wg_units, **kw)
    torch.cuda.synchronize()
    if own_ws:
        assert rejection_ws_clean(ws, B), "workspace not left clean"
    return acc.cpu().numpy(), em.cpu().numpy()


def assert_rejection_parity(blk, bl, tp, ua, us, mask=None, mp=None, wg_units=0, ws=None):
    acc, em = gpu_rejection(blk, bl, tp, ua, us, mask, mp, wg_units, ws)
    oacc, oem = oracle.rejection_accept(blk, bl, tp, ua, us, model_mask=mask, model_probs=mp)
    bad = np.nonzero((acc != oacc) | np.any(em != oem, axis=1))[0]
    assert bad.size == 0, (f"{bad.size} requests differ; first r={bad[0]}: gpu a={acc[bad[0]]} "
                           f"em={em[bad[0]].tolist()} oracle a={oacc[bad[0]]} "
                           f"em={oem[bad[0]].tolist()}")
    return acc, em


def test_full_size_sampled_batch(gpu):
    """64 requests over 248,320 ids, draft-model rows given; every request, in
    several launch shapes, twice on one workspace."""
    import context_lookup_drafting_amd as lcd
    sb = wl.sampled_batch()
    ws = lcd.alloc_rejection_workspace(sb.B, sb.V, gpu)
    args = (sb.block, sb.block_len, sb.target_probs, sb.u_accept, sb.u_sample, sb.model_mask,
            sb.model_probs)
    acc, _ = assert_rejection_parity(*args, ws=ws)
    for wg in (0, 1, 4, 8, 61, 243):          # 0: 32 units, 8 workgroups per request
        assert_rejection_parity(*args, wg_units=wg, ws=ws)
    assert rejection_ws_clean(ws, sb.B)
    # the batch exercises every kind of draw: point-mass and draft-model
    # residuals, and plain draws after fully accepted blocks
    assert (acc == sb.block_len).any() and (acc < sb.block_len).any()
    # without draft-model rows every slot is a point mass
    assert_rejection_parity(sb.block, sb.block_len, sb.target_probs, sb.u_accept, sb.u_sample,
                            sb.model_mask, None)


@pytest.mark.parametrize("V", [4, 8, 1020, 1024, 1028, 4100, 40_960])
def test_vocabulary_sizes_and_launch_shapes(gpu, V):
    for B, with_model, seed in ((1, True, 1), (5, False, 2), (64, True, 3)):
        sb = wl.sampled_batch(seed=seed, B=B, V=V, with_model=with_model)
        for wg in (0, 1, 3):
            assert_rejection_parity(sb.block, sb.block_len, sb.target_probs, sb.u_accept,
                                    sb.u_sample, sb.model_mask, sb.model_probs, wg_units=wg)


@pytest.mark.parametrize("units", [260, 600, 4096])
def test_large_vocabularies(gpu, units):
    """Past 256 units each lane of the gathering loads its unit sums in batches
    of 8: 260 units (5 a lane, one partial batch), 600 (10 a lane, a full and a
    partial batch) and V = 2^22, 4096 units, the most a request's gathering
    handles (64 a lane)."""
    import context_lookup_drafting_amd as lcd
    V = units * 1024
    assert V <= lcd.SAMPLE_MAX_VOCAB
    sb = wl.sampled_batch(seed=4, B=2, V=V)
    assert_rejection_parity(sb.block, sb.block_len, sb.target_probs, sb.u_accept, sb.u_sample,
                            sb.model_mask, sb.model_probs)


def test_exact_enumeration_grids(gpu):
    """The grids whose law the oracle pins prove equal to the target's: the
    GPU emits exactly the oracle's tokens on every grid point."""
    (blk, bl, tp, ua, us), _ = point_mass_grid_batch()
    assert_rejection_parity(blk, bl, tp, ua, us)
    (blk, bl, tp, ua, us, mask, mp), _ = model_grid_batch()
    assert_rejection_parity(blk, bl, tp, ua, us, mask, mp)


def test_draw_word_boundaries(gpu):
    (blk, bl, tp, ua, us), want = boundary_batch(V=37, pad_to=40)
    acc, em = assert_rejection_parity(blk, bl, tp, ua, us)
    assert em[:, 0].tolist() == want


def test_edge_cases(gpu):
    blk, bl, tp, ua, us, mask, mp = edge_batch()
    acc, _ = assert_rejection_parity(blk, bl, tp, ua, us, mask, mp)
    assert (acc == -1).any()


def test_special_values_and_fallbacks(gpu):
    """Subnormal, NaN, infinite, negative and > 1 probabilities; uniforms of
    exactly 0 and >= 1; residuals with no mass (both kinds); mask bits past
    the head; a mask without draft-model rows."""
    rng = np.random.Generator(np.random.PCG64(21))
    B, V = 256, 12
    blk = rng.integers(-2, V + 2, (B, 15)).astype(np.int32)
    bl = rng.integers(-1, 17, B).astype(np.int32)
    tp = rng.dirichlet(np.full(V, 0.5), (B, 16)).astype(np.float32)
    specials = np.array([0.0, 1e-45, 1e-39, 2.0 ** -40, 2.0 ** -41, 1.0, 1.5, -0.25, np.inf,
                         -np.inf, np.nan], np.float32)
    hit = rng.random((B, 16, V)) < 0.15
    tp[hit] = rng.choice(specials, int(hit.sum()))
    mp = rng.dirichlet(np.full(V, 0.5), (B, 7)).astype(np.float32)
    hitq = rng.random((B, 7, V)) < 0.15
    mp[hitq] = rng.choice(specials, int(hitq.sum()))
    # requests 0..31: the target gives the token no mass (even r) or a
    # subnormal one (odd r: accepted only at u = 0, which these have), and 1/4
    # to the next token; draft-model rows of 1/2 everywhere leave a draft-model
    # residual with no mass, which falls back to the target row
    for r in range(32):
        x = int(rng.integers(0, V))
        blk[r, 0] = x
        bl[r] = 1
        tp[r, 0] = 0.0
        tp[r, 0, (x + 1) % V] = 0.25
        if r % 2:
            tp[r, 0, x] = 1e-42
        mp[r, 0] = 0.5
    ua = rng.random((B, 15))
    ua[rng.random((B, 15)) < 0.1] = 0.0
    ua[rng.random((B, 15)) < 0.05] = 1.0
    ua[:32, 0] = 0.0
    us = rng.integers(0, 2 ** 64, B, dtype=np.uint64)
    mask = rng.integers(0, 1 << 15, B).astype(np.uint32)
    assert_rejection_parity(blk, bl, tp, ua, us, mask, mp)
    assert_rejection_parity(blk, bl, tp, ua, us, mask, None)
    assert_rejection_parity(blk, bl, tp, ua, us, None, None)


def test_append_parity(gpu):
    import torch
    rng = np.random.Generator(np.random.PCG64(23))
    sb = wl.sampled_batch(seed=9, B=200, V=1024)
    cap = rng.integers(1, 24, sb.B).astype(np.int32)
    lens = np.minimum(rng.integers(-3, 24, sb.B), cap).astype(np.int32)
    row_off = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    hist0 = rng.integers(0, 9, int(cap.sum())).astype(np.int32)
    args = (sb.block, sb.block_len, sb.target_probs, sb.u_accept, sb.u_sample, sb.model_mask,
            sb.model_probs)
    h_d = torch.from_numpy(hist0.copy()).cuda()
    ln_d = torch.from_numpy(lens.copy()).cuda()
    acc, em = gpu_rejection(*args, hist=h_d, row_off=row_off, lens=ln_d, cap=cap)
    oh, ol = hist0.copy(), lens.copy()
    oacc, oem = oracle.rejection_accept(*args[:5], model_mask=args[5], model_probs=args[6],
                                        hist=oh, row_off=row_off, lens=ol, cap=cap)
    np.testing.assert_array_equal(acc, oacc)
    np.testing.assert_array_equal(em, oem)
    np.testing.assert_array_equal(h_d.cpu().numpy(), oh)
    np.testing.assert_array_equal(ln_d.cpu().numpy(), ol)
    assert (acc == -1).any() and (acc >= 0).any()
