"""Pins of the oracle's sampled verification (point-mass lookup proposals).

The method's claim (HyperQwen lookup-drafting article, closing paragraph on
losslessness) is that verifying lookup slots as point-mass proposals leaves
the output distribution equal to the target's.  These pins hold the oracle to
that claim exactly, not statistically: every probability below is dyadic and
every residual mass a power of two, so each accept decision and each integer
draw changes value only on a known grid, and enumerating the grid's
midpoints gives the exact law of the emitted tokens as fractions.  That law
must equal sampling from the target rows one token at a time.  Further pins:
the greedy special case (one-hot target rows reduce to greedy_accept), the
draw's exact boundaries against big-integer arithmetic, the draw's empirical
counts on evenly spaced words, and every edge case the definition names.
"""

import itertools
from fractions import Fraction as F

import numpy as np
import pytest

import oracle
from test_oracle_pins import _fusion_rows

PAD = -1


def _mk(B, V):
    return (np.full((B, 15), PAD, np.int32), np.zeros(B, np.int32),
            np.zeros((B, 16, V), np.float32), np.zeros((B, 15), np.float64),
            np.zeros(B, np.uint64))


def _grid_u(m):
    """Midpoints of the 2^m equal cells of [0, 1): each stands for mass 2^-m."""
    return [(k + 0.5) / 2 ** m for k in range(2 ** m)]


def _grid_words(g):
    """64-bit words at the midpoints of 2^g equal cells of [0, 2^64)."""
    return [((2 * k + 1) << (63 - g)) for k in range(2 ** g)]


def _law(acc, em, weights):
    """Exact law of the emitted sequence: {tuple(tokens): Fraction}."""
    law = {}
    for a, row, w in zip(acc, em, weights):
        assert a >= 0
        key = tuple(int(t) for t in row[:a + 1])
        assert (row[a + 1:] == PAD).all()
        law[key] = law.get(key, F(0)) + w
    return law


def _target_law(rows, drafts):
    """The law of sampling token by token from the target rows, written as
    the verified-block outcome: row i is only defined after the drafts
    d_0..d_{i-1} (the block's prefix), so a sequence leaves the draft path at
    its first token that differs from the draft, or at the bonus row."""
    law = {}
    prefix_p = F(1)
    for i, row in enumerate(rows):
        for z, pz in enumerate(row):
            if pz == 0:
                continue
            if i < len(drafts) and z == drafts[i]:
                continue                  # stays on the draft path: counted below
            law[tuple(drafts[:i]) + (z,)] = prefix_p * pz
        if i < len(drafts):
            prefix_p *= row[drafts[i]]
    return {k: v for k, v in law.items() if v != 0}


POINT_ROWS = [[F(1, 8), F(1, 2), F(1, 4), F(1, 8)],   # draft 1: accept 1/2, residual mass 1/2
              [F(1, 8), F(1, 8), F(3, 4), F(0)],      # draft 2: accept 3/4, residual mass 1/4
              [F(3, 8), F(1, 8), F(1, 4), F(1, 4)]]   # bonus row
POINT_DRAFTS = [1, 2]


def point_mass_grid_batch():
    """Two lookup slots and the bonus row over V = 4, one request per grid
    point (accept uniforms of both slots x draw word).  Returns the inputs and
    each request's weight (the grid cell's mass)."""
    V = 4
    us, ws = _grid_u(3), _grid_words(4)
    combos = list(itertools.product(range(len(us)), range(len(us)), range(len(ws))))
    B = len(combos)
    blk, bl, tp, ua, usm = _mk(B, V)
    blk[:, 0], blk[:, 1] = POINT_DRAFTS
    bl[:] = 2
    for i, row in enumerate(POINT_ROWS):
        tp[:, i, :] = np.array([float(x) for x in row], np.float32)
    for b, (i0, i1, k) in enumerate(combos):
        ua[b, 0], ua[b, 1], usm[b] = us[i0], us[i1], ws[k]
    return (blk, bl, tp, ua, usm), [F(1, len(us) ** 2 * len(ws))] * B


def test_point_mass_verification_is_lossless_exactly():
    """Two lookup slots plus the bonus row; every accept uniform and every draw
    word on its grid; the emitted sequence's law equals the target's."""
    (blk, bl, tp, ua, usm), weights = point_mass_grid_batch()
    B = len(bl)
    acc, em = oracle.rejection_accept(blk, bl, tp, ua, usm)
    assert _law(acc, em, weights) == _target_law(POINT_ROWS, POINT_DRAFTS)
    # the accept counts' law: a = 0, 1, 2 with 1/2, 1/2 * 1/4, 1/2 * 3/4
    cnt = np.bincount(acc, minlength=3) / B
    assert cnt.tolist() == [0.5, 0.125, 0.375]


MODEL_Q0 = [F(1, 4), F(1, 2), F(1, 4), F(0)]          # powers of two: u*Q is exact
MODEL_ROWS = [[F(1, 2), F(1, 4), F(1, 4), F(0)],      # residual max(p-q,0) = [1/4,0,0,0]
              [F(1, 4), F(1, 4), F(1, 2), F(0)],      # lookup draft 2: accept 1/2
              [F(1, 8), F(1, 8), F(1, 4), F(1, 2)]]


def model_grid_batch():
    """Slot 0 holds the draft model's token x (enumerated with weight q(x)),
    slot 1 the lookup token 2, over V = 4; one request per grid point."""
    V = 4
    q0, rows = MODEL_Q0, MODEL_ROWS
    us, ws = _grid_u(3), _grid_words(4)
    xs = [x for x in range(V) if q0[x] > 0]
    combos = list(itertools.product(xs, range(len(us)), range(len(us)), range(len(ws))))
    B = len(combos)
    blk, bl, tp, ua, usm = _mk(B, V)
    bl[:] = 2
    blk[:, 1] = 2
    mp = np.zeros((B, 7, V), np.float32)
    mp[:, 0, :] = np.array([float(x) for x in q0], np.float32)
    for i, row in enumerate(rows):
        tp[:, i, :] = np.array([float(x) for x in row], np.float32)
    weights = []
    for b, (x, i0, i1, k) in enumerate(combos):
        blk[b, 0] = x
        ua[b, 0], ua[b, 1], usm[b] = us[i0], us[i1], ws[k]
        weights.append(q0[x] / (len(us) ** 2 * len(ws)))
    mask = np.ones(B, np.uint32)
    return (blk, bl, tp, ua, usm, mask, mp), weights


def test_model_slot_verification_is_lossless_exactly():
    """Slot 0 carries the draft model's own proposal x ~ q (so the
    enumeration also runs over x with weight q(x)); slot 1 is a lookup slot.
    The law of the emitted tokens is still the target's."""
    (blk, bl, tp, ua, usm, mask, mp), weights = model_grid_batch()
    q0, rows = MODEL_Q0, MODEL_ROWS
    xs = [x for x in range(4) if q0[x] > 0]
    acc, em = oracle.rejection_accept(blk, bl, tp, ua, usm, model_mask=mask, model_probs=mp)
    law = _law(acc, em, weights)
    # the first emitted token is distributed as the target's row 0
    first = {}
    for seq, pr in law.items():
        first[seq[0]] = first.get(seq[0], F(0)) + pr
    assert first == {z: pz for z, pz in enumerate(rows[0]) if pz}
    # once slot 0 is accepted (whatever x was), the rest follows rows 1 and 2
    # along the lookup draft of slot 1
    for x in xs:
        accepted_x = {s: pr for s, pr in law.items() if len(s) >= 2 and s[0] == x}
        tot = sum(accepted_x.values())
        assert tot == q0[x] * min(F(1), rows[0][x] / q0[x])
        cond = {s[1:]: pr / tot for s, pr in accepted_x.items()}
        assert cond == _target_law(rows[1:], [2])


def test_model_slots_with_point_mass_rows_equal_lookup_slots():
    """A draft-model row that is the point mass on its own token makes the
    slot a point-mass slot: identical outputs for any uniforms."""
    rng = np.random.Generator(np.random.PCG64(3))
    B, V = 400, 9
    blk, bl, tp, ua, usm = _mk(B, V)
    tp[:] = rng.dirichlet(np.ones(V), (B, 16)).astype(np.float32)
    blk[:, :7] = rng.integers(0, V, (B, 7))
    bl[:] = 7
    ua[:] = rng.random((B, 15))
    usm[:] = rng.integers(0, 2 ** 64, B, dtype=np.uint64)
    mp = np.zeros((B, 7, V), np.float32)
    mp[np.arange(B)[:, None], np.arange(7)[None, :], blk[:, :7]] = 1.0
    mask = rng.integers(0, 128, B).astype(np.uint32)
    a1, e1 = oracle.rejection_accept(blk, bl, tp, ua, usm)
    a2, e2 = oracle.rejection_accept(blk, bl, tp, ua, usm, model_mask=mask, model_probs=mp)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(e1, e2)


@pytest.mark.parametrize("with_model", [False, True])
def test_one_hot_target_rows_reduce_to_greedy_accept(with_model):
    """Temperature zero: target rows one-hot at the argmax tokens make the
    sampled verifier the greedy one, for any uniforms and any draft-model rows."""
    rng = np.random.Generator(np.random.PCG64(7 + with_model))
    B, V = 2000, 6
    blk, bl, tp, ua, usm = _mk(B, V)
    tgt = rng.integers(0, V, (B, 16)).astype(np.int32)
    # drafts agree with the target for a random prefix, then anything (incl. PAD)
    agree = rng.integers(0, 16, B)
    cand = rng.integers(-1, V, (B, 15))
    for r in range(B):
        blk[r] = np.where(np.arange(15) < agree[r], tgt[r, :15], cand[r])
    bl[:] = rng.choice([0, 3, 7, 15], B)
    blk[np.arange(15)[None, :] >= bl[:, None]] = PAD
    tp[np.arange(B)[:, None], np.arange(16)[None, :], tgt] = 1.0
    ua[:] = rng.random((B, 15))
    usm[:] = rng.integers(0, 2 ** 64, B, dtype=np.uint64)
    kw = {}
    if with_model:
        mp = rng.dirichlet(np.ones(V), (B, 7)).astype(np.float32)
        kw = dict(model_mask=rng.integers(0, 128, B).astype(np.uint32), model_probs=mp)
    acc, em = oracle.rejection_accept(blk, bl, tp, ua, usm, **kw)
    gacc = oracle.greedy_accept(blk, bl, tgt)
    np.testing.assert_array_equal(acc, gacc)
    for r in range(B):
        assert em[r, :acc[r] + 1].tolist() == tgt[r, :acc[r] + 1].tolist()


def boundary_batch(V=37, pad_to=None):
    """Bonus draws at both ends of every token's range of words (computed with
    Python integers); the row may be padded with zero-probability entries."""
    rng = np.random.Generator(np.random.PCG64(11))
    p = rng.dirichlet(np.full(V, 0.3)).astype(np.float32)
    p[5] = 0.0
    if pad_to is not None:
        p = np.concatenate([p, np.zeros(pad_to - V, np.float32)])
        V = pad_to
    W = [int(np.floor(float(x) * 2 ** 40)) for x in p]   # float32 -> exact double
    C = np.cumsum([0] + W).tolist()
    S = C[-1]
    words, want = [], []
    for j in range(V):
        lo = -(-C[j] * 2 ** 64 // S)
        hi = -(-C[j + 1] * 2 ** 64 // S)
        if hi > lo:                                      # token j has words of its own
            for u in (lo, hi - 1):
                words.append(u)
                want.append(j)
    B = len(words)
    blk, bl, tp, ua, usm = _mk(B, V)
    tp[:, 0, :] = p
    usm[:] = np.array(words, np.uint64)
    return (blk, bl, tp, ua, usm), want


def test_draw_boundaries_match_big_integer_arithmetic():
    """The bonus draw picks token j exactly for the words u with
    ceil(C_{j-1} 2^64 / S) <= u < ceil(C_j 2^64 / S), where C_j is the running
    total of the weights floor(p * 2^40) and S their sum (Python integers)."""
    (blk, bl, tp, ua, usm), want = boundary_batch()
    acc, em = oracle.rejection_accept(blk, bl, tp, ua, usm)
    assert (acc == 0).all()
    assert em[:, 0].tolist() == want
    assert 5 not in want


def test_draw_counts_on_evenly_spaced_words():
    """Evenly spaced draw words over [0, 2^64): each token's count is within 1
    of count * W_j / S.  Three groups of requests draw from three different
    rows, reached three ways (nothing proposed at slot 0; a PAD slot after
    accepted ones; the bonus row of a fully accepted block), so a row, stride
    or offset mistake fails."""
    rng = np.random.Generator(np.random.PCG64(13))
    V, n = 101, 1 << 12
    rows = rng.dirichlet(np.full(V, 0.3), 3).astype(np.float32)
    B = 3 * n
    blk, bl, tp, ua, usm = _mk(B, V)
    g = [slice(k * n, (k + 1) * n) for k in range(3)]
    tp[:] = rows[(np.arange(B) // n + 1) % 3][:, None, :]     # decoy rows everywhere
    bl[g[0]] = 15                                   # slot 0 PAD: draws from row 0
    tp[g[0], 0] = rows[0]
    blk[g[1], :2] = [3, 4]                          # two certain slots, then PAD
    bl[g[1]] = 7
    tp[g[1], 0] = 0.0
    tp[g[1], 0, 3] = 1.0
    tp[g[1], 1] = 0.0
    tp[g[1], 1, 4] = 1.0
    tp[g[1], 2] = rows[1]
    blk[g[2], :3] = [5, 6, 7]                       # a 3-slot block fully accepted
    bl[g[2]] = 3
    for i, x in enumerate((5, 6, 7)):
        tp[g[2], i] = 0.0
        tp[g[2], i, x] = 1.0
    tp[g[2], 3] = rows[2]
    usm[:] = np.tile(np.arange(n, dtype=np.uint64) << np.uint64(64 - 12), 3)
    acc, em = oracle.rejection_accept(blk, bl, tp, ua, usm)
    for k, a in enumerate((0, 2, 3)):
        assert (acc[g[k]] == a).all()
        W = np.floor(rows[k].astype(np.float64) * 2 ** 40)
        got = np.bincount(em[g[k], a], minlength=V)
        assert np.abs(got - n * W / W.sum()).max() <= 1.0


def edge_batch():
    """One request per edge case the definition names (V = 4)."""
    V = 4
    B = 9
    blk, bl, tp, ua, usm = _mk(B, V)
    tp[:] = 0.25
    usm[:] = np.uint64(3) << np.uint64(62)            # t = 3/4 of S: token 3 of a uniform row
    # 0: L = 0 -> bonus from row 0
    # 1: every slot certain -> all 15 accepted, bonus from row 15
    blk[1] = 2
    bl[1] = 15
    tp[1, :15, :] = 0.0
    tp[1, :15, 2] = 1.0
    tp[1, 15] = [0.0, 0.0, 0.0, 1.0]
    # 2: PAD at slot 3 of a 7-slot block -> a = 3, token drawn from row 3 in full
    blk[2, :3] = 1
    tp[2, :3, :] = [0, 1, 0, 0]
    bl[2] = 7
    tp[2, 3] = [0.0, 1.0, 0.0, 0.0]
    # 3: token >= V at slot 0 -> same as PAD
    blk[3, 0] = 7
    bl[3] = 7
    # 4: block_len > 15 clamps; negative reads as 0
    blk[4] = 2
    bl[4] = 99
    tp[4, :, :] = [0, 0, 1, 0]
    # 5: all-zero row -> accept -1, nothing emitted (its block holds tokens that
    # request 4 would accept if it read past its own 15 slots)
    tp[5] = 0.0
    blk[5] = 2
    # 6: rejected slot whose residual is zero falls back to the target row
    blk[6, 0] = 0
    bl[6] = 1
    tp[6, 0] = [0.0, 0.25, 0.25, 0.0]                 # P = 0: always rejected
    # 7: clamps: p > 1 reads 1, negatives and NaN read 0
    blk[7, 0] = 1
    bl[7] = 1
    tp[7, 0] = [np.nan, 7.0, -1.0, 0.0]               # slot 0 accepted (P = 1)
    tp[7, 1] = [np.nan, -2.0, 0.5, np.inf]            # inf clamps to 1 -> weights 0,0,1/2,1
    # 8: negative block length
    bl[8] = -4
    blk[8, 0] = 1
    mp = np.zeros((B, 7, V), np.float32)
    mp[6, 0] = [0.5, 0.25, 0.25, 0.0]
    mask = np.zeros(B, np.uint32)
    mask[6] = 1
    return blk, bl, tp, ua, usm, mask, mp


def test_edge_cases():
    blk, bl, tp, ua, usm, mask, mp = edge_batch()
    B = len(bl)
    acc, em = oracle.rejection_accept(blk, bl, tp, ua, usm, model_mask=mask, model_probs=mp)
    assert acc[0] == 0 and em[0, 0] == 3
    assert acc[1] == 15 and em[1, :15].tolist() == [2] * 15 and em[1, 15] == 3
    assert acc[2] == 3 and em[2, :4].tolist() == [1, 1, 1, 1]
    assert acc[3] == 0 and em[3, 0] == 3
    assert acc[4] == 15 and em[4].tolist() == [2] * 16
    assert acc[5] == -1 and (em[5] == PAD).all()
    assert acc[6] == 0 and em[6, 0] == 2              # t = 3/4 of [0,1/4,1/4,0]: token 2
    assert acc[7] == 1 and em[7, :2].tolist() == [1, 3]
    assert acc[8] == 0 and em[8, 0] == 3
    for r in range(B):
        if acc[r] >= 0:
            assert (em[r, acc[r] + 1:] == PAD).all()


def test_append_matches_emitted_and_respects_capacity():
    rng = np.random.Generator(np.random.PCG64(17))
    B, V = 64, 11
    blk, bl, tp, ua, usm = _mk(B, V)
    tp[:] = rng.dirichlet(np.full(V, 0.2), (B, 16)).astype(np.float32)
    blk[:] = np.argmax(tp[:, :15], axis=2)            # drafts are each row's mode
    bl[:] = 15
    ua[:] = rng.random((B, 15))
    usm[:] = rng.integers(0, 2 ** 64, B, dtype=np.uint64)
    cap = rng.integers(3, 12, B).astype(np.int32)
    lens = np.minimum(rng.integers(-3, 12, B), cap).astype(np.int32)
    row_off = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    hist = np.full(int(cap.sum()), -7, np.int32)
    lens0 = lens.copy()
    acc0, em0 = oracle.rejection_accept(blk, bl, tp, ua, usm)
    acc, em = oracle.rejection_accept(blk, bl, tp, ua, usm, hist=hist, row_off=row_off,
                                      lens=lens, cap=cap)
    for r in range(B):
        have = max(int(lens0[r]), 0)
        row = hist[row_off[r]:row_off[r] + cap[r]]
        if have + acc0[r] + 1 > cap[r]:
            assert acc[r] == -1 and lens[r] == lens0[r] and (row == -7).all()
        else:
            assert acc[r] == acc0[r] and lens[r] == have + acc0[r] + 1
            assert row[have:lens[r]].tolist() == em0[r, :acc0[r] + 1].tolist()
            assert (row[lens[r]:] == -7).all()
    assert (acc == -1).any() and (acc >= 0).any()


def test_fusion_model_mask_follows_the_truth_table():
    """Bit i of the fusion's model mask is set exactly for the head slots the
    golden fusion table sources from the draft model (q)."""
    p = oracle.default_params()
    for m, lg, heads, tail, blk_exp in _fusion_rows():
        for ai, (a0, a1) in enumerate([(0, 0), (0, 1), (1, 0), (1, 1)]):
            d = np.arange(100, 115, dtype=np.int32)
            q = np.arange(200, 207, dtype=np.int32)
            if a0:
                q[0] = d[0]
            if a1:
                q[1] = d[1]
            _, _, mask = oracle.fuse_verify_block(d[None], np.array([m]), q[None],
                                                  np.array([lg]), p, with_mask=True)
            assert mask[0] == (0x7F if heads[ai] == "q" else 0)
    # a lookup draft shorter than the head: the slots past k_max keep q
    d = np.array(list(range(100, 105)) + [PAD] * 10, np.int32)
    _, _, mask = oracle.fuse_verify_block(d[None], np.array([12]),
                                          np.arange(200, 207, dtype=np.int32)[None],
                                          np.array([1]), oracle.default_params(k_max=5),
                                          with_mask=True)
    assert mask[0] == 0b1100000
