"""The fused decode step with appends, at launch shapes whose workgroups do not
all fit on the GPU at once, the merge's bounded wait when it gives up, and a
decode saved and resumed mid-way -- each checked against the CPU oracle.

The workgroups of one lookup_decode_step launch read the rows' lengths while
others have already finished (and appended to) their rows, so the step reads
`lens` and writes the new lengths to `lens_out`; these tests alternate the two
arrays as a decode loop does and hold every step's outputs to the oracle's
four-call step, with the workspace left clean after every call.
"""

import numpy as np
import pytest

import oracle
from context_lookup_drafting_amd import workloads as wl
from simulate import _extra, simulate_oracle
from test_gpu_parity import _oparams

pytestmark = pytest.mark.gpu

PAD = -1
REQ_WORDS = 8208 // 8          # LCD_WORKSPACE_PER_REQUEST in 8-byte words


def _ws_clean(ws, B):
    """Every arrival count, pad word and slot of the lookup workspace is zero
    (the upper half of each header word is the request's call epoch)."""
    w = ws.cpu().numpy()[: B * REQ_WORDS].reshape(B, REQ_WORDS)
    return bool((w[:, 0] & 0xFFFFFFFF == 0).all() and (w[:, 1:] == 0).all())


def _decode_alternating(w, steps, params, oracle_recs, check_ws=True):
    """`steps` decode steps of workload w through lookup_decode_step with
    append, lengths alternating between two arrays; every step's outputs are
    compared with the oracle's recorded step."""
    import torch
    import context_lookup_drafting_amd as lcd
    dev = torch.device("cuda:0")
    flat, ro, lens, cap = wl.pack_rows(w.hists, extra=_extra(steps))
    B = w.B
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h_d, ro_d, cap_d = t(flat), t(ro), t(cap)
    L = [t(lens.copy()), torch.empty(B, dtype=torch.int32, device=dev)]
    max_len = int(lens.max()) + _extra(steps)
    ws = lcd.alloc_decode_workspace(B, max_len, dev, params)
    state = torch.zeros((B, 3), dtype=torch.int32, device=dev)
    mk = lambda *s: torch.empty(s, dtype=torch.int32, device=dev)
    m, e, d, blk, bl, acc, lnx = mk(B), mk(B), mk(B, 15), mk(B, 15), mk(B), mk(B), mk(B)
    pos = np.zeros(B, np.int64)
    for k in range(steps):
        q, tgt = w.step_inputs(pos, k)
        lin, lout = L[k % 2], L[(k + 1) % 2]
        lcd.lookup_decode_step(h_d, ro_d, lin, cap_d, max_len, t(q), t(tgt), state, ws, m, e, d,
                               blk, bl, acc, lnx, True, params, lens_out=lout)
        rec = oracle_recs[k]
        got = dict(m=m, e=e, d=d, block=blk, blk=bl, acc=acc, state=state, long_next=lnx)
        for name, g in got.items():
            np.testing.assert_array_equal(g.cpu().numpy(), rec[name], err_msg=f"step {k}: {name}")
        acc_h = acc.cpu().numpy()
        if check_ws:
            assert _ws_clean(ws, B), f"step {k}: workspace not clean"
        pos = pos + np.maximum(acc_h, 0) + 1
    torch.cuda.synchronize()
    return h_d.cpu().numpy(), L[steps % 2].cpu().numpy()


@pytest.fixture(scope="module")
def c5_oracle_256():
    w = wl.config5()
    return w, simulate_oracle(w, 256)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("shape", [dict(scan_balance=1, scan_wgs=3000), dict(scan_wgs=4096)],
                         ids=["balanced-3000", "equal-4096"])
def test_c5_decode_with_appends_beyond_one_dispatch_round(gpu, c5_oracle_256, shape):
    """256 steps of config 5 (256 ragged rows of 1k-262k tokens) through the
    fused step with appends, at 3000 token-balanced and 4096 equal-chunk
    workgroups -- more than the GPU holds at once, so later workgroups start
    after earlier ones have appended to their rows."""
    import context_lookup_drafting_amd as lcd
    w, orc = c5_oracle_256
    p = lcd.default_params(**shape)
    flat, lens = _decode_alternating(w, 256, p, orc["recs"])
    np.testing.assert_array_equal(lens, orc["lens"])
    np.testing.assert_array_equal(flat, orc["flat"])


def _ragged_rows(seed=21, B=48):
    """Rows of 3k-40k tokens (several chunks at 4 workgroups per row) and of
    40-2k tokens (one chunk), shaped like config 3's texts."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cdf = wl.zipf_cdf(40_960)
    hs = []
    for r in range(B):
        n = int(rng.integers(3000, 40_000)) if r % 3 else int(rng.integers(40, 2000))
        h = wl.zipf_tokens(rng, n, cdf)
        if r % 2:
            k = min(500, n // 3)
            s0 = int(rng.integers(0, n - 2 * k))
            h[n - k:] = h[s0:s0 + k]                # ends restating an earlier window
        hs.append(h.astype(np.int32))
    return hs


def _participants(lcd, lens, B, max_len, p):
    wgs, T = lcd.launch_shape(B, max_len, p, None)
    cpr = wgs // B
    nc = np.maximum(lens.astype(np.int64) - 1, 0)
    return np.minimum(np.maximum((nc + T - 1) // T, 1), cpr)


def test_lookup_merge_give_up_is_reported(gpu):
    """With no poll allowed, every request scanned by several workgroups
    reports match_len = -1 (and an empty draft) instead of a result; rows of
    one chunk are answered as usual.  The next call on the same workspace is
    exact again and leaves it clean."""
    import torch
    import context_lookup_drafting_amd as lcd
    hs = _ragged_rows()
    flat, ro, lens, cap = wl.pack_rows(hs)
    B = len(hs)
    max_len = int(lens.max())
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h_d, ro_d, ln_d = t(flat), t(ro), t(lens)
    ws = lcd.alloc_workspace(B, dev)
    m = torch.empty(B, dtype=torch.int32, device=dev)
    e, d = torch.empty_like(m), torch.empty((B, 15), dtype=torch.int32, device=dev)
    om, oe, od = oracle.lookup_propose(flat, ro, lens)
    give_up = lcd.default_params(scan_wgs=4 * B, merge_polls=-1)
    merged = _participants(lcd, lens, B, max_len, give_up) > 1
    assert merged.any() and (~merged).any()
    lcd.lookup_propose(h_d, ro_d, ln_d, max_len, ws, m, e, d, give_up)
    torch.cuda.synchronize()
    mh, eh, dh = m.cpu().numpy(), e.cpu().numpy(), d.cpu().numpy()
    assert (mh[merged] == -1).all() and (eh[merged] == -1).all() and (dh[merged] == PAD).all()
    np.testing.assert_array_equal(mh[~merged], om[~merged])
    np.testing.assert_array_equal(eh[~merged], oe[~merged])
    np.testing.assert_array_equal(dh[~merged], od[~merged])
    hdr = ws.cpu().numpy()[: B * REQ_WORDS].reshape(B, REQ_WORDS)[:, 0]
    assert (hdr & 0xFFFFFFFF == 0).all()                      # counts reset
    assert ((hdr >> 32)[merged] == 1).all()                    # one epoch used
    for _ in range(3):                                         # late slots never taken
        lcd.lookup_propose(h_d, ro_d, ln_d, max_len, ws, m, e, d,
                           lcd.default_params(scan_wgs=4 * B))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(m.cpu().numpy(), om)
        np.testing.assert_array_equal(e.cpu().numpy(), oe)
        np.testing.assert_array_equal(d.cpu().numpy(), od)
        assert _ws_clean(ws, B)


def test_decode_step_merge_give_up_goes_on_without_the_lookup(gpu):
    """A request whose merge gave up is fused, accepted, appended and
    scheduled as one without a match: the block is the draft model's, and the
    rest equals the oracle's fuse / accept / schedule on those outputs."""
    import torch
    import context_lookup_drafting_amd as lcd
    hs = _ragged_rows(seed=22)
    B = len(hs)
    flat, ro, lens, cap = wl.pack_rows(hs, extra=16)
    rng = np.random.Generator(np.random.PCG64(23))
    q = rng.integers(0, 40_960, (B, 7)).astype(np.int32)
    tgt = rng.integers(0, 40_960, (B, 16)).astype(np.int32)
    tgt[:, :7] = np.where(rng.random((B, 7)) < 0.7, q, tgt[:, :7])
    long0 = (np.arange(B) % 2).astype(np.int32)
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h_d, ro_d, ln_d, cap_d = t(flat), t(ro), t(lens), t(cap)
    ln_out = torch.empty_like(ln_d)
    max_len = int(lens.max())
    p = lcd.default_params(scan_wgs=4 * B, merge_polls=-1)
    ws = lcd.alloc_decode_workspace(B, max_len, dev, p)
    state = torch.zeros((B, 3), dtype=torch.int32, device=dev)
    state[:, 0] = t(long0)
    mk = lambda *s: torch.empty(s, dtype=torch.int32, device=dev)
    m, e, d, blk, bl, acc, lnx = mk(B), mk(B), mk(B, 15), mk(B, 15), mk(B), mk(B), mk(B)
    lcd.lookup_decode_step(h_d, ro_d, ln_d, cap_d, max_len, t(q), t(tgt), state, ws, m, e, d, blk,
                           bl, acc, lnx, True, p, lens_out=ln_out)
    torch.cuda.synchronize()
    merged = _participants(lcd, lens, B, max_len, p) > 1
    mh, dh = m.cpu().numpy(), d.cpu().numpy()
    assert (mh[merged] == -1).all() and (dh[merged] == PAD).all()
    om, oe, od = oracle.lookup_propose(flat, ro, lens)
    np.testing.assert_array_equal(mh[~merged], om[~merged])
    op = _oparams(p)
    oblk, obl = oracle.fuse_verify_block(dh, mh, q, long0, op)
    o_flat, o_ln = flat.copy(), lens.copy()
    oacc = oracle.greedy_accept(oblk, obl, tgt, o_flat, ro, o_ln, cap)
    ost = np.zeros((B, 3), np.int32)
    ost[:, 0] = long0
    oln = oracle.lookup_schedule_step(ost, mh, oacc, obl, op)
    for name, g, o in [("block", blk, oblk), ("blk", bl, obl), ("acc", acc, oacc),
                       ("lens_out", ln_out, o_ln), ("hist", h_d, o_flat), ("state", state, ost),
                       ("long_next", lnx, oln)]:
        np.testing.assert_array_equal(g.cpu().numpy(), o, err_msg=name)
    # merged rows verified the draft model's head only
    assert (oblk[merged][:, :7] == q[merged]).all()


def test_rejection_give_up_is_reported(gpu):
    """rejection_accept with no poll allowed reports accept = -1 and emits
    nothing for every request (no append); the next calls on the same
    workspace equal the oracle."""
    import torch
    import context_lookup_drafting_amd as lcd
    sb = wl.sampled_batch(B=16, V=40_960)
    dev = torch.device("cuda:0")
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)
    args = (t(sb.block, np.int32), t(sb.block_len, np.int32), t(sb.target_probs, np.float32),
            t(sb.u_accept, np.float64), t(sb.u_sample.view(np.int64), np.int64))
    kw = dict(model_mask=t(sb.model_mask.view(np.int32), np.int32),
              model_probs=t(sb.model_probs, np.float32))
    ws = lcd.alloc_rejection_workspace(sb.B, sb.V, dev)
    acc = torch.empty(sb.B, dtype=torch.int32, device=dev)
    em = torch.empty((sb.B, 16), dtype=torch.int32, device=dev)
    hist = torch.zeros(sb.B * 32, dtype=torch.int32, device=dev)
    ro = t(np.arange(sb.B) * 32, np.int64)
    lens = t(np.full(sb.B, 3), np.int32)
    cap = t(np.full(sb.B, 32), np.int32)
    lcd.rejection_accept(*args, ws, acc, em, **kw, hist=hist, row_off=ro, lens=lens, cap=cap,
                         merge_polls=-1)
    torch.cuda.synchronize()
    assert (acc.cpu().numpy() == -1).all() and (em.cpu().numpy() == PAD).all()
    assert (hist.cpu().numpy() == 0).all() and (lens.cpu().numpy() == 3).all()
    oacc, oem = oracle.rejection_accept(sb.block, sb.block_len, sb.target_probs, sb.u_accept,
                                        sb.u_sample, sb.model_mask, sb.model_probs)
    for _ in range(3):
        lcd.rejection_accept(*args, ws, acc, em, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), oacc)
        np.testing.assert_array_equal(em.cpu().numpy(), oem)
        w = ws.cpu().numpy().reshape(sb.B, -1)
        assert (w[:, 0] & 0xFFFFFFFF == 0).all() and (w[:, 1:] == 0).all()


def test_decode_saved_and_resumed(gpu):
    """Config 3: 100 steps through one LookupDrafter, then its scheduler state
    and telemetry, the histories and the lengths are copied to the host and
    restored into a fresh drafter (fresh workspaces) on fresh device buffers;
    the continuation to step 256 equals the oracle's uninterrupted decode."""
    import torch
    import context_lookup_drafting_amd as lcd
    w = wl.config3()
    steps, cut = 256, 100
    orc = simulate_oracle(w, steps)
    flat, ro, lens, cap = wl.pack_rows(w.hists, extra=_extra(steps))
    B = w.B
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    max_len = int(lens.max()) + _extra(steps)
    h_d, ro_d, ln_d, cap_d = t(flat), t(ro), t(lens.copy()), t(cap)
    dr = lcd.LookupDrafter(B, max_len, dev, telemetry=True)
    pos = np.zeros(B, np.int64)

    def run(dr, h_d, ln_d, k):
        q, tgt = w.step_inputs(pos, k)
        out = dr.step(h_d, ro_d, ln_d, cap_d, t(q), t(tgt), append=True)
        rec = orc["recs"][k]
        for name in ("match_len", "match_end", "draft", "block", "block_len", "accept",
                     "long_next"):
            key = dict(match_len="m", match_end="e", draft="d", block="block", block_len="blk",
                       accept="acc", long_next="long_next")[name]
            np.testing.assert_array_equal(out[name].cpu().numpy(), rec[key],
                                          err_msg=f"step {k}: {name}")
        np.testing.assert_array_equal(dr.state.cpu().numpy(), rec["state"], err_msg=f"step {k}")
        return out["accept"].cpu().numpy()

    for k in range(cut):
        pos = pos + np.maximum(run(dr, h_d, ln_d, k), 0) + 1
    torch.cuda.synchronize()
    saved = dict(hist=h_d.cpu().numpy(), lens=ln_d.cpu().numpy(), state=dr.state.cpu().numpy(),
                 tele=dr.telemetry.cpu().numpy())
    del dr, h_d, ln_d
    dr2 = lcd.LookupDrafter(B, max_len, dev, telemetry=True)
    dr2.state.copy_(t(saved["state"]))
    dr2.telemetry.copy_(t(saved["tele"]))
    h2, ln2 = t(saved["hist"]), t(saved["lens"])
    for k in range(cut, steps):
        pos = pos + np.maximum(run(dr2, h2, ln2, k), 0) + 1
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ln2.cpu().numpy(), orc["lens"])
    np.testing.assert_array_equal(h2.cpu().numpy(), orc["flat"])
    np.testing.assert_array_equal(dr2.telemetry.cpu().numpy().view(np.uint32), orc["tele"])
