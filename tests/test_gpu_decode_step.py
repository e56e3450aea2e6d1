"""Parity of the fused lookup_decode_step entry point with the CPU oracle:
every row of the step (lookup, draft, fused block, accept, append, scheduler)
bit-exact, per step, over whole simulated decodes and single-step batches."""

import numpy as np
import pytest

import oracle
from context_lookup_drafting_amd import workloads as wl
from test_gpu_parity import _compare_sims, _oparams, _stress_batch

pytestmark = pytest.mark.gpu


def _fused_single_step(w_hists, q, tgt, long0, params=None, append=False, packed="rows",
                       max_len=None):
    import torch
    import context_lookup_drafting_amd as lcd
    p = params or lcd.default_params()
    if packed == "rows":
        flat, ro, ln, cap = wl.pack_rows(w_hists, extra=16)
    else:
        flat, ro, ln = wl.pack_csr(w_hists)
        cap = ln.copy()
    B = len(ln)
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h_d, ro_d, ln_d, cap_d = t(flat), t(ro), t(ln.copy()), t(cap)
    ln_out = torch.full((B,), -77, dtype=torch.int32, device=dev)
    ml = int(ln.max()) if max_len is None else max_len
    ws = lcd.alloc_decode_workspace(B, ml, dev, p)
    state = torch.zeros((B, 3), dtype=torch.int32, device=dev)
    state[:, 0] = t(long0)
    outs = [torch.full((B,), 77, dtype=torch.int32, device=dev) for _ in range(5)]
    d = torch.full((B, 15), 77, dtype=torch.int32, device=dev)
    blk = torch.full((B, 15), 77, dtype=torch.int32, device=dev)
    lcd.lookup_decode_step(h_d, ro_d, ln_d, cap_d, ml, t(q), t(tgt), state, ws, outs[0], outs[1], d,
                           blk, outs[2], outs[3], outs[4], append, p, lens_out=ln_out)
    torch.cuda.synchronize()
    got = dict(m=outs[0], e=outs[1], d=d, block=blk, blk=outs[2], acc=outs[3], ln=outs[4],
               state=state, lens=ln_out if append else ln_d, flat=h_d)
    got = {k: v.cpu().numpy() for k, v in got.items()}
    np.testing.assert_array_equal(ln_d.cpu().numpy(), ln)             # the lengths read stay
    if not append:
        assert (ln_out.cpu().numpy() == -77).all()                      # not touched

    op = _oparams(p)
    om, oe, od = oracle.lookup_propose(flat, ro, ln, op)
    oblk, obl = oracle.fuse_verify_block(od, om, q, long0, op)
    o_flat, o_ln = flat.copy(), ln.copy()
    if append:
        oacc = oracle.greedy_accept(oblk, obl, tgt, o_flat, ro, o_ln, cap)
    else:
        oacc = oracle.greedy_accept(oblk, obl, tgt)
    ost = np.zeros((B, 3), np.int32)
    ost[:, 0] = long0
    oln = oracle.lookup_schedule_step(ost, om, oacc, obl, op)
    exp = dict(m=om, e=oe, d=od, block=oblk, blk=obl, acc=oacc, ln=oln, state=ost, lens=o_ln,
               flat=o_flat)
    for k in exp:
        np.testing.assert_array_equal(got[k], exp[k], err_msg=k)


def test_fused_config1(gpu):
    w = wl.config1()
    for lg in (0, 1):
        _fused_single_step(w.hists, w.q0, w.target0, np.array([lg], np.int32), append=True)


@pytest.mark.parametrize("k", [4, 5])
def test_fused_single_step_configs(gpu, k):
    w = wl.make_config(k)
    for lg in (0, 1):
        _fused_single_step(w.hists, w.q0, w.target0, np.full(w.B, lg, np.int32))


def test_fused_ragged_csr_and_params(gpu):
    import context_lookup_drafting_amd as lcd
    rng = np.random.Generator(np.random.PCG64(31))
    hs = _stress_batch(seed=3, B=200)
    B = len(hs)
    q = rng.integers(0, 5, (B, 7)).astype(np.int32)
    tgt = rng.integers(0, 5, (B, 16)).astype(np.int32)
    lg = rng.integers(0, 2, B).astype(np.int32)
    for prm in (dict(), dict(l_min=2, l_max=7, k_max=9, n_head=5, n_block=11),
                dict(scan_wgs=4000), dict(l_min=1, l_max=16)):
        p = lcd.default_params(**prm)
        _fused_single_step(hs, q, tgt, lg, p, packed="csr")
        _fused_single_step(hs, q, tgt, lg, p, packed="csr", max_len=0)
        _fused_single_step(hs, q, tgt, lg, p, append=True)


def test_fused_simulation_config2(gpu):
    from simulate import simulate_gpu_fused, simulate_oracle
    w = wl.config2()
    _compare_sims(simulate_gpu_fused(w, 200), simulate_oracle(w, 200))


def test_fused_simulation_config3(gpu):
    from simulate import simulate_gpu_fused, simulate_oracle
    w = wl.config3()
    g = simulate_gpu_fused(w, 256)
    _compare_sims(g, simulate_oracle(w, 256))
    for r in range(w.B):
        em = g["emitted"][r]
        assert em == w.truths[r][:len(em)].tolist()
