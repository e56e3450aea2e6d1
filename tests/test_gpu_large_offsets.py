"""Rows stored past 2^31 tokens of the history buffer.

Row offsets are 64-bit (`row_off` is int64): a serving engine's token buffer
of several requests at long context passes 8 GiB.  These tests place rows
straddling and beyond token 2^31 of one 8.6 GB device buffer, next to a row
near its start, a one-token row and an empty row, and compare the scan's
lookup, the one-kernel decode step with append and the index's decode step
with append against the oracle run on the same rows packed compactly.
"""

import numpy as np
import pytest

import oracle
from context_lookup_drafting_amd import workloads as wl
from test_gpu_parity import _oparams

pytestmark = pytest.mark.gpu

G2 = 1 << 31


def _rows():
    w = wl.config4()
    hs = [w.hists[0], w.hists[1][-60_000:], w.hists[2][:25_000], w.hists[3][-3_000:],
          w.hists[4][:1], w.hists[5][:0]]
    # device offsets: straddling 2^31 (odd, so the first granule is partial),
    # past it, near the start, past it again, and the two degenerate rows
    off = np.array([G2 - 70_001, G2 + 123_457, 5, G2 + 200_000, G2 + 400_000, G2 + 400_032],
                   np.int64)
    return hs, off


@pytest.fixture(scope="module")
def big(gpu):
    import torch
    hs, off = _rows()
    flat, ro, ln, cap = wl.pack_rows(hs, extra=16)
    end = off + cap
    assert all(end[i] <= off[j] or end[j] <= off[i]
               for i in range(len(off)) for j in range(i + 1, len(off))), "rows overlap"
    h = torch.empty((int(end.max()) + 64,), dtype=torch.int32, device=gpu)
    assert h.numel() > G2
    yield h, flat, ro, ln, cap, off
    del h
    torch.cuda.empty_cache()


def _place(h, flat, ro, cap, off):
    """Fill the buffer with a token no row holds, then copy each row's whole
    capacity (its tokens and its zeroed room) to its device offset."""
    import torch
    h.fill_(-5)
    for r in range(len(off)):
        src = torch.from_numpy(np.ascontiguousarray(flat[ro[r]:ro[r] + cap[r]])).to(h.device)
        h[int(off[r]):int(off[r]) + int(cap[r])].copy_(src)


def _rows_back(h, cap, off):
    return [h[int(off[r]):int(off[r]) + int(cap[r])].cpu().numpy() for r in range(len(off))]


def _oracle_rows(o_flat, ro, cap):
    return [o_flat[ro[r]:ro[r] + cap[r]] for r in range(len(ro))]


def test_lookup_rows_past_2g(gpu, big):
    import torch
    import context_lookup_drafting_amd as lcd
    h, flat, ro, ln, cap, off = big
    _place(h, flat, ro, cap, off)
    B = len(ln)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    for p in (lcd.default_params(), lcd.default_params(scan_balance=1),
              lcd.default_params(scan_wgs=4096)):
        ws = lcd.alloc_workspace(B, gpu)
        m = torch.full((B,), 77, dtype=torch.int32, device=gpu)
        e = torch.full((B,), 77, dtype=torch.int32, device=gpu)
        d = torch.full((B, 15), 77, dtype=torch.int32, device=gpu)
        lcd.lookup_propose(h, t(off), t(ln), int(ln.max()), ws, m, e, d, p)
        torch.cuda.synchronize()
        om, oe, od = oracle.lookup_propose(flat, ro, ln, _oparams(p))
        np.testing.assert_array_equal(m.cpu().numpy(), om)
        np.testing.assert_array_equal(e.cpu().numpy(), oe)
        np.testing.assert_array_equal(d.cpu().numpy(), od)
    assert (om[[0, 1, 3]] > 0).all()          # the rows past 2^31 do find matches


def _expected_step(flat, ro, ln, cap, q, tgt, op):
    om, oe, od = oracle.lookup_propose(flat, ro, ln, op)
    B = len(ln)
    oblk, obl = oracle.fuse_verify_block(od, om, q, np.zeros(B, np.int32), op)
    o_flat, o_ln = flat.copy(), ln.copy()
    oacc = oracle.greedy_accept(oblk, obl, tgt, o_flat, ro, o_ln, cap)
    ost = np.zeros((B, 3), np.int32)
    oln = oracle.lookup_schedule_step(ost, om, oacc, obl, op)
    return dict(m=om, e=oe, d=od, block=oblk, blk=obl, acc=oacc, ln=oln, state=ost, lens=o_ln), \
        o_flat


def _step_inputs(flat, ro, ln, op):
    """Config 4's proposals and targets for the first rows, with the targets of
    rows 0, 1 and 3 set to the oracle's fused block (up to its length), so that
    those rows accept their whole block and append its length + 1 tokens."""
    B = len(ln)
    w = wl.config4()
    q, tgt = w.step_inputs(np.zeros(w.B, np.int64), 0)
    q, tgt = q[:B].copy(), tgt[:B].copy()
    om, oe, od = oracle.lookup_propose(flat, ro, ln, op)
    oblk, obl = oracle.fuse_verify_block(od, om, q, np.zeros(B, np.int32), op)
    for r in (0, 1, 3):
        tgt[r, :obl[r]] = oblk[r, :obl[r]]
    return q, tgt


def test_fused_step_append_rows_past_2g(gpu, big):
    import torch
    import context_lookup_drafting_amd as lcd
    h, flat, ro, ln, cap, off = big
    _place(h, flat, ro, cap, off)
    B = len(ln)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    p = lcd.default_params()
    q, tgt = _step_inputs(flat, ro, ln, _oparams(p))
    ml = int(ln.max())
    ws = lcd.alloc_decode_workspace(B, ml, gpu, p)
    state = torch.zeros((B, 3), dtype=torch.int32, device=gpu)
    outs = [torch.full((B,), 77, dtype=torch.int32, device=gpu) for _ in range(5)]
    d = torch.full((B, 15), 77, dtype=torch.int32, device=gpu)
    blk = torch.full((B, 15), 77, dtype=torch.int32, device=gpu)
    ln_out = torch.full((B,), -77, dtype=torch.int32, device=gpu)
    lcd.lookup_decode_step(h, t(off), t(ln), t(cap), ml, t(q), t(tgt), state, ws, outs[0], outs[1],
                           d, blk, outs[2], outs[3], outs[4], True, p, lens_out=ln_out)
    torch.cuda.synchronize()
    got = dict(m=outs[0], e=outs[1], d=d, block=blk, blk=outs[2], acc=outs[3], ln=outs[4],
               state=state, lens=ln_out)
    exp, o_flat = _expected_step(flat, ro, ln, cap, q, tgt, _oparams(p))
    assert exp["acc"][[0, 1, 3]].max() >= 4     # long appends past 2^31
    for k in exp:
        np.testing.assert_array_equal(got[k].cpu().numpy(), exp[k], err_msg=k)
    for r, (a, b) in enumerate(zip(_rows_back(h, cap, off), _oracle_rows(o_flat, ro, cap))):
        np.testing.assert_array_equal(a, b, err_msg=f"row {r} after the append")


def test_index_step_append_rows_past_2g(gpu, big):
    import torch
    import context_lookup_drafting_amd as lcd
    h, flat, ro, ln, cap, off = big
    _place(h, flat, ro, cap, off)
    B = len(ln)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    p = lcd.default_params()
    q, tgt = _step_inputs(flat, ro, ln, _oparams(p))
    off_d, ln_d = t(off), t(ln.copy())
    idx = lcd.LookupIndex(cap, gpu, p)
    idx.build(h, off_d, ln_d, int(ln.max()))
    state = torch.zeros((B, 3), dtype=torch.int32, device=gpu)
    outs = [torch.full((B,), 77, dtype=torch.int32, device=gpu) for _ in range(5)]
    d = torch.full((B, 15), 77, dtype=torch.int32, device=gpu)
    blk = torch.full((B, 15), 77, dtype=torch.int32, device=gpu)
    idx.decode_step(h, off_d, ln_d, t(cap), t(q), t(tgt), state, outs[0], outs[1], d, blk,
                    outs[2], outs[3], outs[4], True)
    torch.cuda.synchronize()
    got = dict(m=outs[0], e=outs[1], d=d, block=blk, blk=outs[2], acc=outs[3], ln=outs[4],
               state=state, lens=ln_d)
    exp, o_flat = _expected_step(flat, ro, ln, cap, q, tgt, _oparams(p))
    assert exp["acc"][[0, 1, 3]].max() >= 4     # long appends past 2^31
    for k in exp:
        np.testing.assert_array_equal(got[k].cpu().numpy(), exp[k], err_msg=k)
    for r, (a, b) in enumerate(zip(_rows_back(h, cap, off), _oracle_rows(o_flat, ro, cap))):
        np.testing.assert_array_equal(a, b, err_msg=f"row {r} after the append")
