"""lookup_decode_step_noalloc -- the decode step whose workspace is the
library's static per-GPU array -- gives exactly what lookup_decode_step gives
with a caller-owned workspace: two calls in a row, the second on a smaller
batch (so it runs on what the first left in the array)."""

import numpy as np
import pytest

from context_lookup_drafting_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _step(noalloc, hists, q, tgt, long0, params):
    import torch
    import context_lookup_drafting_amd as lcd
    dev = torch.device("cuda:0")
    flat, ro, lens, cap = wl.pack_rows(hists, extra=16)
    B = len(hists)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h_d, ro_d, ln_d, cap_d = t(flat), t(ro), t(lens), t(cap)
    ln_out = torch.full((B,), -5, dtype=torch.int32, device=dev)
    state = torch.zeros((B, 3), dtype=torch.int32, device=dev)
    state[:, 0] = t(long0)
    mk = lambda *s: torch.full(s, 77, dtype=torch.int32, device=dev)
    m, e, d, blk, bl, acc, lnx = mk(B), mk(B), mk(B, 15), mk(B, 15), mk(B), mk(B), mk(B)
    tele = lcd.alloc_telemetry(B, dev)
    max_len = int(lens.max())
    if noalloc:
        lcd.lookup_decode_step_noalloc(h_d, ro_d, ln_d, cap_d, max_len, t(q), t(tgt), state, m, e,
                                       d, blk, bl, acc, lnx, True, params, telemetry=tele,
                                       lens_out=ln_out)
    else:
        ws = lcd.alloc_decode_workspace(B, max_len, dev, params)
        lcd.lookup_decode_step(h_d, ro_d, ln_d, cap_d, max_len, t(q), t(tgt), state, ws, m, e, d,
                               blk, bl, acc, lnx, True, params, telemetry=tele, lens_out=ln_out)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in dict(m=m, e=e, d=d, blk=blk, bl=bl, acc=acc, lnx=lnx,
                                                 lens_out=ln_out, hist=h_d, state=state,
                                                 tele=tele).items()}


def test_noalloc_step_equals_the_workspace_step(gpu):
    import context_lookup_drafting_amd as lcd
    w3 = wl.config3(steps=1)
    q3, t3 = w3.step_inputs(np.zeros(w3.B, np.int64), 0)
    long3 = (np.arange(w3.B) % 2).astype(np.int32)
    w1 = wl.config1()
    small = wl.prefix_batch(w1.hists[0])[::101]
    B1 = len(small)
    q1 = np.tile(w1.q0, (B1, 1)).astype(np.int32)
    t1 = np.tile(w1.target0, (B1, 1)).astype(np.int32)
    long1 = np.ones(B1, np.int32)
    assert B1 < w3.B
    for hists, q, tgt, lg, prm in [(w3.hists, q3, t3, long3, dict()),
                                   (small, q1, t1, long1, dict(scan_wgs=4 * B1))]:
        p = lcd.default_params(**prm)
        want = _step(False, hists, q, tgt, lg, p)
        got = _step(True, hists, q, tgt, lg, p)
        for k in want:
            np.testing.assert_array_equal(got[k], want[k], err_msg=k)
        assert (got["m"] > 0).any() and (got["acc"] >= 0).all()


def test_noalloc_rejects_oversized_batches(gpu):
    """More requests than the static array holds: LCD_EINVAL from the C ABI,
    before anything is launched."""
    import ctypes
    import context_lookup_drafting_amd as lcd
    L = lcd.load()
    p = lcd.default_params()
    f = ctypes.c_void_p(0x10000)
    args = [f, f, f, f, f, lcd.NOALLOC_MAX_B + 1, 100, f, f, f, ctypes.byref(p), f, f, f, f, f, f,
            f, None, 1, None]
    assert L.lookup_decode_step_noalloc(*args) == lcd.LCD_EINVAL
