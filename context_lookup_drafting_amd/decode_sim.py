"""Replay a synthetic decode through a LookupDrafter on the GPU.

Each step: the draft model's proposal and the target's argmax tokens come from
the workload's truth stream (workloads.Workload.step_inputs), one
lookup_decode_step launch does lookup, fusion, greedy acceptance with append
and the scheduler update, and the emitted tokens advance each request's
position in its truth stream.  Acceptance telemetry is kept on the GPU and
summarised per request class -- the diagnostics the article's forum thread
asks for before any speed claim: hit rate, mean accepted length and its
distribution, long-block residency.

    python -m context_lookup_drafting_amd.decode_sim [--config 3] [--steps 256]
"""

from __future__ import annotations

import argparse
import json

import numpy as np

from . import workloads as wl


def run_fused(w: wl.Workload, steps: int, params=None, device="cuda:0", record=False,
              index: bool = False):
    """Runs `steps` decode steps through a LookupDrafter (one fused kernel per
    step, or with ``index`` the lookup from the incremental index); returns a
    dict with the emitted tokens per request, the final history, lengths and
    telemetry rows (uint32 [B,32]) and, with record=True, every step's
    outputs."""
    import torch
    import context_lookup_drafting_amd as lcd
    params = params or lcd.default_params()
    flat, row_off, lens, cap = wl.pack_rows(w.hists, extra=wl.N_TARGET * (steps + 1))
    B = w.B
    dev = torch.device(device)
    h_d = torch.from_numpy(flat).to(dev)
    ro_d = torch.from_numpy(row_off).to(dev)
    len_d = torch.from_numpy(lens.copy()).to(dev)
    cap_d = torch.from_numpy(cap).to(dev)
    max_len = int(lens.max()) + wl.N_TARGET * (steps + 1) if B else 0
    dr = lcd.LookupDrafter(B, max_len, dev, params, telemetry=True,
                           index_cap=cap if index else None)
    if index:
        dr.build_index(h_d, ro_d, len_d)
    pos = np.zeros(B, np.int64)
    recs = []
    emitted = [[] for _ in range(B)]
    for t in range(steps):
        q, tgt = w.step_inputs(pos, t)
        long_used = dr.state[:, 0].clone() if record else None
        out = dr.step(h_d, ro_d, len_d, cap_d, torch.from_numpy(q).to(dev),
                      torch.from_numpy(tgt).to(dev), append=True)
        acc_h = out["accept"].cpu().numpy()
        for r in range(B):
            if acc_h[r] >= 0:
                emitted[r].extend(tgt[r, :acc_h[r] + 1].tolist())
        pos = pos + np.maximum(acc_h, 0) + 1
        if record:
            recs.append(dict(m=out["match_len"].cpu().numpy(), e=out["match_end"].cpu().numpy(),
                             d=out["draft"].cpu().numpy(), q=q, tgt=tgt,
                             long=long_used.cpu().numpy(), block=out["block"].cpu().numpy(),
                             blk=out["block_len"].cpu().numpy(), acc=acc_h,
                             state=dr.state.cpu().numpy(),
                             long_next=out["long_next"].cpu().numpy()))
    torch.cuda.synchronize()
    return dict(recs=recs, emitted=emitted, lens=len_d.cpu().numpy(), flat=h_d.cpu().numpy(),
                row_off=row_off, tele=dr.telemetry.cpu().numpy().view(np.uint32),
                tele_d=dr.telemetry)


def summarise(tele_d, class_ids, names):
    """Per-class report from the GPU telemetry rows (totals via
    lookup_telemetry_reduce)."""
    import torch
    import context_lookup_drafting_amd as lcd
    cls = torch.from_numpy(np.asarray(class_ids, np.int32)).to(tele_d.device)
    tot = lcd.telemetry_reduce(tele_d, cls, len(names)).cpu().numpy().view(np.uint64).astype(np.float64)
    rep = {}
    for k, name in enumerate(names):
        t = tot[k]
        steps = t[0]
        if steps == 0:
            continue
        hist = t[lcd.TELE_HIST:lcd.TELE_HIST + 16]
        ok = max(hist.sum(), 1.0)
        rep[name] = {
            "requests": int(np.sum(np.asarray(class_ids) == k)),
            "steps": int(steps),
            "hit_rate": round(t[1] / steps, 4),
            "tokens_per_step": round(t[7] / steps, 3),
            "mean_accepted": round(float((hist * np.arange(16)).sum() / ok), 3),
            "head_from_lookup": round(t[2] / steps, 4),
            "tail_from_lookup": round(t[3] / steps, 4),
            "long_residency": round(t[4] / steps, 4),
            "long_entries": int(t[5]),
            "long_exits": int(t[6]),
            "failed_appends": int(t[8]),
            "accepted_hist": [int(x) for x in hist],
        }
    return rep


def main():
    ap = argparse.ArgumentParser(description="fused decode replay with acceptance telemetry")
    ap.add_argument("--config", type=int, default=3, choices=[2, 3])
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--index", action="store_true", help="lookup from the incremental index")
    args = ap.parse_args()
    w = wl.make_config(args.config)
    res = run_fused(w, args.steps, index=args.index)
    for r in range(w.B):
        em = res["emitted"][r]
        if em != w.truths[r][:len(em)].tolist():
            raise SystemExit(f"request {r}: emitted stream differs from the target's")
    print(json.dumps({"workload": w.name, "steps": args.steps,
                      "classes": summarise(res["tele_d"], w.class_ids, w.CLASS_NAMES)}))


if __name__ == "__main__":
    main()
