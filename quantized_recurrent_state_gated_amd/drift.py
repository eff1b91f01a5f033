"""Long-decode drift report for the quantized state.

Runs the same seeded decode (initial states, q/k/v, gates) through several
state formats on the GPU and reports, per step, the relative error of each
readout against an FP32-state run of the same decode:

    e[n, h, t] = ||o_fmt - o_fp32||_2 / ||o_fp32||_2

Formats: the workload's mixed 4/6/8-bit allocation with FP16 pivots, uniform
4-bit (same dual-axis max-abs scales re-derived for 4 bits, no pivots),
uniform 8-bit, and an unquantized bfloat16 state (a 16-bit baseline).  This mirrors the pages' comparison of mixed-precision state
against uniform INT4 / INT8 ("K1 論文詳解" 實驗結果; "线性注意力状态量化难题"
数据说话) and the accumulation of error over decode steps (直接量化为什么会翻车,
时间维度); it is a report, not a correctness gate.  The per-head mean error is
also rank-correlated (Spearman) with the head's gate half-life, the synthetic
analogue of the pages' half-life / accumulated-error correlation (时间维度).

    python -m quantized_recurrent_state_gated_amd.drift [--workload drift] [--steps N] [--out report.json]
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np
import torch

from . import inputs as I


def _ranks(x: np.ndarray) -> np.ndarray:
    order = np.argsort(x, kind="stable")
    r = np.empty(len(x), np.float64)
    r[order] = np.arange(len(x), dtype=np.float64)
    # average ranks over ties
    xs = x[order]
    i = 0
    while i < len(xs):
        j = i
        while j + 1 < len(xs) and xs[j + 1] == xs[i]:
            j += 1
        r[order[i:j + 1]] = (i + j) / 2.0
        i = j + 1
    return r


def spearman(a, b) -> float:
    ra, rb = _ranks(np.asarray(a, np.float64)), _ranks(np.asarray(b, np.float64))
    ra -= ra.mean()
    rb -= rb.mean()
    return float((ra * rb).sum() / np.sqrt((ra * ra).sum() * (rb * rb).sum()))


class Run:
    def __init__(self, w, bits, dev, scales=None):
        from . import sq  # the HIP library; raises if it is not built
        self.sq = sq
        self.bits = np.asarray(bits, np.uint8)
        if scales is None:
            self.r, self.c = I.scales(w, device=dev, bits=self.bits)
        else:
            self.r, self.c = (x.to(dev).float().contiguous() for x in scales)
        nbytes = self.sq.sq_pool_bytes(w.n_req, w.n_heads, w.dk, w.dv, self.bits)
        self.state = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.pool = self.sq.sq_pool_alloc(w.n_req, w.n_heads, w.dk, w.dv, self.bits, self.r, self.c,
                                     self.state)
        self.slots = torch.arange(w.n_req, dtype=torch.int32, device=dev)
        for p in range(w.n_req):
            self.sq.sq_pool_store(self.pool, self.slots[p:p + 1], I.initial_state(w, p, dev))
        self.o = torch.empty(w.n_req, w.n_heads, w.dv, device=dev)

    def step(self, si, kda=False):
        step = self.sq.sq_decode_step_kda if kda else self.sq.sq_decode_step
        step(self.pool, self.slots, si.q, si.k, si.v, si.alpha, si.beta, self.o)
        return self.o


def report(workload: str = "drift", steps: int | None = None, device: str = "cuda",
           calibrated: bool = False, kda: bool = False) -> dict:
    """kda: every run (the FP32 reference included) steps with the per-key-channel
    gate, alpha from inputs.channel_gates."""
    w = I.WORKLOADS[workload]
    steps = steps or w.steps
    dev = torch.device(device)
    H = w.n_heads
    formats = {"mixed": I.head_bits(w), "uniform_int4": np.full(H, 4, np.uint8),
               "uniform_int8": np.full(H, 8, np.uint8),
               "uniform_bf16": np.full(H, I.BITS_BF16, np.uint8)}
    ref = Run(w, np.full(H, 32, np.uint8), dev)
    runs = {k: Run(w, b, dev) for k, b in formats.items()}
    calib_info = {}
    if calibrated:
        from . import calibrate as CAL
        bits0 = formats["mixed"]
        n_piv = int((bits0 == 16).sum())
        mean_bits = float(np.mean(bits0[bits0 <= 8]))
        t0 = time.time()
        cal = CAL.calibrate(w, mean_bits, n_piv, device=device)
        print(f"[drift] calibration: {cal['report']} ({time.time() - t0:.1f} s)", flush=True)
        # spatial part alone: the half-life-ranked widths with fitted factors
        S = CAL.calibration_states(I.Workload(w.name + "-calib", 4, H, w.dk, w.dv, 256, dict(w.counts),
                                              w.half_life, w.beta_range, w.qkv_dtype, w.tiny_recipe,
                                              w.persistent_outliers, w.seed,
                                              dict(w.extra, input_seed=w.seed + 7777)),
                                   256, 32, 4, device)
        wc = I.Workload(w.name + "-calib", 4, H, w.dk, w.dv, 256, dict(w.counts), w.half_life,
                        w.beta_range, w.qkv_dtype, w.tiny_recipe, w.persistent_outliers, w.seed,
                        dict(w.extra, input_seed=w.seed + 7777))
        infl = CAL.row_influence(wc, 256, device)
        r_s, c_s, hist = CAL.fit_scales(S, infl, bits0, iters=3)
        del S
        runs["mixed_fitted_scales"] = Run(w, bits0, dev, (r_s, c_s))
        formats["mixed_fitted_scales"] = bits0
        runs["calibrated"] = Run(w, cal["bits"], dev, (cal["r"], cal["c"]))
        formats["calibrated"] = cal["bits"]
        calib_info = {"calibrated": cal["report"],
                      "fit_gain_mixed_widths": float((hist[-1].sum() / hist[0].sum()).item())}
    curves = {k: {"mean": [], "p50": [], "p99": []} for k in runs}
    head_sum = {k: torch.zeros(H, device=dev, dtype=torch.float64) for k in runs}
    qs = torch.tensor([0.5, 0.99], device=dev)
    t0 = time.time()
    for t in range(steps):
        si = I.step_inputs(w, t, dev)
        if kda:
            si.alpha = I.channel_gates(w, t, dev)
        o_ref = ref.step(si, kda)
        nref = o_ref.norm(dim=-1).clamp_min(1e-30)
        for k, run in runs.items():
            e = (run.step(si, kda) - o_ref).norm(dim=-1) / nref  # [n_req, H]
            flat = e.flatten()
            qv = torch.quantile(flat, qs)
            curves[k]["mean"].append(float(flat.mean()))
            curves[k]["p50"].append(float(qv[0]))
            curves[k]["p99"].append(float(qv[1]))
            head_sum[k] += e.sum(dim=0).double()
        if t % 256 == 0 or t == steps - 1:
            msg = " ".join(f"{k}={curves[k]['mean'][-1]:.2e}" for k in runs)
            print(f"[drift] step {t}: mean rel err {msg} ({time.time() - t0:.1f} s)", flush=True)
    hl = I.half_lives(w)
    mixed_bits = formats["mixed"]
    out = {
        "workload": {"name": w.name, "n_req": w.n_req, "n_heads": H, "d": w.dk, "steps": steps,
                     "half_life": list(w.half_life),
                     "mixed_bits": {str(int(b)): int((mixed_bits == b).sum()) for b in sorted(set(mixed_bits))}},
        "reference": "FP32-state run of the same decode (same S0, q/k/v, gates)",
        "gate": "per-key-channel (KDA reading)" if kda else "scalar per head",
        "metric": "||o - o_fp32||_2 / ||o_fp32||_2 per (request, head), stats over requests x heads",
        "curves": curves,
        "summary": {},
        "spearman_head_error_vs_half_life": {},
        "calibration": calib_info,
    }
    for k in runs:
        out["summary"][k] = {str(t): {s: curves[k][s][t] for s in ("mean", "p50", "p99")}
                             for t in sorted({0, 15, 127, 511, 1023, steps - 1}) if t < steps}
        per_head = (head_sum[k] / (steps * w.n_req)).cpu().numpy()
        quant = formats[k] <= 8
        if quant.sum() < 3:  # an unquantized format: rank over every head
            quant = np.ones_like(quant)
        out["spearman_head_error_vs_half_life"][k] = spearman(per_head[quant], hl[quant])
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="drift")
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--out", default=None)
    ap.add_argument("--calibrated", action="store_true",
                    help="also run the calibrated widths and factors (offline calibration)")
    ap.add_argument("--kda", action="store_true",
                    help="step every format with the per-key-channel gate")
    a = ap.parse_args(argv)
    rep = report(a.workload, a.steps, calibrated=a.calibrated, kda=a.kda)
    text = json.dumps(rep)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    brief = {k: v for k, v in rep.items() if k != "curves"}
    print(json.dumps(brief, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
