"""Long-decode drift report for the quantized state.

Runs the same seeded decode (initial states, q/k/v, gates) through several
state formats on the GPU and reports, per step, the relative error of each
readout against an FP32-state run of the same decode:

    e[n, h, t] = ||o_fmt - o_fp32||_2 / ||o_fp32||_2

Formats: the workload's mixed 4/6/8-bit allocation with FP16 pivots, uniform
4-bit and uniform 8-bit (no pivots), each with row x column factors fitted to
the states of a separate calibration decode; the mixed and uniform 4-bit
widths again with the max-abs factors of the initial state; an unquantized
bfloat16 state (a 16-bit baseline); and the calibrated widths + factors.
Besides the error over all heads, the report splits it over the heads the
mixed allocation upgrades (more than 4 bits) and the heads it leaves at 4
bits (identical in the mixed and uniform 4-bit runs), and samples the share
of stored codes at +-Q every 16 steps.  This mirrors the pages' comparison of mixed-precision state
against uniform INT4 / INT8 ("K1 論文詳解" 實驗結果; "线性注意力状态量化难题"
数据说话) and the accumulation of error over decode steps (直接量化为什么会翻车,
时间维度); it is a report, not a correctness gate.  The per-head mean error is
also rank-correlated (Spearman) with the head's gate half-life, the synthetic
analogue of the pages' half-life / accumulated-error correlation (时间维度).

    python -m quantized_recurrent_state_gated_amd.drift [--workload drift] [--steps N] [--out report.json]
        [--curves full.json] [--no-calibrated] [--kda]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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
        self.w = w
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
        # byte index of every code tile, per width, for the saturation count
        self._idx = {}
        for b in (4, 6, 8):
            hs = np.nonzero(self.bits == b)[0]
            if hs.size:
                offs = [self.sq.sq_pool_tile_offset(self.pool, 0, int(h)) for h in hs]
                self._idx[b] = (torch.tensor([o for o, _ in offs], device=dev)[:, None] +
                                torch.arange(offs[0][1], device=dev)[None, :])

    def step(self, si, kda=False):
        step = self.sq.sq_decode_step_kda if kda else self.sq.sq_decode_step
        step(self.pool, self.slots, si.q, si.k, si.v, si.alpha, si.beta, self.o)
        return self.o

    def saturated(self):
        """Fraction of the stored codes at +-Q (clamped or rounded onto the
        bound), over every code tile of the pool; None without code heads."""
        rows = self.state.view(self.w.n_req, -1)
        hit = tot = 0
        for b, idx in self._idx.items():
            t = rows[:, idx].to(torch.int32)
            if b == 8:
                f = t
            elif b == 4:
                f = torch.stack([t & 15, t >> 4], -1)
            else:
                g = t.view(t.shape[0], t.shape[1], -1, 3)
                word = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
                f = torch.stack([(word >> sh) & 63 for sh in (0, 6, 12, 18)], -1)
            hit += int(((f == 1) | (f == (1 << b) - 1)).sum())
            tot += f.numel()
        return hit / tot if tot else None


def _calib_workload(w, n_req=4, steps=256, seed_offset=7777):
    """The calibration decode of workload w: the same heads (half-lives,
    outlier positions), other decode inputs and states."""
    return I.Workload(w.name + "-calib", n_req, w.n_heads, w.dk, w.dv, steps, dict(w.counts),
                      w.half_life, w.beta_range, w.qkv_dtype, w.tiny_recipe, w.persistent_outliers,
                      w.seed, dict(w.extra, input_seed=w.seed + seed_offset))


def report(workload: str = "drift", steps: int | None = None, device: str = "cuda",
           calibrated: bool = True, kda: bool = False, sat_every: int = 16) -> dict:
    """Per-step readout error of every format against the FP32-state run.

    Primary formats take factors fitted to states of a separate calibration
    decode (the pages' offline fit, [P5] 空间维度): the workload's mixed
    widths, uniform 4-bit and uniform 8-bit.  The secondary ones take the
    two-pass max-abs of the initial states, which the state can outgrow as it
    drifts.  With calibrated, the calibrated widths + factors run as well.
    kda: every run (the FP32 reference included) steps with the per-key-channel
    gate, alpha from inputs.channel_gates."""
    from . import calibrate as CAL

    w = I.WORKLOADS[workload]
    steps = steps or w.steps
    dev = torch.device(device)
    H = w.n_heads
    mixed = I.head_bits(w)
    u4, u8 = np.full(H, 4, np.uint8), np.full(H, 8, np.uint8)
    t0 = time.time()
    wc = _calib_workload(w)
    S = CAL.calibration_states(wc, wc.steps, 32, wc.n_req, device)
    infl = CAL.row_influence(wc, wc.steps, device)
    fitted, gains = {}, {}
    for name, b in (("mixed", mixed), ("uniform_int4", u4), ("uniform_int8", u8)):
        r, c, hist = CAL.fit_scales(S, infl, b, iters=3)
        fitted[name] = (b, (r, c))
        gains[name] = float((hist[-1].sum() / hist[0].sum()).item())
    del S
    print(f"[drift] factors fitted on the calibration decode ({time.time() - t0:.1f} s)", flush=True)
    formats = {k: v[0] for k, v in fitted.items()}
    formats["uniform_bf16"] = np.full(H, I.BITS_BF16, np.uint8)
    formats["mixed_maxabs_s0"] = mixed
    formats["uniform_int4_maxabs_s0"] = u4
    ref = Run(w, np.full(H, 32, np.uint8), dev)
    runs = {k: Run(w, b, dev, fitted[k][1] if k in fitted else None) for k, b in formats.items()}
    calib_info = {"fit_gain_vs_maxabs": gains}
    if calibrated:
        n_piv = int((mixed == 16).sum())
        cal = CAL.calibrate(w, float(np.mean(mixed[mixed <= 8])), n_piv, device=device)
        runs["calibrated"] = Run(w, cal["bits"], dev, (cal["r"], cal["c"]))
        formats["calibrated"] = cal["bits"]
        calib_info["calibrated"] = cal["report"]
    # heads the mixed allocation gives more than 4 bits, and those it leaves at 4
    groups = {"upgraded": torch.from_numpy(mixed != 4).to(dev),
              "shared_4bit": torch.from_numpy(mixed == 4).to(dev)}
    curves = {k: {"mean": [], "p50": [], "p99": []} for k in runs}
    gcurves = {k: {g: [] for g in groups} for k in runs}
    sat = {k: {} for k in runs}
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
            for g, m in groups.items():
                gcurves[k][g].append(float(e[:, m].mean()) if bool(m.any()) else None)
            head_sum[k] += e.sum(dim=0).double()
            if t % sat_every == 0 or t == steps - 1:
                sat[k][t] = run.saturated()
        if t % 256 == 0 or t == steps - 1:
            msg = " ".join(f"{k}={curves[k]['mean'][-1]:.2e}" for k in runs)
            print(f"[drift] step {t}: mean rel err {msg} ({time.time() - t0:.1f} s)", flush=True)
    hl = I.half_lives(w)
    marks = sorted({0, 15, 127, 511, 1023, steps - 1} & set(range(steps)))
    out = {
        "workload": {"name": w.name, "n_req": w.n_req, "n_heads": H, "d": w.dk, "steps": steps,
                     "half_life": list(w.half_life),
                     "mixed_bits": {str(int(b)): int((mixed == b).sum()) for b in sorted(set(mixed))},
                     "upgraded_heads": int((mixed != 4).sum())},
        "reference": "FP32-state run of the same decode (same S0, q/k/v, gates)",
        "gate": "per-key-channel (KDA reading)" if kda else "scalar per head",
        "metric": "||o - o_fp32||_2 / ||o_fp32||_2 per (request, head), stats over requests x heads",
        "factors": {k: ("fitted on the calibration decode" if k in fitted else
                        "calibrated" if k == "calibrated" else
                        "none (unquantized)" if k == "uniform_bf16" else "max-abs of S0")
                    for k in runs},
        "summary": {}, "groups": {}, "saturated_code_fraction": {},
        "spearman_head_error_vs_half_life": {},
        "calibration": calib_info,
        "curves": curves,
    }
    for k in runs:
        out["summary"][k] = {str(t): {s: curves[k][s][t] for s in ("mean", "p50", "p99")}
                             for t in marks}
        out["groups"][k] = {g: {str(t): gcurves[k][g][t] for t in marks} for g in groups}
        out["saturated_code_fraction"][k] = {str(t): v for t, v in sorted(sat[k].items())
                                             if v is not None and (t in marks or t % 256 == 0)}
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
    ap.add_argument("--out", default=None,
                    help="write the report (without the per-step curves) here")
    ap.add_argument("--curves", default=None, help="write the full report with per-step curves here")
    ap.add_argument("--no-calibrated", action="store_true",
                    help="skip the run with calibrated widths and factors")
    ap.add_argument("--kda", action="store_true",
                    help="step every format with the per-key-channel gate")
    a = ap.parse_args(argv)
    rep = report(a.workload, a.steps, calibrated=not a.no_calibrated, kda=a.kda)
    brief = {k: v for k, v in rep.items() if k != "curves"}
    brief["command"] = "python -m quantized_recurrent_state_gated_amd.drift " + " ".join(
        argv if argv is not None else sys.argv[1:])
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "sq_kernels.hip"), "rb") as f:
        brief["kernel_source_sha"] = hashlib.sha256(f.read()).hexdigest()[:16]
    if a.curves:
        with open(a.curves, "w") as f:
            json.dump(rep, f)
    if a.out:
        with open(a.out, "w") as f:
            json.dump(brief, f, indent=1)
    print(json.dumps(brief, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
