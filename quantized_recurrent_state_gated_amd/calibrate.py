"""Offline calibration of a quantized state pool: per-head bit widths and
FP16 pivots (temporal) and per-row x per-column scales (spatial).

The STEPQuant pages describe both parts only in words:
  [P1] "K1 論文詳解" (k1-news, 2026-10-09), 方法;
  [P5] "线性注意力状态量化难题:Qwen状态池70并发就超模型权重" (aitest123),
       时间维度 (lifetime-aware allocation under a fixed budget, FP16 pivots for
       the highest-risk units) and 空间维度 (row influence = expected squared
       weight of a row's error in the output; row scale from magnitude and
       influence; column scale by influence-weighted least squares; the two
       fitted jointly).
Their formulas are not printed; the readings below are this module's own.

Row influence.  An error e in row i of the state entering a step reaches that
step's readout as  o' = alpha (S + e)^T (q - beta (q.k) k) + beta (q.k) v,  so
row i's error is weighted by  w_i = alpha (q - beta (q.k) k)_i  -- a weight
set by the current key, query and gate.  influence_i = E[w_i^2] over the
calibration decode.

Spatial fit.  Objective (per head, over calibration states S):
    J(r, c) = sum_states sum_ij infl_i (S_ij - s_ij quant(S_ij / s_ij))^2,
    s_ij = fl32(r_i c_j), the step's own quantizer.
Start from the two-pass max-abs factors (no clipping), then alternate, with
the codes of the current factors held fixed: column factors by weighted least
squares with row weights infl_i r_i^2 (c_j = sum infl_i r_i q_ij S_ij /
sum infl_i r_i^2 q_ij^2), then row factors by least squares per row.  An
update is kept only if J drops, so J never exceeds the max-abs fit.

Temporal allocation.  Lifetime weight L_h = 1 / (1 - abar_h^2), abar_h =
exp(mean ln alpha): the energy an error keeps under the head's average decay.
Distortion D_h(b) = J_h at width b with the fitted factors.  The n_pivots heads
of highest risk L_h D_h(8) -- the ones 8 bits cannot make safe -- stay FP16;
the rest take b_h in {4, 6, 8} minimising sum_h L_h D_h(b_h) subject to
sum_h b_h <= budget, solved exactly by dynamic programming (a multiple-choice
knapsack in units of 2 bits).
"""
from __future__ import annotations

import numpy as np
import torch

from . import inputs as I

WIDTHS = (4, 6, 8)


# ------------------------------------------------------------------ quantizer (offline copy)

def _quant_err(S: torch.Tensor, s: torch.Tensor, Q: int) -> torch.Tensor:
    """Per-element squared error of the symmetric quantizer with step s."""
    q = torch.clamp(torch.round(S / s), -Q, Q)
    return (S - q * s) ** 2


def _codes(S: torch.Tensor, s: torch.Tensor, Q: int) -> torch.Tensor:
    return torch.clamp(torch.round(S / s), -Q, Q)


# ------------------------------------------------------------------ statistics

def row_influence(w: I.Workload, steps: int, device="cpu") -> torch.Tensor:
    """E[(alpha (q - beta (q.k) k))_i^2] per head and row, [H][dk], over the
    calibration decode of workload w (all requests, `steps` steps)."""
    acc = torch.zeros(w.n_heads, w.dk, dtype=torch.float64, device=device)
    for t in range(steps):
        si = I.step_inputs(w, t, device)
        q, k = si.q.double(), si.k.double()
        qk = (q * k).sum(-1, keepdim=True)
        wv = si.alpha.double()[..., None] * (q - si.beta.double()[..., None] * qk * k)
        acc += (wv * wv).sum(0)
    return (acc / (steps * w.n_req)).float()


def lifetime_weight(w: I.Workload, steps: int, device="cpu") -> torch.Tensor:
    """L_h = 1 / (1 - abar_h^2), abar_h = exp(mean over the calibration decode
    of ln alpha)."""
    acc = torch.zeros(w.n_heads, dtype=torch.float64, device=device)
    for t in range(steps):
        acc += torch.log(I.step_inputs(w, t, device).alpha.double()).sum(0)
    abar = torch.exp(acc / (steps * w.n_req))
    return (1.0 / (1.0 - abar * abar).clamp_min(1e-12)).float()


# ------------------------------------------------------------------ spatial fit

def maxabs_scales(S: torch.Tensor, bits) -> tuple:
    """Two-pass max-abs factors over states S [N][H][dk][dv]: r_i = max |S_i.|,
    c_j = max_i (|S_ij| / r_i) / Q.  Widths > 8 get 1."""
    bits = np.asarray(bits)
    A = S.abs()
    R = A.amax(dim=(0, 3)).clamp_min(1e-30)
    C = (A / R[None, :, :, None]).amax(dim=(0, 2))
    Qb = torch.tensor([(2 ** (int(b) - 1) - 1) if b <= 8 else 1 for b in bits], dtype=S.dtype,
                      device=S.device)
    c = (C / Qb[:, None]).clamp_min(1e-30)
    quant = torch.from_numpy(bits <= 8).to(S.device)
    r = torch.where(quant[:, None], R, torch.ones_like(R))
    c = torch.where(quant[:, None], c, torch.ones_like(c))
    return r.float(), c.float()


def weighted_error(S: torch.Tensor, infl: torch.Tensor, r: torch.Tensor, c: torch.Tensor,
                   bits) -> torch.Tensor:
    """J per head: sum over states and elements of infl_i (S - deq(quant(S)))^2,
    with the fp32 step fl32(r_i c_j).  Widths > 8 count as lossless."""
    bits = np.asarray(bits)
    J = torch.zeros(S.shape[1], dtype=torch.float64, device=S.device)
    for b in sorted(set(int(x) for x in bits)):
        if b > 8:
            continue
        hs = torch.from_numpy(np.nonzero(bits == b)[0]).to(S.device)
        s = (r[hs][:, :, None] * c[hs][:, None, :]).float()
        e = _quant_err(S[:, hs].float(), s[None], 2 ** (b - 1) - 1).double()
        J[hs] = (e.sum(dim=(0, 3)) * infl[hs].double()).sum(-1)
    return J


def column_step(S: torch.Tensor, infl: torch.Tensor, r: torch.Tensor, c: torch.Tensor, bits):
    """One column update of the fit: with the codes q of the current factors
    held fixed, c_j minimises sum_states sum_i infl_i (S_ij - r_i c_j q_ij)^2,
    i.e. c_j = sum infl_i r_i q_ij S_ij / sum infl_i r_i^2 q_ij^2 (a column
    whose codes are all zero, or whose solution is not positive, keeps its
    factor).  Heads wider than 8 bits are left alone."""
    bits = np.asarray(bits)
    c2 = c.clone()
    for b in sorted(set(int(x) for x in bits)):
        if b > 8:
            continue
        hs = torch.from_numpy(np.nonzero(bits == b)[0]).to(S.device)
        Sh, rh, ch = S[:, hs].double(), r[hs].double(), c[hs].double()
        q = _codes(Sh, (rh[:, :, None] * ch[:, None, :])[None], 2 ** (b - 1) - 1)
        wi = infl[hs].double()[None, :, :, None]
        X = rh[None, :, :, None] * q                      # the regressor of c_j
        num = (wi * X * Sh).sum(dim=(0, 2))
        den = (wi * X * X).sum(dim=(0, 2))
        new = torch.where(den > 0, num / den.clamp_min(1e-300), ch)
        c2[hs] = torch.where(new > 0, new, ch).float()
    return c2


def row_step(S: torch.Tensor, infl: torch.Tensor, r: torch.Tensor, c: torch.Tensor, bits):
    """One row update: codes fixed, r_i minimises sum_states sum_j
    infl_i (S_ij - r_i c_j q_ij)^2 -- infl_i is one weight for the whole row,
    so r_i = sum c_j q_ij S_ij / sum c_j^2 q_ij^2 (same keep rules as
    column_step)."""
    bits = np.asarray(bits)
    r2 = r.clone()
    for b in sorted(set(int(x) for x in bits)):
        if b > 8:
            continue
        hs = torch.from_numpy(np.nonzero(bits == b)[0]).to(S.device)
        Sh, rh, ch = S[:, hs].double(), r[hs].double(), c[hs].double()
        q = _codes(Sh, (rh[:, :, None] * ch[:, None, :])[None], 2 ** (b - 1) - 1)
        X = ch[None, :, None, :] * q                      # the regressor of r_i
        num = (X * Sh).sum(dim=(0, 3))
        den = (X * X).sum(dim=(0, 3))
        new = torch.where(den > 0, num / den.clamp_min(1e-300), rh)
        r2[hs] = torch.where(new > 0, new, rh).float()
    return r2


def fit_scales(S: torch.Tensor, infl: torch.Tensor, bits, iters: int = 4):
    """Key-row-aware dual-axis fit (see the module docstring): from the
    max-abs factors, alternate column_step and row_step, keeping each update
    only where the head's weighted error J drops.  Returns (r, c, history)
    with history[k] = J per head after iteration k (k = 0 is the max-abs
    fit)."""
    bits = np.asarray(bits)
    r, c = maxabs_scales(S, bits)
    J = weighted_error(S, infl, r, c, bits)
    hist = [J.clone()]
    for _ in range(iters):
        for axis in ("col", "row"):
            if axis == "col":
                r2, c2 = r, column_step(S, infl, r, c, bits)
            else:
                r2, c2 = row_step(S, infl, r, c, bits), c
            J2 = weighted_error(S, infl, r2, c2, bits)
            keep = (J2 < J)
            r = torch.where(keep[:, None], r2, r)
            c = torch.where(keep[:, None], c2, c)
            J = torch.where(keep, J2, J)
        hist.append(J.clone())
    return r, c, hist


# ------------------------------------------------------------------ temporal allocation

def allocate(L, D, budget_bits: int, n_pivots: int = 0):
    """Per-head widths.  L [H] lifetime weights, D [H][3] distortion at
    4/6/8 bits.  The n_pivots heads of largest L * D[:, 8-bit] become 16 (FP16
    pivots); the others take widths from {4, 6, 8} minimising sum L_h D_h(b)
    with sum b <= budget_bits (exact DP).  Returns uint8 widths [H]."""
    L = np.asarray(L, np.float64)
    D = np.asarray(D, np.float64)
    H = L.size
    bits = np.zeros(H, np.uint8)
    risk = L * D[:, 2]
    piv = np.argsort(-risk, kind="stable")[:n_pivots]
    bits[piv] = 16
    rest = np.array([h for h in range(H) if bits[h] == 0], np.int64)
    cost = np.array([2, 3, 4])  # widths in units of 2 bits
    B = budget_bits // 2
    if rest.size and cost.min() * rest.size > B:
        raise ValueError("budget below the narrowest width for every head")
    INF = float("inf")
    # best[h][u]: minimal weighted distortion of the first h heads using exactly u units
    best = np.full(B + 1, INF)
    best[0] = 0.0
    choice = np.zeros((rest.size, B + 1), np.int8)
    for n, h in enumerate(rest):
        new = np.full(B + 1, INF)
        for w_i, cst in enumerate(cost):
            cand = np.full(B + 1, INF)
            cand[cst:] = best[:-cst] + L[h] * D[h, w_i]
            better = cand < new
            new[better] = cand[better]
            choice[n, better] = w_i
        best = new
    u = int(np.argmin(best))
    for n in range(rest.size - 1, -1, -1):
        w_i = int(choice[n, u])
        bits[rest[n]] = WIDTHS[w_i]
        u -= int(cost[w_i])
    return bits


# ------------------------------------------------------------------ end to end (GPU)

def calibration_states(w: I.Workload, steps: int, stride: int, n_req: int, device="cuda"):
    """FP32-state trajectory of the calibration decode through the HIP step
    (all heads FP32), sampled every `stride` steps: [samples*n_req][H][dk][dv]."""
    from . import sq

    wc = I.scaled(w, n_req=n_req)
    H = wc.n_heads
    bits = np.full(H, 32, np.uint8)
    ones_r = torch.ones(H, wc.dk, device=device)
    ones_c = torch.ones(H, wc.dv, device=device)
    nbytes = sq.sq_pool_bytes(wc.n_req, H, wc.dk, wc.dv, bits)
    state = torch.empty(nbytes, dtype=torch.uint8, device=device)
    pool = sq.sq_pool_alloc(wc.n_req, H, wc.dk, wc.dv, bits, ones_r, ones_c, state)
    slots = torch.arange(wc.n_req, dtype=torch.int32, device=device)
    for p in range(wc.n_req):
        sq.sq_pool_store(pool, slots[p:p + 1], I.initial_state(wc, p, device))
    snaps = []
    buf = torch.empty(wc.n_req, H, wc.dk, wc.dv, device=device)
    for t in range(steps):
        si = I.step_inputs(wc, t, device)
        sq.sq_decode_step(pool, slots, si.q, si.k, si.v, si.alpha, si.beta, None)
        if (t + 1) % stride == 0:
            sq.sq_pool_load(pool, slots, buf)
            snaps.append(buf.clone())
    return torch.cat(snaps)


def calibrate(w: I.Workload, budget_mean_bits: float, n_pivots: int, steps: int = 256,
              stride: int = 32, n_req: int = 4, iters: int = 3, seed_offset: int = 7777,
              device="cuda"):
    """Calibrate widths and factors for workload w on a separate calibration
    decode (seed w.seed + seed_offset).  Returns dict(bits, r, c, report)."""
    # the head set (half-lives, outlier positions) is the model's; only the
    # decode inputs and states differ from the evaluation run
    wc_inputs = I.Workload(w.name + "-calib", n_req, w.n_heads, w.dk, w.dv, steps, dict(w.counts),
                           w.half_life, w.beta_range, w.qkv_dtype, w.tiny_recipe,
                           w.persistent_outliers, w.seed,
                           dict(w.extra, input_seed=w.seed + seed_offset))
    S = calibration_states(wc_inputs, steps, stride, n_req, device)
    infl = row_influence(wc_inputs, steps, device)
    L = lifetime_weight(wc_inputs, steps, device)
    H = w.n_heads
    D = np.zeros((H, 3))
    fits = {}
    for i, b in enumerate(WIDTHS):
        bb = np.full(H, b, np.uint8)
        r, c, hist = fit_scales(S, infl, bb, iters)
        fits[b] = (r, c)
        D[:, i] = hist[-1].cpu().numpy()
    D_maxabs = np.zeros((H, 3))
    for i, b in enumerate(WIDTHS):
        D_maxabs[:, i] = weighted_error(S, infl, *maxabs_scales(S, np.full(H, b)),
                                        np.full(H, b)).cpu().numpy()
    n_quant = H - n_pivots
    bits = allocate(L.cpu().numpy(), D, int(round(budget_mean_bits * n_quant)), n_pivots)
    r = torch.ones(H, w.dk, device=device)
    c = torch.ones(H, w.dv, device=device)
    for b in WIDTHS:
        hs = torch.from_numpy(np.nonzero(bits == b)[0]).to(device)
        r[hs] = fits[b][0][hs]
        c[hs] = fits[b][1][hs]
    return {"bits": bits, "r": r.contiguous(), "c": c.contiguous(),
            "report": {"mean_bits_nonpivot": float(np.mean(bits[bits <= 8])),
                       "counts": {str(int(b)): int((bits == b).sum()) for b in sorted(set(bits))},
                       "weighted_distortion": float((L.cpu().numpy() *
                                                     np.where(bits[:, None] == np.array(WIDTHS)[None], D, 0).sum(1)).sum()),
                       # the same widths with the max-abs factors the fit starts from
                       "weighted_distortion_maxabs": float((L.cpu().numpy() *
                                                            np.where(bits[:, None] == np.array(WIDTHS)[None], D_maxabs, 0).sum(1)).sum())}}
