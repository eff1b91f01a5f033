"""Seeded synthetic inputs for the quantized decode step.

This module only draws random numbers with the shapes and statistics of the
workloads the STEPQuant pages describe; it holds none of the step's
arithmetic (no quantization, packing, update or readout).  Both the GPU path
and the CPU oracle consume what it produces.

Sources:
  [P1] "K1 論文詳解" (k1-news, 2026-10-09), STEPQuant article, 背景 / 方法.
  [P5] "线性注意力状态量化难题:Qwen状态池70并发就超模型权重" (aitest123),
       时间维度 (half-life, 2304 heads, 1.39 % FP16 pivots),
       空间维度 (row / column outliers 10.3x / 19.4x, persistent over 2048 steps).

Workloads (the pages measure real models on benchmarks; these synthetic
activations stand in for them, with the pages' shapes):
  tiny     1 request x 4 heads, d=16, 8 steps, all 8-bit, fp32 q/k/v
  layer    8 x 48, d=128, 256 steps, 12/23/12 heads at 4/6/8 bit + 1 pivot
  serving  70 x 2304, d=128, 64 steps, 568/1136/568 + 32 pivots (6-bit mean)
  highconc 256 x 2304, d=128, 32 steps, 2080/128/64 + 32 pivots (4.225-bit mean)
  drift    16 x 576, d=128, 2048 steps, 520/32/16 + 8 pivots, persistent outliers
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

# Row / column max-over-median ratios of the recurrent state ([P5] 空间维度).
ROW_RATIO_TARGET = 10.3
COL_RATIO_TARGET = 19.4
N_OUTLIER_ROWS = 4
N_OUTLIER_COLS = 4
STATE_SIGMA = 0.5  # element std of the non-outlier state
BITS_BF16 = 144    # head_bits value of a bfloat16 state (16-bit fields)


def field_width(bits: int) -> int:
    """Bits per stored element of a head format (head_bits value)."""
    return 16 if int(bits) == BITS_BF16 else int(bits)


@dataclass(frozen=True)
class Workload:
    name: str
    n_req: int
    n_heads: int
    dk: int
    dv: int
    steps: int
    counts: dict            # {bits: number of heads}; 16 = FP16 pivot
    half_life: tuple = (1.0, 1000.0)
    beta_range: tuple = (0.05, 0.95)
    qkv_dtype: str = "bf16"  # "bf16" or "f32"
    tiny_recipe: bool = False
    persistent_outliers: bool = False
    seed: int = 20261009
    extra: dict = field(default_factory=dict)

    @property
    def tiles(self) -> int:
        return self.n_req * self.n_heads


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 16, 16, 8, {8: 4}, beta_range=(0.0, 1.0), qkv_dtype="f32",
                     tiny_recipe=True, seed=20261009 + 1),
    "layer": Workload("layer", 8, 48, 128, 128, 256, {4: 12, 6: 23, 8: 12, 16: 1}, seed=20261009 + 2),
    "serving": Workload("serving", 70, 2304, 128, 128, 64, {4: 568, 6: 1136, 8: 568, 16: 32},
                        seed=20261009 + 3),
    "highconc": Workload("highconc", 256, 2304, 128, 128, 32, {4: 2080, 6: 128, 8: 64, 16: 32},
                         seed=20261009 + 4),
    "drift": Workload("drift", 16, 576, 128, 128, 2048, {4: 520, 6: 32, 8: 16, 16: 8},
                      half_life=(1.0, 4000.0), persistent_outliers=True, seed=20261009 + 5),
}


def scaled(w: Workload, n_req: int | None = None, n_heads: int | None = None,
           steps: int | None = None, name: str | None = None) -> Workload:
    """A workload with the same recipe at another size (bit counts rescaled,
    at least one head per width present in the original)."""
    H = n_heads or w.n_heads
    counts = dict(w.counts)
    if H != w.n_heads:
        tot = sum(counts.values())
        new = {b: max(1, round(n * H / tot)) for b, n in counts.items()}
        big = max(new, key=lambda b: new[b])
        new[big] += H - sum(new.values())
        counts = new
    return Workload(name or w.name, n_req or w.n_req, H, w.dk, w.dv, steps or w.steps, counts,
                    w.half_life, w.beta_range, w.qkv_dtype, w.tiny_recipe,
                    w.persistent_outliers, w.seed, dict(w.extra))


def _rng(w: Workload, stream: int) -> np.random.Generator:
    return np.random.default_rng([w.seed, stream])


def _torch_gen(w: Workload, stream: int, device) -> torch.Generator:
    """Generator for decode inputs and initial states.  They use the workload's
    input seed (extra["input_seed"], default the workload seed); per-head
    properties (half-lives, widths, outlier positions) always use the workload
    seed, so a calibration decode of the same heads differs only in its inputs."""
    g = torch.Generator(device=device)
    seed = int(w.extra.get("input_seed", w.seed))
    g.manual_seed((seed * 1000003 + stream * 7919) % (2 ** 62))
    return g


# ------------------------------------------------------------------ per head

def half_lives(w: Workload) -> np.ndarray:
    """Per-head gate half-life in steps, log-uniform over w.half_life ([P5] 时间维度)."""
    lo, hi = w.half_life
    return np.exp(_rng(w, 1).uniform(math.log(lo), math.log(hi), w.n_heads))


def head_bits(w: Workload) -> np.ndarray:
    """Bit width per head.  Heads are ranked by half-life, longest first; the
    longest-lived become FP16 pivots, then 8-, 6- and 4-bit heads in that
    order -- the plainest stand-in for the pages' lifetime-aware allocation
    ([P1] 方法; [P5] 时间维度), which needs calibration data."""
    assert sum(w.counts.values()) == w.n_heads
    order = np.argsort(-half_lives(w), kind="stable")
    bits = np.zeros(w.n_heads, np.uint8)
    pos = 0
    for b in (32, BITS_BF16, 16, 8, 6, 4):
        n = w.counts.get(b, 0)
        bits[order[pos:pos + n]] = b
        pos += n
    return bits


def outlier_positions(w: Workload):
    """Per head: indices of the outlier rows and columns (fixed across requests)."""
    rng = _rng(w, 2)
    rows = np.stack([rng.choice(w.dk, N_OUTLIER_ROWS, replace=False) for _ in range(w.n_heads)])
    cols = np.stack([rng.choice(w.dv, N_OUTLIER_COLS, replace=False) for _ in range(w.n_heads)])
    return rows, cols


def _ratios(S: torch.Tensor):
    """Per tile: (max_i R_i / median_i R_i, max_j C_j / median_j C_j), R/C = row/col max-abs."""
    A = S.abs()
    R = A.amax(dim=-1)
    C = A.amax(dim=-2)
    return R.amax(-1) / R.median(-1).values, C.amax(-1) / C.median(-1).values


def outlier_gains(w: Workload):
    """(row gain, column gain) chosen so that the median over sampled states of
    the row and column max/median ratios match the pages' 10.3x and 19.4x
    ([P5] 空间维度).  A few multiplicative fixed-point passes on a fixed sample."""
    if w.tiny_recipe:
        return 1.0, 1.0
    g = torch.Generator().manual_seed(12345)
    G = torch.randn(64, w.dk, w.dv, generator=g, dtype=torch.float64)
    rows = torch.stack([torch.randperm(w.dk, generator=g)[:N_OUTLIER_ROWS] for _ in range(64)])
    cols = torch.stack([torch.randperm(w.dv, generator=g)[:N_OUTLIER_COLS] for _ in range(64)])
    gr, gc = ROW_RATIO_TARGET, COL_RATIO_TARGET
    for _ in range(6):
        rg = torch.ones(64, w.dk, dtype=torch.float64)
        cg = torch.ones(64, w.dv, dtype=torch.float64)
        rg.scatter_(1, rows, gr)
        cg.scatter_(1, cols, gc)
        rr, cr = _ratios(G * rg[:, :, None] * cg[:, None, :])
        gr *= ROW_RATIO_TARGET / float(rr.median())
        gc *= COL_RATIO_TARGET / float(cr.median())
    return gr, gc


_GAIN_CACHE: dict = {}


def _gain_vectors(w: Workload, device="cpu"):
    key = (w.name, w.seed, w.n_heads, w.dk, w.dv, w.tiny_recipe, str(device))
    if key not in _GAIN_CACHE:
        _GAIN_CACHE[key] = _make_gain_vectors(w, device)
    return _GAIN_CACHE[key]


def _make_gain_vectors(w: Workload, device):
    rows, cols = outlier_positions(w)
    gr, gc = outlier_gains(w)
    rg = torch.ones(w.n_heads, w.dk, dtype=torch.float32)
    cg = torch.ones(w.n_heads, w.dv, dtype=torch.float32)
    rg.scatter_(1, torch.from_numpy(rows).long(), gr)
    cg.scatter_(1, torch.from_numpy(cols).long(), gc)
    return rg.to(device), cg.to(device)


# ------------------------------------------------------------------ states

def initial_state(w: Workload, req: int, device="cpu") -> torch.Tensor:
    """fp32 S0 for request `req`, [H][dk][dv].  tiny: N(0, 0.1^2).  Otherwise
    N(0, 0.5^2) times per-head row and column outlier gains."""
    gen = _torch_gen(w, 1000 + req, device)
    G = torch.randn(w.n_heads, w.dk, w.dv, generator=gen, device=device, dtype=torch.float32)
    if w.tiny_recipe:
        return G * 0.1
    rg, cg = _gain_vectors(w, device)
    return G * STATE_SIGMA * rg[:, :, None] * cg[:, None, :]


def scales(w: Workload, device="cpu", chunk: int = 8, bits=None):
    """Per-head row and column factors r[H][dk], c[H][dv] (fp32).

    tiny: r_i = 1 and c_j ~ LogUniform(0.5, 2) read as the column's range, so
    the column's step is c_j / 127.  Otherwise a two-pass max-abs over every
    request's S0 (a stand-in for the pages' offline fitting, [P5] 空间维度):
    r_i = max |S0_ij| over requests and columns, then
    c_j = max over requests and rows of |S0_ij| / r_i, divided by Q_b, so that
    no element of S0 exceeds the code range.  Pivot and FP32 heads get 1.
    `bits` overrides the workload's width table (e.g. a uniform comparator)."""
    bits = head_bits(w) if bits is None else np.asarray(bits, np.uint8)
    Qb = torch.tensor([(2 ** (int(b) - 1) - 1) if b <= 8 else 1 for b in bits], dtype=torch.float32)
    if w.tiny_recipe:
        rng = _rng(w, 3)
        r = np.ones((w.n_heads, w.dk), np.float32)
        c = np.exp(rng.uniform(math.log(0.5), math.log(2.0), (w.n_heads, w.dv))).astype(np.float32)
        c = c / Qb.numpy()[:, None]
        return torch.from_numpy(r).to(device), torch.from_numpy(c.astype(np.float32)).to(device)
    R = torch.zeros(w.n_heads, w.dk, device=device)
    for p0 in range(0, w.n_req, chunk):
        S = torch.stack([initial_state(w, p, device) for p in range(p0, min(w.n_req, p0 + chunk))])
        R = torch.maximum(R, S.abs().amax(dim=(0, 3)))
    C = torch.zeros(w.n_heads, w.dv, device=device)
    for p0 in range(0, w.n_req, chunk):
        S = torch.stack([initial_state(w, p, device) for p in range(p0, min(w.n_req, p0 + chunk))])
        C = torch.maximum(C, (S.abs() / R[None, :, :, None]).amax(dim=(0, 2)))
    c = C / Qb.to(device)[:, None]
    quant = torch.from_numpy(bits <= 8).to(device)
    r = torch.where(quant[:, None], R, torch.ones_like(R))
    c = torch.where(quant[:, None], c, torch.ones_like(c))
    return r.contiguous(), c.contiguous()


# ------------------------------------------------------------------ per step

@dataclass
class StepInputs:
    q: torch.Tensor      # [n_req][H][dk]  bf16 or f32
    k: torch.Tensor      # [n_req][H][dk]
    v: torch.Tensor      # [n_req][H][dv]
    alpha: torch.Tensor  # [n_req][H] f32
    beta: torch.Tensor   # [n_req][H] f32


def step_inputs(w: Workload, t: int, device="cpu") -> StepInputs:
    """Inputs of decode step t for every request of the batch.

    q, k ~ N(0, 1) normalised to unit length in fp32, then cast; v ~ N(0, 1).
    beta ~ U(beta_range).  tiny: alpha = exp(-softplus(a)), a ~ N(0, 1).
    Otherwise ln alpha = -(ln 2 / h) exp(0.5 z - 0.125), z ~ N(0, 1), with h the
    head's half-life: mean log-retention -ln2/h ([P5] 时间维度), alpha <= 1.
    drift: the outlier rows and columns are kept alive by scaling k's outlier
    rows and v's outlier columns by the state's gains ([P5] 空间维度)."""
    gen = _torch_gen(w, 10 + t, device)
    n, H = w.n_req, w.n_heads
    f32 = torch.float32
    q = torch.randn(n, H, w.dk, generator=gen, device=device, dtype=f32)
    k = torch.randn(n, H, w.dk, generator=gen, device=device, dtype=f32)
    v = torch.randn(n, H, w.dv, generator=gen, device=device, dtype=f32)
    if w.persistent_outliers:
        rg, cg = _gain_vectors(w, device)
        k = k * rg[None]
        v = v * cg[None]
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    lo, hi = w.beta_range
    beta = lo + (hi - lo) * torch.rand(n, H, generator=gen, device=device, dtype=f32)
    z = torch.randn(n, H, generator=gen, device=device, dtype=f32)
    if w.tiny_recipe:
        alpha = torch.exp(-torch.nn.functional.softplus(z))
    else:
        h = torch.from_numpy(half_lives(w).astype(np.float32)).to(device)
        alpha = torch.exp(-(math.log(2.0) / h)[None, :] * torch.exp(0.5 * z - 0.125))
    dt = torch.bfloat16 if w.qkv_dtype == "bf16" else f32
    return StepInputs(q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous(),
                      alpha.contiguous(), beta.contiguous())


def channel_gates(w: Workload, t: int, device="cpu") -> torch.Tensor:
    """Per-key-channel gates alpha [n_req][H][d_k] of decode step t, for the
    per-channel (KDA) step; q, k, v and beta come from step_inputs.

    tiny: alpha = exp(-softplus(a)), a ~ N(0, 1) per channel.  Otherwise
    ln alpha_i = -(ln 2 / h) exp(0.5 z + 0.5 z_i - 0.25), z ~ N(0, 1) per
    (request, head) and z_i ~ N(0, 1) per channel: every channel decays at its
    own rate around the head's half-life h, with the head's mean
    log-retention -ln2/h as in step_inputs ([P5] 时间维度)."""
    gen = _torch_gen(w, 1_000_000_000 + t, device)
    n, H = w.n_req, w.n_heads
    f32 = torch.float32
    zc = torch.randn(n, H, w.dk, generator=gen, device=device, dtype=f32)
    if w.tiny_recipe:
        return torch.exp(-torch.nn.functional.softplus(zc)).contiguous()
    z = torch.randn(n, H, 1, generator=gen, device=device, dtype=f32)
    h = torch.from_numpy(half_lives(w).astype(np.float32)).to(device)
    rate = (math.log(2.0) / h)[None, :, None]
    return torch.exp(-rate * torch.exp(0.5 * z + 0.5 * zc - 0.25)).contiguous()


def pool_stats(w: Workload) -> dict:
    """Sizes of the workload's pool and per-step traffic at the layout's tile sizes."""
    bits = head_bits(w)
    d2 = w.dk * w.dv
    tile = [d2 * field_width(b) // 8 for b in bits]
    slab = sum((t + 255) // 256 * 256 for t in tile)
    qkv_bytes = 2 if w.qkv_dtype == "bf16" else 4
    per_head_tok_io = qkv_bytes * (2 * w.dk + w.dv) + 8 + 4 * w.dv
    step_bytes = w.n_req * (2 * sum(tile) + w.n_heads * per_head_tok_io)
    return {"slab_bytes": slab, "pool_bytes": slab * w.n_req, "step_bytes": step_bytes,
            "fp32_pool_bytes": w.n_req * w.n_heads * d2 * 4,
            "mean_bits_nonpivot": float(np.mean([b for b in bits if b <= 8])) if (bits <= 8).any() else 0.0}
