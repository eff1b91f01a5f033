"""Helpers shared by the GPU parity tests: field unpacking (written here from
the state format's definition, independently of both the oracle and the HIP
library), tolerance checks, and pool set-up.

Tolerances (GPU fp32 arithmetic against the fp64 oracle, teacher-forced: the
oracle always starts from the GPU's own pre-step bytes):
  quantized codes  >= 99.99 % identical, every mismatch exactly +-1 code;
  FP16 pivots      |a - b| <= 1e-3 |b| + 2^-20 max|tile|: the stated 1e-3 relative
                   bound (one binary16 ulp is <= 2^-10 relative), plus an absolute
                   floor for elements that come out of cancellation between the
                   decay term and the key-direction term, whose fp32 evaluation
                   error is a few fp32 ulps of the tile's magnitude, not of the
                   (small) result;
  FP32 states      |a - b| <= 2e-6 * max|tile| (a few fp32 ulps of the tile);
  BF16 states      |a - b| <= 2^-7 |b| + 2^-16 max|tile|: one bfloat16 ulp (at most
                   2^-7 relative: fp32 evaluation order can move a value across a
                   rounding boundary) plus the same cancellation floor as pivots,
                   scaled to bfloat16's precision;
  readout o        per (request, head): max_j |o - o_ref| <= 1e-5 + 1e-3 max_j |o_ref|.
Non-finite values (FP16/BF16/FP32 elements, readouts) must be non-finite on both
sides in the same class (NaN, +Inf, -Inf); the NaN payload is not compared, and
the finite rest is held to the bars above.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from quantized_recurrent_state_gated_amd import inputs as I

ORACLE_THREADS = 16
CODE_MATCH_MIN = 0.9999
O_ATOL, O_RTOL = 1e-5, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def unpack_fields(tiles: np.ndarray, w: int) -> np.ndarray:
    """tiles: uint8 [n_tiles, tile_bytes] -> [n_tiles, n_fields], field n at
    bits [n*w, n*w+w) of each tile's little-endian bit stream (w = a head_bits
    value; the bfloat16 state has 16-bit fields).  Codes come back as uint8,
    16-bit fields as uint16, 32-bit fields as uint32."""
    w = I.field_width(w)
    tiles = np.ascontiguousarray(tiles, np.uint8)
    nt = tiles.shape[0]
    if w == 8:
        return tiles.copy()
    if w == 16:
        return tiles.view("<u2").reshape(nt, -1).astype(np.uint16)
    if w == 32:
        return tiles.view("<u4").reshape(nt, -1).astype(np.uint32)
    if w == 4:
        out = np.empty((nt, tiles.shape[1] * 2), np.uint8)
        out[:, 0::2] = tiles & 0xF
        out[:, 1::2] = tiles >> 4
        return out
    if w == 6:
        g = tiles.reshape(nt, -1, 3).astype(np.uint32)
        word = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
        out = np.stack([((word >> s) & 0x3F).astype(np.uint8) for s in (0, 6, 12, 18)], axis=-1)
        return out.reshape(nt, -1)
    raise ValueError(w)


def f16_order_key(h: np.ndarray) -> np.ndarray:
    h = h.astype(np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h)


class Tally:
    """Accumulates code/pivot/fp32/o comparisons over a run."""

    def __init__(self):
        self.codes = 0
        self.code_mismatch = 0
        self.code_maxdiff = 0
        self.pivot_vals = 0
        self.pivot_maxulp = 0
        self.pivot_worst = 0.0  # max of |a-b| / (1e-3 |b| + 2^-20 max|tile|)
        self.fp32_maxrel = 0.0
        self.bf16_vals = 0
        self.bf16_worst = 0.0  # max of |a-b| / (2^-7 |b| + 2^-16 max|tile|)
        self.o_worst = 0.0  # max over tiles of err / (atol + rtol * max|o_ref|)
        self.tiles = 0
        self.nonfinite = 0       # non-finite elements that matched in class
        self.nonfinite_bad = 0   # elements whose class (finite, NaN, +Inf, -Inf) differs

    def _split(self, fa, fb):
        """Count non-finite class agreement; return copies with those elements zeroed."""
        ca = np.where(np.isnan(fa), 1, np.where(np.isinf(fa), 2 + (fa > 0), 0))
        cb = np.where(np.isnan(fb), 1, np.where(np.isinf(fb), 2 + (fb > 0), 0))
        self.nonfinite_bad += int((ca != cb).sum())
        self.nonfinite += int(((ca == cb) & (cb != 0)).sum())
        keep = (ca == 0) & (cb == 0)
        return np.where(keep, fa, 0.0), np.where(keep, fb, 0.0), keep

    def add_tiles(self, gpu: np.ndarray, ref: np.ndarray, bits: int):
        """gpu, ref: uint8 [n_tiles, tile_bytes] of one width."""
        if gpu.shape[0] == 0:
            return
        self.tiles += gpu.shape[0]
        if bits <= 8:
            # a code tile whose bytes match is counted (every code equal)
            # without unpacking; only tiles with a differing byte are unpacked
            same = (gpu == ref).all(axis=1)
            self.codes += int(same.sum()) * (gpu.shape[1] * 8 // I.field_width(bits))
            if same.all():
                return
            gpu, ref = gpu[~same], ref[~same]
        a, b = unpack_fields(gpu, bits), unpack_fields(ref, bits)
        if bits <= 8:
            d = np.abs(a.astype(np.int16) - b.astype(np.int16))
            self.codes += d.size
            self.code_mismatch += int((d != 0).sum())
            self.code_maxdiff = max(self.code_maxdiff, int(d.max()))
        elif bits == I.BITS_BF16:
            fa = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            fb = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            fa, fb, _ = self._split(fa, fb)
            lim = 2.0 ** -7 * np.abs(fb) + 2.0 ** -16 * np.abs(fb).max(axis=1, keepdims=True)
            self.bf16_vals += fa.size
            self.bf16_worst = max(self.bf16_worst, float((np.abs(fa - fb) / np.maximum(lim, 1e-38)).max()))
        elif bits == 16:
            fa = a.astype(np.uint16).view(np.float16).astype(np.float64)
            fb = b.astype(np.uint16).view(np.float16).astype(np.float64)
            fa, fb, keep = self._split(fa, fb)
            d = np.where(keep, np.abs(f16_order_key(a) - f16_order_key(b)), 0)
            self.pivot_vals += d.size
            self.pivot_maxulp = max(self.pivot_maxulp, int(d.max()))
            lim = 1e-3 * np.abs(fb) + 2.0 ** -20 * np.abs(fb).max(axis=1, keepdims=True)
            lim = np.maximum(lim, 1e-300)
            self.pivot_worst = max(self.pivot_worst, float((np.abs(fa - fb) / lim).max()))
        else:
            fa, fb = a.view(np.float32).astype(np.float64), b.view(np.float32).astype(np.float64)
            fa, fb, _ = self._split(fa, fb)
            scale = np.maximum(np.abs(fb).max(axis=1, keepdims=True), 1e-30)
            self.fp32_maxrel = max(self.fp32_maxrel, float((np.abs(fa - fb) / scale).max()))

    def add_o(self, o_gpu: np.ndarray, o_ref: np.ndarray):
        """o arrays [..., dv].  A readout element that is non-finite on either side
        must be non-finite on both; its class is not compared (an infinite state
        column read by a mixed-sign query is NaN in one evaluation order and
        +-Inf in another)."""
        fa, fb = o_gpu.astype(np.float64), o_ref.astype(np.float64)
        na, nb = ~np.isfinite(fa), ~np.isfinite(fb)
        self.nonfinite_bad += int((na != nb).sum())
        self.nonfinite += int((na & nb).sum())
        o_gpu, o_ref = np.where(na | nb, 0.0, fa), np.where(na | nb, 0.0, fb)
        err = np.abs(o_gpu - o_ref).max(axis=-1)
        lim = O_ATOL + O_RTOL * np.abs(o_ref).max(axis=-1)
        self.o_worst = max(self.o_worst, float((err / lim).max()))

    def match_rate(self) -> float:
        return 1.0 - self.code_mismatch / self.codes if self.codes else 1.0

    def summary(self) -> str:
        return (f"tiles={self.tiles} codes={self.codes} mismatch={self.code_mismatch} "
                f"(match {100 * self.match_rate():.5f}%) maxdiff={self.code_maxdiff} "
                f"pivot_maxulp={self.pivot_maxulp} pivot_worst={self.pivot_worst:.3f} fp32_maxrel={self.fp32_maxrel:.2e} "
                f"bf16_worst={self.bf16_worst:.3f} "
                f"o_worst={self.o_worst:.3f} nonfinite={self.nonfinite} "
                f"nonfinite_bad={self.nonfinite_bad}")

    def check(self):
        assert self.code_maxdiff <= 1, self.summary()
        assert self.match_rate() >= CODE_MATCH_MIN, self.summary()
        assert self.pivot_worst <= 1.0, self.summary()
        assert self.fp32_maxrel <= 2e-6, self.summary()
        assert self.bf16_worst <= 1.0, self.summary()
        assert self.o_worst <= 1.0, self.summary()
        assert self.nonfinite_bad == 0, self.summary()


def compare_pools(tally: Tally, gpu_pool: np.ndarray, ref_pool: np.ndarray, head_bits, off, slab,
                  slots, dk, dv, slots_per_chunk: int = 1):
    """Compare the tiles of `slots` (all heads) of two host pool images, a few
    slots at a time (a full-size pool holds hundreds of thousands of tiles)."""
    head_bits = np.asarray(head_bits)
    slots = [int(p) for p in slots]
    widths = [(b, np.nonzero(head_bits == b)[0], dk * dv * I.field_width(b) // 8)
              for b in sorted(set(int(x) for x in head_bits))]
    for c0 in range(0, len(slots), slots_per_chunk):
        chunk = slots[c0:c0 + slots_per_chunk]
        for b, hs, tb in widths:
            idx = np.array([p * slab + off[h] for p in chunk for h in hs], np.int64)
            if idx.size == 0:
                continue
            sel = idx[:, None] + np.arange(tb)[None, :]
            tally.add_tiles(gpu_pool[sel], ref_pool[sel], b)


def compare_pools_fast(tally: Tally, gpu_pool: np.ndarray, ref_pool: np.ndarray, head_bits, off,
                       slab, slots, dk, dv):
    """compare_pools for whole pools: a code tile whose bytes are identical on
    both sides is counted (every code equal) without unpacking; only tiles
    with a differing byte, and every FP16/BF16/FP32 tile, are unpacked.
    Bytes outside the tiles (alignment padding) must be identical."""
    head_bits = np.asarray(head_bits)
    H = head_bits.size
    sizes = np.array([dk * dv * I.field_width(int(b)) // 8 for b in head_bits], np.int64)
    starts = np.asarray(off, np.int64)[:H]
    order = np.argsort(starts)
    st_sorted = starts[order]
    fields = dk * dv
    code_heads = head_bits <= 8
    for p in (int(x) for x in slots):
        a = gpu_pool[p * slab:(p + 1) * slab]
        b = ref_pool[p * slab:(p + 1) * slab]
        pos = np.flatnonzero(a != b)
        k = np.searchsorted(st_sorted, pos, side="right") - 1
        assert np.all(k >= 0), f"slot {p}: a byte before the first tile differs"
        hd = order[k]
        assert np.all(pos < starts[hd] + sizes[hd]), f"slot {p}: padding bytes differ"
        diff = np.zeros(H, bool)
        diff[np.unique(hd)] = True
        same = code_heads & ~diff
        tally.tiles += int(same.sum())
        tally.codes += int(same.sum()) * fields
        for bw in sorted(set(int(x) for x in head_bits)):
            hs = np.nonzero((head_bits == bw) & ~same)[0]
            if hs.size == 0:
                continue
            sel = starts[hs][:, None] + np.arange(int(sizes[hs[0]]))[None, :]
            tally.add_tiles(a[sel], b[sel], bw)


def host_f32(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy()


# ------------------------------------------------------------------ pools

def per_slot_scales(w, n_slots: int, stride: int, seed: int):
    """Factors for a pool with a scale slot stride: slot p, head h gets the
    head's own factors times a seeded per-slot, per-row (per-column) factor in
    [1, 1.5] (a step at least as coarse, so the initial state stays in range);
    vectors at p * stride + h, the unused ones (h >= H) filled with 1."""
    r0, c0 = I.scales(w)
    r0, c0 = r0.numpy().astype(np.float64), c0.numpy().astype(np.float64)
    rng = np.random.default_rng(seed)
    H = w.n_heads
    r = np.ones((n_slots * stride, w.dk), np.float32)
    c = np.ones((n_slots * stride, w.dv), np.float32)
    for p in range(n_slots):
        r[p * stride:p * stride + H] = r0 * rng.uniform(1.0, 1.5, (H, w.dk))
        c[p * stride:p * stride + H] = c0 * rng.uniform(1.0, 1.5, (H, w.dv))
    return r, c


class Case:
    """A pool on the GPU initialised from the oracle's quantize-and-store.
    With scale_stride S > 0 every slot has its own factors (per_slot_scales)."""

    def __init__(self, sq, orc, w, n_slots=None, slots=None, bits=None, scales=None, S0=None,
                 scale_stride: int = 0):
        self.sq, self.orc, self.w = sq, orc, w
        self.bits = np.asarray(I.head_bits(w) if bits is None else bits, np.uint8)
        H, dk, dv = w.n_heads, w.dk, w.dv
        self.n_slots = n_slots or w.n_req
        self.stride = int(scale_stride)
        if scales is None and self.stride:
            r, c = per_slot_scales(w, self.n_slots, self.stride, w.seed + 1000)
        elif scales is None:
            r, c = I.scales(w)
            r, c = r.numpy(), c.numpy()
        else:
            r, c = scales
        self.r, self.c = np.ascontiguousarray(r, np.float32), np.ascontiguousarray(c, np.float32)
        self.off, self.slab = orc.pool_layout(self.bits, dk, dv)
        self.slots = np.arange(w.n_req, dtype=np.int32) if slots is None else np.asarray(slots, np.int32)
        host = np.zeros(self.n_slots * self.slab, np.uint8)
        if S0 is None:
            S0 = torch.stack([I.initial_state(w, p) for p in range(w.n_req)]).numpy()
        self.S0 = np.ascontiguousarray(S0, np.float32)
        orc.store_pool(host, self.bits, dk, dv, self.r, self.c, self.slots, self.S0,
                       scale_stride=self.stride)
        self.dev = torch.from_numpy(host).cuda()
        self.rd = torch.from_numpy(self.r).cuda()
        self.cd = torch.from_numpy(self.c).cuda()
        self.pool = sq.sq_pool_alloc(self.n_slots, H, dk, dv, self.bits, self.rd, self.cd, self.dev,
                                     scale_slot_stride=self.stride)
        self.slots_d = torch.from_numpy(self.slots).cuda()

    def host(self):
        torch.cuda.synchronize()
        return self.dev.cpu().numpy()

    def inputs(self, t):
        return I.step_inputs(self.w, t)

    def step(self, si, want_o=True):
        w = self.w
        o = torch.empty(w.n_req, w.n_heads, w.dv, device="cuda") if want_o else None
        self.sq.sq_decode_step(self.pool, self.slots_d, si.q.cuda(), si.k.cuda(), si.v.cuda(),
                               si.alpha.cuda(), si.beta.cuda(), o)
        return o

    def oracle_step(self, pre, si, return_flagged=False):
        ref = pre.copy()
        res = self.orc.step_pool(ref, self.bits, self.w.dk, self.w.dv, self.r, self.c, self.slots,
                                 host_f32(si.q), host_f32(si.k), host_f32(si.v),
                                 host_f32(si.alpha), host_f32(si.beta), n_threads=ORACLE_THREADS,
                                 scale_stride=self.stride, return_flagged=return_flagged)
        return (ref, *res) if return_flagged else (ref, res)

    def compare(self, tally, post, ref):
        compare_pools(tally, post, ref, self.bits, self.off, self.slab, self.slots, self.w.dk,
                      self.w.dv)


def run_teacher_forced(case, steps, label, check_changes=True):
    tally = Tally()
    changed = 0
    for t in range(steps):
        si = case.inputs(t)
        pre = case.host()
        o = case.step(si)
        post = case.host()
        ref, o_ref = case.oracle_step(pre, si)
        case.compare(tally, post, ref)
        tally.add_o(o.cpu().numpy(), o_ref)
        changed += int((post != pre).any())
        if t % 32 == 0 or t == steps - 1:
            say(f"[{label}] step {t}: {tally.summary()}")
    tally.check()
    if check_changes:
        assert changed == steps  # every step moved the state
    return tally


class KdaCase(Case):
    """A Case stepped with the per-key-channel gate: alpha is [n_req][H][d_k]."""

    def inputs(self, t):
        si = I.step_inputs(self.w, t)
        si.alpha = I.channel_gates(self.w, t)
        return si

    def step(self, si, want_o=True):
        w = self.w
        o = torch.empty(w.n_req, w.n_heads, w.dv, device="cuda") if want_o else None
        self.sq.sq_decode_step_kda(self.pool, self.slots_d, si.q.cuda(), si.k.cuda(), si.v.cuda(),
                                   si.alpha.cuda(), si.beta.cuda(), o)
        return o

    def oracle_step(self, pre, si, return_flagged=False):
        ref = pre.copy()
        res = self.orc.step_pool_kda(ref, self.bits, self.w.dk, self.w.dv, self.r, self.c,
                                     self.slots, host_f32(si.q), host_f32(si.k), host_f32(si.v),
                                     host_f32(si.alpha), host_f32(si.beta),
                                     n_threads=ORACLE_THREADS, scale_stride=self.stride,
                                     return_flagged=return_flagged)
        return (ref, *res) if return_flagged else (ref, res)
