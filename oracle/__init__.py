"""CPU oracle for the quantized gated delta-rule decode step (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does.

This module is a thin numpy/ctypes wrapper over ``sq_oracle.c``; every piece
of arithmetic lives in the C file, which documents the definitions it follows:

* [P1] "K1 論文詳解" (k1-news, 2026-10-09), STEPQuant article, section 方法.
* [P5] "线性注意力状态量化难题:Qwen状态池70并发就超模型权重" (aitest123),
  sections 直接量化为什么会翻车, 时间维度, 空间维度.

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: exhaustive packing round trips, the quantizer's error bound, numpy's
binary16 conversion, an fp64 dense-matrix recurrence, exact rational
arithmetic on a tiny case, and the closed-form invariants of the delta rule.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# tests/test_oracle_mutants.py points child test runs at deliberately broken
# builds through SQ_ORACLE_LIB; nothing else sets it
_LIB_PATH = os.environ.get("SQ_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # noqa: F401  (oracle/build.py)
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_f32_to_f16_array": (None, [_f32p, _u16p, ctypes.c_long]),
        "orc_f16_to_f32_array": (None, [_u16p, _f32p, ctypes.c_long]),
        "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_f32_to_bf16_array": (None, [_f32p, _u16p, ctypes.c_long]),
        "orc_bf16_to_f32_array": (None, [_u16p, _f32p, ctypes.c_long]),
        "orc_elem_index": (ctypes.c_long, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "orc_field_width": (ctypes.c_int, [ctypes.c_int]),
        "orc_tile_bytes": (ctypes.c_long, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "orc_field_get": (ctypes.c_uint32, [_u8p, ctypes.c_int, ctypes.c_long]),
        "orc_field_put": (None, [_u8p, ctypes.c_int, ctypes.c_long, ctypes.c_uint32]),
        "orc_pool_layout": (ctypes.c_long, [ctypes.c_int, _u8p, ctypes.c_int, ctypes.c_int, _i64p]),
        "orc_step_size": (ctypes.c_double, [ctypes.c_float, ctypes.c_float]),
        "orc_decode_field": (ctypes.c_double, [ctypes.c_int, ctypes.c_uint32, ctypes.c_double]),
        "orc_quantize": (ctypes.c_int, [ctypes.c_int, ctypes.c_double, ctypes.c_double]),
        "orc_encode_field": (ctypes.c_uint32, [ctypes.c_int, ctypes.c_double, ctypes.c_double]),
        "orc_decode_tile": (None, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, _f32p, _f32p, _f64p]),
        "orc_nonfinite_field": (ctypes.c_int, [ctypes.c_int, ctypes.c_double, ctypes.c_double]),
        "orc_encode_tile": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p, _f32p, _f32p, _u8p]),
        "orc_step_tile": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, _f32p, _f32p,
                                 _f32p, _f32p, _f32p, ctypes.c_float, ctypes.c_float, _f32p]),
        "orc_readout_tile": (None, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, _f32p, _f32p,
                                    _f32p, _f32p]),
        "orc_step_pool": (ctypes.c_long, [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, _f32p,
                                          _f32p, ctypes.c_long, _i32p, ctypes.c_int, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p,
                                 ctypes.c_int]),
        "orc_readout_pool": (None, [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, _f32p,
                                    _f32p, ctypes.c_long, _i32p, ctypes.c_int, _f32p, _f32p, ctypes.c_int]),
        "orc_store_pool": (ctypes.c_long, [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p,
                                           _f32p, _f32p, ctypes.c_long, _i32p, ctypes.c_int, _f32p]),
        "orc_load_pool": (None, [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, _f32p,
                                 _f32p, ctypes.c_long, _i32p, ctypes.c_int, _f32p]),
        "orc_step_tile_kda": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, _f32p, _f32p,
                                     _f32p, _f32p, _f32p, _f32p, ctypes.c_float, _f32p]),
        "orc_step_pool_kda": (ctypes.c_long, [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p,
                                              _f32p, _f32p, ctypes.c_long, _i32p, ctypes.c_int, _f32p, _f32p, _f32p, _f32p, _f32p,
                                     _f32p, ctypes.c_int]),
        "orc_bruteforce_kda": (None, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p, _f64p, _f64p,
                                      _f64p, _f64p, _f64p, _f64p, _f64p]),
        "orc_bruteforce": (None, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p, _f64p, _f64p,
                                  _f64p, _f64p, _f64p, _f64p, _f64p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a: np.ndarray, ptype):
    return a.ctypes.data_as(ptype)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


# ---------------------------------------------------------------- formats

def f32_to_f16_bits(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().orc_f32_to_f16_array(_p(x, _f32p), _p(out, _u16p), x.size)
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().orc_f16_to_f32_array(_p(h, _u16p), _p(out, _f32p), h.size)
    return out


BITS_BF16 = 144  # head_bits value of a bfloat16 state (16-bit fields)


def f32_to_bf16_bits(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().orc_f32_to_bf16_array(_p(x, _f32p), _p(out, _u16p), x.size)
    return out


def bf16_bits_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().orc_bf16_to_f32_array(_p(h, _u16p), _p(out, _f32p), h.size)
    return out


def elem_index(i: int, j: int, dv: int) -> int:
    return int(_load().orc_elem_index(i, j, dv))


def field_width(bits: int) -> int:
    return int(_load().orc_field_width(bits))


def tile_bytes(bits: int, dk: int, dv: int) -> int:
    return int(_load().orc_tile_bytes(bits, dk, dv))


def field_get(tile: np.ndarray, w: int, n: int) -> int:
    assert tile.dtype == np.uint8 and tile.flags.c_contiguous
    return int(_load().orc_field_get(_p(tile, _u8p), w, n))


def field_put(tile: np.ndarray, w: int, n: int, value: int) -> None:
    assert tile.dtype == np.uint8 and tile.flags.c_contiguous
    _load().orc_field_put(_p(tile, _u8p), w, n, value)


def pool_layout(head_bits, dk: int, dv: int):
    """Return (tile offsets int64[H], slab bytes)."""
    hb = _c(head_bits, np.uint8)
    off = np.zeros(max(hb.size, 1), np.int64)
    slab = _load().orc_pool_layout(hb.size, _p(hb, _u8p), dk, dv, _p(off, _i64p))
    return off[: hb.size], int(slab)


def step_size(r: float, c: float) -> float:
    return float(_load().orc_step_size(r, c))


def quantize(bits: int, x: float, s: float) -> int:
    return int(_load().orc_quantize(bits, x, s))


def encode_field(bits: int, x: float, s: float) -> int:
    return int(_load().orc_encode_field(bits, x, s))


def decode_field(bits: int, f: int, s: float) -> float:
    return float(_load().orc_decode_field(bits, f, s))


def nonfinite_field(bits: int, x: float, s: float) -> bool:
    """Is the value a field is decided on (fl32(x/s) for a code, fl32(x) else) not finite?"""
    return bool(_load().orc_nonfinite_field(bits, x, s))


# ---------------------------------------------------------------- tiles

def decode_tile(bits: int, dk: int, dv: int, tile, r, c) -> np.ndarray:
    tile = _c(tile, np.uint8)
    r, c = _c(r, np.float32), _c(c, np.float32)
    S = np.empty((dk, dv), np.float64)
    _load().orc_decode_tile(bits, dk, dv, _p(tile, _u8p), _p(r, _f32p), _p(c, _f32p), _p(S, _f64p))
    return S


def encode_tile(bits: int, dk: int, dv: int, S, r, c, return_flag: bool = False):
    """Packed tile of S; with return_flag, (tile, whether a stored-from value was non-finite)."""
    S = _c(S, np.float64)
    r, c = _c(r, np.float32), _c(c, np.float32)
    tile = np.zeros(tile_bytes(bits, dk, dv), np.uint8)
    bad = _load().orc_encode_tile(bits, dk, dv, _p(S, _f64p), _p(r, _f32p), _p(c, _f32p),
                                  _p(tile, _u8p))
    return (tile, bool(bad)) if return_flag else tile


def step_tile(bits: int, dk: int, dv: int, tile, r, c, q, k, v, alpha: float, beta: float,
              return_flag: bool = False):
    """Return (new tile bytes, o float32[dv]) and, with return_flag, whether the step
    met a non-finite value; the input tile is not modified."""
    tile = _c(tile, np.uint8).copy()
    r, c = _c(r, np.float32), _c(c, np.float32)
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    o = np.empty(dv, np.float32)
    bad = _load().orc_step_tile(bits, dk, dv, _p(tile, _u8p), _p(r, _f32p), _p(c, _f32p),
                                _p(q, _f32p), _p(k, _f32p), _p(v, _f32p), float(alpha),
                                float(beta), _p(o, _f32p))
    return (tile, o, bool(bad)) if return_flag else (tile, o)


def readout_tile(bits: int, dk: int, dv: int, tile, r, c, q) -> np.ndarray:
    tile = _c(tile, np.uint8)
    r, c, q = _c(r, np.float32), _c(c, np.float32), _c(q, np.float32)
    o = np.empty(dv, np.float32)
    _load().orc_readout_tile(bits, dk, dv, _p(tile, _u8p), _p(r, _f32p), _p(c, _f32p),
                             _p(q, _f32p), _p(o, _f32p))
    return o


# ---------------------------------------------------------------- pools

def _threads(n_threads):
    if n_threads is None:
        n_threads = len(os.sched_getaffinity(0))
    return int(n_threads)


def _check_factors(r, c, H, dk, dv, sid, scale_stride):
    """Factors of slot p, head h sit at r[(p*S + h)*dk] (S = scale_stride; 0 = shared)."""
    S = int(scale_stride)
    assert S == 0 or S >= H
    top = 0 if (S == 0 or sid.size == 0) else int(sid.max()) * S
    assert r.size >= (top + H) * dk and c.size >= (top + H) * dv
    return S


def _check_slots(hb, dk, dv, sid, pool):
    _, slab = pool_layout(hb, dk, dv)
    assert sid.size == 0 or (sid.min() >= 0 and (int(sid.max()) + 1) * slab <= pool.size)


def step_pool(pool: np.ndarray, head_bits, dk: int, dv: int, r, c, slot_ids, q, k, v, alpha, beta,
              want_o: bool = True, n_threads=None, scale_stride: int = 0,
              return_flagged: bool = False):
    """Advance the pool in place by one step; return o float32[n_req][H][dv] (or None),
    and with return_flagged also the number of tiles that met a non-finite value."""
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    hb = _c(head_bits, np.uint8)
    H = hb.size
    sid = _c(slot_ids, np.int32)
    n_req = sid.size
    r, c = _c(r, np.float32), _c(c, np.float32)
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    alpha, beta = _c(alpha, np.float32), _c(beta, np.float32)
    assert q.size == n_req * H * dk and k.size == n_req * H * dk and v.size == n_req * H * dv
    assert alpha.size == n_req * H and beta.size == n_req * H
    S = _check_factors(r, c, H, dk, dv, sid, scale_stride)
    _check_slots(hb, dk, dv, sid, pool)
    o = np.empty((n_req, H, dv), np.float32) if want_o else None
    bad = _load().orc_step_pool(_p(pool, _u8p), H, dk, dv, _p(hb, _u8p), _p(r, _f32p),
                                _p(c, _f32p), S, _p(sid, _i32p), n_req, _p(q, _f32p),
                                _p(k, _f32p), _p(v, _f32p), _p(alpha, _f32p), _p(beta, _f32p),
                                _p(o, _f32p) if want_o else None, _threads(n_threads))
    return (o, int(bad)) if return_flagged else o


def readout_pool(pool: np.ndarray, head_bits, dk: int, dv: int, r, c, slot_ids, q, n_threads=None,
                 scale_stride: int = 0):
    pool = _c(pool, np.uint8)
    hb = _c(head_bits, np.uint8)
    H = hb.size
    sid = _c(slot_ids, np.int32)
    n_req = sid.size
    r, c, q = _c(r, np.float32), _c(c, np.float32), _c(q, np.float32)
    S = _check_factors(r, c, H, dk, dv, sid, scale_stride)
    _check_slots(hb, dk, dv, sid, pool)
    o = np.empty((n_req, H, dv), np.float32)
    _load().orc_readout_pool(_p(pool, _u8p), H, dk, dv, _p(hb, _u8p), _p(r, _f32p), _p(c, _f32p),
                             S, _p(sid, _i32p), n_req, _p(q, _f32p), _p(o, _f32p),
                             _threads(n_threads))
    return o


def store_pool(pool: np.ndarray, head_bits, dk: int, dv: int, r, c, slot_ids, S,
               scale_stride: int = 0) -> int:
    """Quantize fp32 states S[n_req][H][dk][dv] into the slots' tiles (in place);
    return the number of tiles that stored a value from a non-finite one."""
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    hb = _c(head_bits, np.uint8)
    sid = _c(slot_ids, np.int32)
    r, c, S = _c(r, np.float32), _c(c, np.float32), _c(S, np.float32)
    assert S.size == sid.size * hb.size * dk * dv
    st = _check_factors(r, c, hb.size, dk, dv, sid, scale_stride)
    _check_slots(hb, dk, dv, sid, pool)
    return int(_load().orc_store_pool(_p(pool, _u8p), hb.size, dk, dv, _p(hb, _u8p), _p(r, _f32p),
                                      _p(c, _f32p), st, _p(sid, _i32p), sid.size, _p(S, _f32p)))


def load_pool(pool: np.ndarray, head_bits, dk: int, dv: int, r, c, slot_ids,
              scale_stride: int = 0) -> np.ndarray:
    """Decoded fp32 states S[n_req][H][dk][dv] of the slots' tiles."""
    pool = _c(pool, np.uint8)
    hb = _c(head_bits, np.uint8)
    sid = _c(slot_ids, np.int32)
    r, c = _c(r, np.float32), _c(c, np.float32)
    st = _check_factors(r, c, hb.size, dk, dv, sid, scale_stride)
    _check_slots(hb, dk, dv, sid, pool)
    S = np.empty((sid.size, hb.size, dk, dv), np.float32)
    _load().orc_load_pool(_p(pool, _u8p), hb.size, dk, dv, _p(hb, _u8p), _p(r, _f32p),
                          _p(c, _f32p), st, _p(sid, _i32p), sid.size, _p(S, _f32p))
    return S


def bruteforce(S0, q, k, v, alpha, beta):
    """Dense fp64 recurrence; return (S_T, o[T][dv])."""
    S0 = _c(S0, np.float64)
    dk, dv = S0.shape
    q, k, v = _c(q, np.float64), _c(k, np.float64), _c(v, np.float64)
    alpha, beta = _c(alpha, np.float64), _c(beta, np.float64)
    T = alpha.size
    ST = np.empty((dk, dv), np.float64)
    o = np.empty((T, dv), np.float64)
    _load().orc_bruteforce(dk, dv, T, _p(S0, _f64p), _p(q, _f64p), _p(k, _f64p), _p(v, _f64p),
                           _p(alpha, _f64p), _p(beta, _f64p), _p(ST, _f64p), _p(o, _f64p))
    return ST, o


# ---------------------------------------------------------------- per-channel gate

def step_tile_kda(bits: int, dk: int, dv: int, tile, r, c, q, k, v, alpha, beta: float,
                  return_flag: bool = False):
    """Per-channel-gate step (alpha float32[dk]); returns (new tile, o) [, flag]."""
    tile = _c(tile, np.uint8).copy()
    r, c = _c(r, np.float32), _c(c, np.float32)
    q, k, v, a = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32), _c(alpha, np.float32)
    o = np.empty(dv, np.float32)
    bad = _load().orc_step_tile_kda(bits, dk, dv, _p(tile, _u8p), _p(r, _f32p), _p(c, _f32p),
                                    _p(q, _f32p), _p(k, _f32p), _p(v, _f32p), _p(a, _f32p),
                                    float(beta), _p(o, _f32p))
    return (tile, o, bool(bad)) if return_flag else (tile, o)


def step_pool_kda(pool: np.ndarray, head_bits, dk: int, dv: int, r, c, slot_ids, q, k, v, alpha,
                  beta, want_o: bool = True, n_threads=None, scale_stride: int = 0,
                  return_flagged: bool = False):
    """Per-channel-gate pool step in place (alpha float32 [n_req][H][dk]); returns o or
    None, and with return_flagged also the number of tiles that met a non-finite value."""
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    hb = _c(head_bits, np.uint8)
    H = hb.size
    sid = _c(slot_ids, np.int32)
    n_req = sid.size
    r, c = _c(r, np.float32), _c(c, np.float32)
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    alpha, beta = _c(alpha, np.float32), _c(beta, np.float32)
    assert q.size == n_req * H * dk and k.size == n_req * H * dk and v.size == n_req * H * dv
    assert alpha.size == n_req * H * dk and beta.size == n_req * H
    S = _check_factors(r, c, H, dk, dv, sid, scale_stride)
    _check_slots(hb, dk, dv, sid, pool)
    o = np.empty((n_req, H, dv), np.float32) if want_o else None
    bad = _load().orc_step_pool_kda(_p(pool, _u8p), H, dk, dv, _p(hb, _u8p), _p(r, _f32p),
                                    _p(c, _f32p), S, _p(sid, _i32p), n_req, _p(q, _f32p),
                                    _p(k, _f32p), _p(v, _f32p), _p(alpha, _f32p), _p(beta, _f32p),
                                    _p(o, _f32p) if want_o else None, _threads(n_threads))
    return (o, int(bad)) if return_flagged else o


def bruteforce_kda(S0, q, k, v, alpha, beta):
    """Dense fp64 per-channel-gate recurrence; alpha [T][dk].  Returns (S_T, o[T][dv])."""
    S0 = _c(S0, np.float64)
    dk, dv = S0.shape
    q, k, v = _c(q, np.float64), _c(k, np.float64), _c(v, np.float64)
    alpha, beta = _c(alpha, np.float64), _c(beta, np.float64)
    T = beta.size
    ST = np.empty((dk, dv), np.float64)
    o = np.empty((T, dv), np.float64)
    _load().orc_bruteforce_kda(dk, dv, T, _p(S0, _f64p), _p(q, _f64p), _p(k, _f64p), _p(v, _f64p),
                               _p(alpha, _f64p), _p(beta, _f64p), _p(ST, _f64p), _p(o, _f64p))
    return ST, o
