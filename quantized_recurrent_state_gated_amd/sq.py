"""Python binding of libsq (include/sq.h): argument marshalling only.

Every function has the name and meaning of the C entry point it wraps.  Device
buffers are torch tensors on the GPU (PyTorch supplies device memory and
streams); the arithmetic runs in the library's HIP kernels.  Importing this
module loads ``libsq.so`` from the package directory and raises if it is
missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m quantized_recurrent_state_gated_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

SQ_OK, SQ_ERR_INVALID, SQ_ERR_UNSUPPORTED, SQ_ERR_HIP, SQ_ERR_NOMEM, SQ_ERR_DEVICE = 0, -1, -2, -3, -4, -5
SQ_F32, SQ_BF16 = 0, 1
EXPORTED = ("sq_pool_bytes", "sq_pool_alloc", "sq_pool_free", "sq_pool_tile_offset",
            "sq_pool_store", "sq_pool_load", "sq_decode_step", "sq_decode_step_kda", "sq_readout",
            "sq_check_slots", "sq_check_slots_noalloc", "sq_pool_last_device_error",
            "sq_status_string")


class SqPoolDesc(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("head_bits", ctypes.POINTER(ctypes.c_uint8)),
                ("row_scale", ctypes.c_void_p), ("col_scale", ctypes.c_void_p),
                ("scale_slot_stride", ctypes.c_int64),
                ("state", ctypes.c_void_p), ("state_bytes", ctypes.c_uint64)]


_vp, _i32 = ctypes.c_void_p, ctypes.c_int32
_lib.sq_pool_bytes.restype = ctypes.c_uint64
_lib.sq_pool_bytes.argtypes = [_i32, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_uint8)]
_lib.sq_pool_alloc.restype = ctypes.c_int
_lib.sq_pool_alloc.argtypes = [ctypes.POINTER(SqPoolDesc), ctypes.POINTER(_vp)]
_lib.sq_pool_free.restype = None
_lib.sq_pool_free.argtypes = [_vp]
_lib.sq_pool_tile_offset.restype = ctypes.c_int
_lib.sq_pool_tile_offset.argtypes = [_vp, _i32, _i32, ctypes.POINTER(ctypes.c_uint64),
                                     ctypes.POINTER(ctypes.c_uint64)]
_lib.sq_pool_store.restype = ctypes.c_int
_lib.sq_pool_store.argtypes = [_vp, _vp, _i32, _vp, _vp]
_lib.sq_pool_load.restype = ctypes.c_int
_lib.sq_pool_load.argtypes = [_vp, _vp, _i32, _vp, _vp]
_lib.sq_decode_step.restype = ctypes.c_int
_lib.sq_decode_step.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp]
_lib.sq_decode_step_kda.restype = ctypes.c_int
_lib.sq_decode_step_kda.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp]
_lib.sq_readout.restype = ctypes.c_int
_lib.sq_readout.argtypes = [_vp, _vp, _i32, _vp, _i32, _vp, _vp]
_lib.sq_check_slots.restype = ctypes.c_int
_lib.sq_check_slots.argtypes = [_vp, _vp, _i32, _vp, _vp]
_lib.sq_check_slots_noalloc.restype = ctypes.c_int
_lib.sq_check_slots_noalloc.argtypes = [_vp, _i32, _i32, _vp, _vp]
_lib.sq_pool_last_device_error.restype = ctypes.c_int
_lib.sq_pool_last_device_error.argtypes = [_vp, _vp]
_lib.sq_status_string.restype = ctypes.c_char_p
_lib.sq_status_string.argtypes = [ctypes.c_int]


class SqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {sq_status_string(status)} ({status})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != SQ_OK:
        raise SqError(status, where)


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SQ_BF16
    if t.dtype == torch.float32:
        return SQ_F32
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


_FLOATS = (torch.float32, torch.bfloat16)
_DEVICE_TYPES = ("cuda",)  # device types a tensor argument may live on


def _arg(x, where: str, name: str, dtypes, numel: int, optional: bool = False) -> None:
    """Host-side check of a device tensor argument: CUDA, contiguous, one of
    `dtypes`, `numel` elements.  A size mismatch is SQ_ERR_INVALID (as the
    library reports for sizes it can check), a wrong dtype a TypeError.  Raw
    integer pointers are passed through unchecked."""
    if x is None:
        if optional:
            return
        raise SqError(SQ_ERR_INVALID, f"{where} ({name} is required)")
    if isinstance(x, int):
        return
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{where}: {name} must be a torch tensor or a device pointer")
    if x.dtype not in dtypes:
        raise TypeError(f"{where}: {name} must be {' or '.join(str(d) for d in dtypes)}, got {x.dtype}")
    if x.numel() and x.device.type not in _DEVICE_TYPES:
        raise SqError(SQ_ERR_INVALID, f"{where} ({name} is not on a GPU)")
    if not x.is_contiguous():
        raise SqError(SQ_ERR_INVALID, f"{where} ({name} is not contiguous)")
    if x.numel() != numel:
        raise SqError(SQ_ERR_INVALID, f"{where} ({name} has {x.numel()} elements, expected {numel})")


def _bits_array(head_bits):
    hb = bytes(int(b) for b in head_bits)
    return (ctypes.c_uint8 * max(len(hb), 1)).from_buffer_copy(hb or b"\0"), len(hb)


def sq_check_slots(pool: SqPool, slot_ids, result, stream=None) -> None:
    """Write into the int32 device tensor `result` 0 for a valid batch, else
    1 (id out of range) | 2 (id repeated)."""
    n_req = 0 if slot_ids is None else int(slot_ids.numel())
    _arg(result, "sq_check_slots", "result", (torch.int32,), 1)
    _check(_lib.sq_check_slots(pool.handle, _ptr(slot_ids), n_req, _ptr(result), _stream(stream)),
           "sq_check_slots")


def sq_check_slots_noalloc(slot_ids, n_slots: int, result, stream=None) -> None:
    """sq_check_slots without a pool and without any allocation: the stamps
    live in a fixed array inside the library (n_slots <= SQ_CHECK_NOALLOC_MAX_SLOTS)."""
    n_req = 0 if slot_ids is None else int(slot_ids.numel())
    _arg(result, "sq_check_slots_noalloc", "result", (torch.int32,), 1)
    _check(_lib.sq_check_slots_noalloc(_ptr(slot_ids), n_req, int(n_slots), _ptr(result),
                                       _stream(stream)), "sq_check_slots_noalloc")


def sq_pool_last_device_error(pool: SqPool, stream=None) -> int:
    """Synchronize the stream, then read and clear the pool's sticky flag:
    SQ_OK, or SQ_ERR_DEVICE if a kernel met a non-finite updated value."""
    st = _lib.sq_pool_last_device_error(pool.handle, _stream(stream))
    if st not in (SQ_OK, SQ_ERR_DEVICE):
        _check(st, "sq_pool_last_device_error")
    return st


def sq_status_string(status: int) -> str:
    return _lib.sq_status_string(int(status)).decode()


def sq_pool_bytes(n_slots: int, n_heads: int, d_k: int, d_v: int, head_bits) -> int:
    arr, _ = _bits_array(head_bits)
    return int(_lib.sq_pool_bytes(n_slots, n_heads, d_k, d_v, arr))


class SqPool:
    """Owner of an sq_pool handle; keeps the borrowed tensors alive."""

    def __init__(self, handle: int, keep: tuple, n_slots: int, n_heads: int, d_k: int, d_v: int,
                 head_bits):
        self.handle = handle
        self._keep = keep
        self._free = _lib.sq_pool_free  # the library that made the handle releases it
        self.n_slots, self.n_heads, self.d_k, self.d_v = n_slots, n_heads, d_k, d_v
        self.head_bits = list(int(b) for b in head_bits)

    @property
    def state(self) -> torch.Tensor:
        return self._keep[0]

    def __del__(self):
        # also runs at interpreter exit, when module globals may already be gone
        handle, free = getattr(self, "handle", None), getattr(self, "_free", None)
        if handle and free is not None:
            try:
                free(handle)
            except Exception:
                pass
        self.handle = None


def sq_pool_alloc(n_slots: int, n_heads: int, d_k: int, d_v: int, head_bits, row_scale,
                  col_scale, state, state_bytes: int | None = None,
                  scale_slot_stride: int = 0) -> SqPool:
    """Wrap sq_pool_alloc; `state` is a uint8 device tensor (the caller's buffer).
    With scale_slot_stride S > 0 the factor tensors hold n_slots * S per-head
    vectors (slot p, head h at vector p * S + h)."""
    arr, nb = _bits_array(head_bits)
    vecs = n_slots * scale_slot_stride if scale_slot_stride > 0 else n_heads
    _arg(row_scale, "sq_pool_alloc", "row_scale", (torch.float32,), vecs * d_k)
    _arg(col_scale, "sq_pool_alloc", "col_scale", (torch.float32,), vecs * d_v)
    if isinstance(state, torch.Tensor):
        _arg(state, "sq_pool_alloc", "state", (state.dtype,), state.numel())
    if state_bytes is None:
        state_bytes = state.numel() * state.element_size() if hasattr(state, "numel") else 0
    desc = SqPoolDesc(n_slots, n_heads, d_k, d_v, arr, _ptr(row_scale), _ptr(col_scale),
                      int(scale_slot_stride), _ptr(state), int(state_bytes))
    h = _vp()
    _check(_lib.sq_pool_alloc(ctypes.byref(desc), ctypes.byref(h)), "sq_pool_alloc")
    return SqPool(h.value, (state, row_scale, col_scale), n_slots, n_heads, d_k, d_v,
                  list(head_bits)[:nb])


def sq_pool_free(pool: SqPool) -> None:
    if pool is not None and getattr(pool, "handle", None):
        pool._free(pool.handle)
        pool.handle = None


def sq_pool_tile_offset(pool: SqPool, slot: int, head: int):
    off, nb = ctypes.c_uint64(), ctypes.c_uint64()
    _check(_lib.sq_pool_tile_offset(pool.handle, slot, head, ctypes.byref(off), ctypes.byref(nb)),
           "sq_pool_tile_offset")
    return int(off.value), int(nb.value)


def _state_elems(pool: SqPool, n_req: int) -> int:
    return n_req * pool.n_heads * pool.d_k * pool.d_v


def sq_pool_store(pool: SqPool, slot_ids, S, stream=None) -> None:
    n_req = 0 if slot_ids is None else int(slot_ids.numel())
    if n_req:
        _arg(slot_ids, "sq_pool_store", "slot_ids", (torch.int32,), n_req)
        _arg(S, "sq_pool_store", "S", (torch.float32,), _state_elems(pool, n_req))
    _check(_lib.sq_pool_store(pool.handle, _ptr(slot_ids), n_req, _ptr(S), _stream(stream)),
           "sq_pool_store")


def sq_pool_load(pool: SqPool, slot_ids, S, stream=None) -> None:
    """Dequantize the slots' states into the fp32 device tensor S [n_req][H][dk][dv]."""
    n_req = 0 if slot_ids is None else int(slot_ids.numel())
    if n_req:
        _arg(slot_ids, "sq_pool_load", "slot_ids", (torch.int32,), n_req)
        _arg(S, "sq_pool_load", "S", (torch.float32,), _state_elems(pool, n_req))
    _check(_lib.sq_pool_load(pool.handle, _ptr(slot_ids), n_req, _ptr(S), _stream(stream)),
           "sq_pool_load")


def _step_args(where, pool, slot_ids, q, k, v, alpha, beta, o, alpha_per_channel):
    n_req = int(slot_ids.numel())
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError(f"{where}: q, k and v must share one dtype")
    H, dk, dv = pool.n_heads, pool.d_k, pool.d_v
    _arg(slot_ids, where, "slot_ids", (torch.int32,), n_req)
    _arg(q, where, "q", _FLOATS, n_req * H * dk)
    _arg(k, where, "k", _FLOATS, n_req * H * dk)
    _arg(v, where, "v", _FLOATS, n_req * H * dv)
    _arg(alpha, where, "alpha", (torch.float32,), n_req * H * (dk if alpha_per_channel else 1))
    _arg(beta, where, "beta", (torch.float32,), n_req * H)
    _arg(o, where, "o", (torch.float32,), n_req * H * dv, optional=True)
    return n_req


def sq_decode_step(pool: SqPool, slot_ids, q, k, v, alpha, beta, o=None, stream=None) -> None:
    n_req = _step_args("sq_decode_step", pool, slot_ids, q, k, v, alpha, beta, o, False)
    _check(_lib.sq_decode_step(pool.handle, _ptr(slot_ids), n_req, _ptr(q), _ptr(k), _ptr(v),
                               _dtype_code(q), _ptr(alpha), _ptr(beta), _ptr(o), _stream(stream)),
           "sq_decode_step")


def sq_decode_step_kda(pool: SqPool, slot_ids, q, k, v, alpha, beta, o=None, stream=None) -> None:
    """Per-key-channel-gate step; alpha is fp32 [n_req][n_heads][d_k]."""
    n_req = _step_args("sq_decode_step_kda", pool, slot_ids, q, k, v, alpha, beta, o, True)
    _check(_lib.sq_decode_step_kda(pool.handle, _ptr(slot_ids), n_req, _ptr(q), _ptr(k), _ptr(v),
                                   _dtype_code(q), _ptr(alpha), _ptr(beta), _ptr(o),
                                   _stream(stream)), "sq_decode_step_kda")


def sq_readout(pool: SqPool, slot_ids, q, o, stream=None) -> None:
    n_req = int(slot_ids.numel())
    _arg(slot_ids, "sq_readout", "slot_ids", (torch.int32,), n_req)
    _arg(q, "sq_readout", "q", _FLOATS, n_req * pool.n_heads * pool.d_k)
    _arg(o, "sq_readout", "o", (torch.float32,), n_req * pool.n_heads * pool.d_v)
    _check(_lib.sq_readout(pool.handle, _ptr(slot_ids), n_req, _ptr(q), _dtype_code(q), _ptr(o),
                           _stream(stream)), "sq_readout")
