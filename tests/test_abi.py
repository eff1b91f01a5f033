"""The C-ABI library: it loads, exports every entry point include/sq.h
declares, computes pool sizes as the state format defines them, and rejects
bad arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sq.h")


@pytest.fixture(scope="module")
def sq():
    from quantized_recurrent_state_gated_amd import sq as m
    return m


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sq_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_names(sq):
    assert _declared() == sorted(sq.EXPORTED)


def test_library_exports_every_declared_symbol(sq):
    lib = ctypes.CDLL(sq.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_pool_bytes_matches_state_format(sq, orc):
    for bits, dk, dv in [([4, 6, 8, 16, 32], 128, 128), ([8] * 4, 16, 16), ([6, 4], 12, 20),
                         ([4], 4, 4), ([16, 6], 256, 128), ([144, 4, 32], 128, 128)]:
        _, slab = orc.pool_layout(bits, dk, dv)
        assert sq.sq_pool_bytes(3, len(bits), dk, dv, bits) == 3 * slab
    # serving shape: 70 x 2304 heads at 568/1136/568 + 32 pivots
    bits = [4] * 568 + [6] * 1136 + [8] * 568 + [16] * 32
    assert sq.sq_pool_bytes(70, 2304, 128, 128, bits) == 2027683840


@pytest.mark.parametrize("args", [
    (0, 1, 16, 16, [8]), (1, 0, 16, 16, []), (1, 1, 16, 16, [5]), (1, 1, 16, 16, [12]),
    (1, 1, 18, 16, [8]), (1, 1, 16, 0, [8]), (1, 1, 512, 16, [8]), (1, 2, 16, 16, [8, 7]),
])
def test_pool_bytes_rejects_bad_shapes(sq, args):
    assert sq.sq_pool_bytes(*args) == 0


def _desc(sq, **kw):
    bits = kw.pop("bits", [8, 4])
    arr = (ctypes.c_uint8 * len(bits))(*bits)
    d = dict(n_slots=2, n_heads=len(bits), d_k=16, d_v=16, head_bits=arr, row_scale=0x10000,
             col_scale=0x20000, state=0x100000, state_bytes=1 << 20)
    d.update(kw)
    return sq.SqPoolDesc(**d), arr


@pytest.mark.parametrize("kw,status", [
    (dict(n_slots=0), -1), (dict(n_heads=0), -1), (dict(state=None), -1), (dict(state=0x100010), -1),
    (dict(row_scale=None), -1), (dict(col_scale=0x20004), -1), (dict(state_bytes=100), -1),
    (dict(bits=[8, 3]), -2), (dict(d_k=18), -2), (dict(d_v=260), -2),
    (dict(scale_slot_stride=1), -1), (dict(scale_slot_stride=-2), -1),
])
def test_pool_alloc_validates_before_any_hip_call(sq, kw, status):
    desc, keep = _desc(sq, **kw)
    h = ctypes.c_void_p()
    assert sq._lib.sq_pool_alloc(ctypes.byref(desc), ctypes.byref(h)) == status
    assert not h.value


@pytest.mark.parametrize("value", ["fast", "GENERIC", "tuned ", "1"])
def test_unknown_kernel_switch_is_rejected_before_any_hip_call(sq, value, monkeypatch):
    """SQ_KERNEL names a kernel family; a value that names none fails the
    allocation (host-side, so it is checked here without a GPU)."""
    monkeypatch.setenv("SQ_KERNEL", value)
    desc, keep = _desc(sq)
    h = ctypes.c_void_p()
    assert sq._lib.sq_pool_alloc(ctypes.byref(desc), ctypes.byref(h)) == sq.SQ_ERR_INVALID
    assert not h.value


def test_null_handles_and_status_strings(sq):
    assert sq._lib.sq_pool_alloc(None, None) == sq.SQ_ERR_INVALID
    sq._lib.sq_pool_free(None)
    assert sq._lib.sq_decode_step(None, None, 1, None, None, None, 0, None, None, None, None) == -1
    assert sq._lib.sq_decode_step_kda(None, None, 1, None, None, None, 0, None, None, None,
                                      None) == -1
    assert sq._lib.sq_readout(None, None, 1, None, 0, None, None) == -1
    assert sq._lib.sq_check_slots(None, None, 0, None, None) == -1
    assert sq._lib.sq_pool_store(None, None, 1, None, None) == -1
    off = ctypes.c_uint64()
    assert sq._lib.sq_pool_tile_offset(None, 0, 0, ctypes.byref(off), ctypes.byref(off)) == -1
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(sq.sq_status_string(s), str) and sq.sq_status_string(s)
    assert sq.sq_status_string(-2) != sq.sq_status_string(-1)


def test_pool_bytes_reports_64_bit_overflow_as_invalid(sq):
    H = 1 << 20
    bits = [32] * H  # 1 Mi FP32 heads of 256 x 256: 2^38 bytes per slot
    assert sq.sq_pool_bytes(1, H, 256, 256, bits) == 1 << 38
    assert sq.sq_pool_bytes((1 << 25) - 1, H, 256, 256, bits) == ((1 << 25) - 1) << 38
    assert sq.sq_pool_bytes(1 << 26, H, 256, 256, bits) == 0  # 2^64 does not fit
    assert sq.sq_pool_bytes(2 ** 31 - 1, H, 256, 256, bits) == 0


def test_header_compiles_as_plain_c(tmp_path):
    """include/sq.h is a C header: a C99 translation unit using every entry
    point compiles without C++."""
    import subprocess
    src = tmp_path / "use.c"
    names = _declared()
    src.write_text('#include "sq.h"\ntypedef void (*fn)(void);\nfn table[] = {' +
                   ", ".join(f"(fn){n}" for n in names) +
                   "};\nint main(void) { return SQ_OK + SQ_F32 + SQ_BITS_BF16 - 144; }\n")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                        f"-I{os.path.join(ROOT, 'include')}", str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


class _FakePool:
    """Shape-only stand-in: the binding's argument checks run before the
    library sees the handle, so a CPU test never reaches a HIP call.  The
    tensors live on torch's "meta" device, admitted for these tests only."""
    handle, n_heads, d_k, d_v = None, 3, 8, 12


@pytest.mark.parametrize("bad, err", [
    (dict(q="cpu"), "not on a GPU"),
    (dict(alpha="f64"), "alpha must be"),
    (dict(beta="short"), "beta has"),
    (dict(slot_ids="i64"), "slot_ids must be"),
    (dict(o="bf16"), "o must be"),
    (dict(v="strided"), "v is not contiguous"),
    (dict(k="f16"), "share one dtype"),
])
def test_binding_checks_tensor_arguments(sq, bad, err, monkeypatch):
    import torch
    monkeypatch.setattr(sq, "_DEVICE_TYPES", ("cuda", "meta"))
    p, n = _FakePool, 2
    meta = torch.device("meta")
    args = dict(slot_ids=torch.zeros(n, dtype=torch.int32, device=meta),
                q=torch.zeros(n, p.n_heads, p.d_k, device=meta),
                k=torch.zeros(n, p.n_heads, p.d_k, device=meta),
                v=torch.zeros(n, p.n_heads, p.d_v, device=meta),
                alpha=torch.zeros(n, p.n_heads, device=meta),
                beta=torch.zeros(n, p.n_heads, device=meta),
                o=torch.zeros(n, p.n_heads, p.d_v, device=meta))
    which, how = next(iter(bad.items()))
    x = args[which]
    args[which] = {"cpu": lambda: torch.zeros(x.shape, dtype=x.dtype),
                   "f64": lambda: x.double(),
                   "short": lambda: x[:1],
                   "i64": lambda: x.long(),
                   "bf16": lambda: x.bfloat16(),
                   "strided": lambda: torch.zeros(n, p.n_heads, 2 * p.d_v, device=meta)[..., ::2],
                   "f16": lambda: x.half()}[how]()
    with pytest.raises((sq.SqError, TypeError), match=err):
        sq.sq_decode_step(p, **args)


def test_binding_checks_per_channel_gate_shape(sq, monkeypatch):
    import torch
    monkeypatch.setattr(sq, "_DEVICE_TYPES", ("cuda", "meta"))
    p, n, meta = _FakePool, 2, torch.device("meta")
    q = torch.zeros(n, p.n_heads, p.d_k, device=meta)
    v = torch.zeros(n, p.n_heads, p.d_v, device=meta)
    ids = torch.zeros(n, dtype=torch.int32, device=meta)
    beta = torch.zeros(n, p.n_heads, device=meta)
    with pytest.raises(sq.SqError, match="alpha has 6 elements, expected 48"):
        sq.sq_decode_step_kda(p, ids, q, q, v, torch.zeros(n, p.n_heads, device=meta), beta)


def test_binding_checks_pool_alloc_scales(sq, monkeypatch):
    import torch
    monkeypatch.setattr(sq, "_DEVICE_TYPES", ("cuda", "meta"))
    meta = torch.device("meta")
    state = torch.empty(1 << 16, dtype=torch.uint8, device=meta)
    r = torch.ones(2, 16, device=meta)
    with pytest.raises(TypeError, match="row_scale must be"):
        sq.sq_pool_alloc(2, 2, 16, 16, [8, 4], r.double(), r, state)
    with pytest.raises(sq.SqError, match="col_scale has 16 elements, expected 32"):
        sq.sq_pool_alloc(2, 2, 16, 16, [8, 4], r, r[0], state)
    with pytest.raises(sq.SqError, match="row_scale is not on a GPU"):
        sq.sq_pool_alloc(2, 2, 16, 16, [8, 4], torch.ones(2, 16), r, state)
    # with a slot stride S the factor arrays hold n_slots * S vectors
    with pytest.raises(sq.SqError, match="row_scale has 32 elements, expected 96"):
        sq.sq_pool_alloc(2, 2, 16, 16, [8, 4], r, r, state, scale_slot_stride=3)
