"""Pins for the oracle's storage formats: bit packing, tile layout, binary16,
and the quantizer.  Expected bytes are computed here from the written
definition with plain Python integer arithmetic, never by the oracle."""
import math

import numpy as np
import pytest


# ---------------------------------------------------------------- layout

def test_elem_index_spot_values(orc):
    dv = 128
    assert orc.elem_index(0, 0, dv) == 0
    assert orc.elem_index(1, 0, dv) == 1          # rows of a column are consecutive
    assert orc.elem_index(3, 0, dv) == 3
    assert orc.elem_index(0, 1, dv) == 4          # next column of the block
    assert orc.elem_index(3, 3, dv) == 15
    assert orc.elem_index(0, 4, dv) == 16         # next block to the right
    assert orc.elem_index(4, 0, dv) == 16 * (dv // 4)  # next block row
    assert orc.elem_index(127, 127, dv) == 128 * 128 - 1


@pytest.mark.parametrize("dk,dv", [(4, 4), (16, 16), (16, 32), (32, 16), (128, 128), (8, 20)])
def test_elem_index_is_bijection(orc, dk, dv):
    seen = np.zeros(dk * dv, bool)
    for i in range(dk):
        for j in range(dv):
            n = orc.elem_index(i, j, dv)
            assert 0 <= n < dk * dv and not seen[n]
            seen[n] = True
    assert seen.all()


def test_tile_bytes_and_pool_layout(orc):
    assert orc.tile_bytes(4, 128, 128) == 8192
    assert orc.tile_bytes(6, 128, 128) == 12288
    assert orc.tile_bytes(8, 128, 128) == 16384
    assert orc.tile_bytes(16, 128, 128) == 32768
    assert orc.tile_bytes(32, 128, 128) == 65536
    assert orc.tile_bytes(4, 16, 16) == 128
    assert orc.tile_bytes(6, 16, 16) == 192
    off, slab = orc.pool_layout([4, 6, 8, 16, 32], 16, 16)
    # each tile starts on a 256-byte boundary
    assert list(off) == [0, 256, 512, 768, 1280]
    assert slab == 1280 + 1024
    off, slab = orc.pool_layout([8, 6, 4, 16], 128, 128)
    assert list(off) == [0, 16384, 16384 + 12288, 16384 + 12288 + 8192]
    assert slab == 16384 + 12288 + 8192 + 32768


# ---------------------------------------------------------------- packing

def _expected_bytes(w, fields, nbytes):
    """Little-endian bit stream written with Python integers."""
    acc = 0  # Python int: arbitrary width
    for n, f in enumerate(fields):
        acc |= (int(f) & ((1 << w) - 1)) << (n * w)
    return acc.to_bytes(nbytes, "little")


@pytest.mark.parametrize("w,group_bytes,per_group", [(4, 1, 2), (6, 3, 4), (8, 1, 1)])
def test_pack_exhaustive_every_value_every_position(orc, w, group_bytes, per_group):
    rng = np.random.default_rng(7)
    for pos in range(per_group):
        for val in range(1 << w):
            for fill in (0x00, 0xFF):
                tile = np.full(4 * group_bytes, fill, np.uint8)
                n = per_group + pos  # second group, so the first and last are neighbours
                orc.field_put(tile, w, n, val)
                assert orc.field_get(tile, w, n) == val
                # neighbours untouched
                fields = [orc.field_get(tile, w, m) for m in range(4 * per_group)]
                other = [(1 << w) - 1 if fill else 0] * (4 * per_group)
                other[n] = val
                assert fields == other
                assert bytes(tile) == _expected_bytes(w, other, 4 * group_bytes)
    # random whole-stream round trip against the integer model
    fields = list(rng.integers(0, 1 << w, size=64))
    tile = np.zeros(64 * w // 8, np.uint8)
    for n, f in enumerate(fields):
        orc.field_put(tile, w, n, int(f))
    assert bytes(tile) == _expected_bytes(w, fields, 64 * w // 8)


def test_six_bit_group_layout_literal(orc):
    # four codes in three bytes: u0 | u1<<6 | u2<<12 | u3<<18, little-endian
    tile = np.zeros(3, np.uint8)
    for n, u in enumerate([0x3F, 0x00, 0x2A, 0x15]):
        orc.field_put(tile, 6, n, u)
    word = 0x3F | (0x00 << 6) | (0x2A << 12) | (0x15 << 18)
    assert bytes(tile) == word.to_bytes(3, "little")


def test_fp16_and_fp32_fields_little_endian(orc):
    tile = np.zeros(8, np.uint8)
    orc.field_put(tile, 16, 1, 0xABCD)
    assert list(tile[2:4]) == [0xCD, 0xAB]
    orc.field_put(tile, 32, 1, 0x12345678)
    assert list(tile[4:8]) == [0x78, 0x56, 0x34, 0x12]


# ---------------------------------------------------------------- binary16

def test_f16_to_f32_exhaustive_vs_numpy(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_vs_numpy(orc):
    rng = np.random.default_rng(11)
    parts = [
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(50000) * 1e-5).astype(np.float32),        # subnormal range
        (rng.standard_normal(50000) * 3e4).astype(np.float32),         # near overflow
        rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]
    # exact ties: midpoints between adjacent binary16 values (RNE decides)
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    parts.append(((lo + hi) / 2).astype(np.float32))
    parts.append(-((lo + hi) / 2).astype(np.float32))
    parts.append(np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.996, 65520, 6e-8, 2.98e-8,
                           2.9802322e-08, 5.96e-8, 6.1035156e-05, 6.1e-5], np.float32))
    x = np.concatenate(parts)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16)
    ours = orc.f32_to_f16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan].view(np.uint16))
    assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all((ours[nan] & 0x3FF) != 0)


# ---------------------------------------------------------------- quantizer

@pytest.mark.parametrize("bits", [4, 6, 8])
def test_quantizer_error_bound_and_saturation(orc, bits):
    Q = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(bits)
    for s in (0.013, 0.25, 1.0, 3.7e-3):
        s32 = float(np.float32(s))
        xs = rng.uniform(-1.5 * Q * s32, 1.5 * Q * s32, 4000)
        for x in xs:
            q = orc.quantize(bits, float(x), s32)
            assert -Q <= q <= Q
            if abs(x) <= Q * s32:
                assert abs(x - q * s32) <= s32 / 2 * (1 + 1e-6)
            elif x > 0:
                assert q == Q
            else:
                assert q == -Q
        # code -> value -> code is the identity on every code
        for q in range(-Q, Q + 1):
            assert orc.quantize(bits, q * s32, s32) == q
            f = orc.encode_field(bits, q * s32, s32)
            assert f == q + 2 ** (bits - 1)
            assert orc.decode_field(bits, f, s32) == q * s32


def test_quantizer_ties_to_even_and_specials(orc):
    for x, want in [(2.5, 2), (3.5, 4), (-2.5, -2), (-3.5, -4), (0.5, 0), (-0.5, 0), (1.5, 2)]:
        assert orc.quantize(8, x, 1.0) == want
    assert orc.quantize(8, math.nan, 1.0) == 0
    assert orc.quantize(8, math.inf, 1.0) == 127
    assert orc.quantize(8, -math.inf, 1.0) == -127
    assert orc.quantize(4, 1e30, 1e-3) == 7
    # the decision is taken on the fp32 quotient: 2.5 + 2^-30 rounds to 2.5 in fp32
    assert orc.quantize(8, 2.5 + 2.0 ** -30, 1.0) == 2


def test_step_size_is_fp32_product(orc):
    rng = np.random.default_rng(3)
    for _ in range(1000):
        r, c = np.float32(rng.uniform(0.01, 10)), np.float32(rng.uniform(0.001, 1))
        assert orc.step_size(float(r), float(c)) == float(np.float32(r) * np.float32(c))


def test_encode_decode_tile_roundtrip(orc):
    rng = np.random.default_rng(5)
    dk, dv = 16, 32
    r = rng.uniform(0.5, 2, dk).astype(np.float32)
    c = rng.uniform(0.01, 0.1, dv).astype(np.float32)
    for bits in (4, 6, 8):
        Q = 2 ** (bits - 1) - 1
        codes = rng.integers(-Q, Q + 1, (dk, dv))
        s = np.array([[orc.step_size(float(r[i]), float(c[j])) for j in range(dv)] for i in range(dk)])
        tile = orc.encode_tile(bits, dk, dv, codes * s, r, c)
        assert tile.size == dk * dv * bits // 8
        S = orc.decode_tile(bits, dk, dv, tile, r, c)
        assert np.array_equal(S, codes * s)
        # the stored field of (i, j) sits at the layout position with excess-2^(b-1) bias
        for (i, j) in [(0, 0), (3, 5), (15, 31), (8, 17)]:
            assert orc.field_get(tile, bits, orc.elem_index(i, j, dv)) == codes[i, j] + 2 ** (bits - 1)
    for bits in (16, 32):
        vals = rng.standard_normal((dk, dv))
        tile = orc.encode_tile(bits, dk, dv, vals, r, c)
        S = orc.decode_tile(bits, dk, dv, tile, r, c)
        want = vals.astype(np.float16 if bits == 16 else np.float32).astype(np.float64)
        assert np.array_equal(S, want)


# ---------------------------------------------------------------- bfloat16 state

def test_bf16_to_f32_exhaustive(orc):
    """Every bfloat16 pattern: the oracle's decoding equals the pattern placed in
    the upper half of a binary32 (bfloat16 is that half) and torch's bfloat16."""
    import torch
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_bits_to_f32(h)
    upper = (h.astype(np.uint32) << 16).view(np.float32)
    via_torch = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(upper)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(np.isnan(via_torch), nan)
    assert np.array_equal(got[~nan].view(np.uint32), upper[~nan].view(np.uint32))
    assert np.array_equal(got[~nan].view(np.uint32), via_torch[~nan].view(np.uint32))


def test_f32_to_bf16_round_half_even_matches_torch(orc):
    import torch
    rng = np.random.default_rng(21)
    u = rng.integers(0, 2 ** 32, 400_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    # exact ties (low 16 bits = 0x8000) with even and odd kept halves, the
    # overflow edge, subnormals and zeros
    ties = ((rng.integers(0, 2 ** 16, 20_000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    edge = np.array([3.3895313892515355e38, 3.3961775292304172e38, 3.4e38, -3.39e38, 1e-40, -1e-45,
                     0.0, -0.0, 1.0, 1.00390625, 1.005859375], np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)], edge])
    got = orc.f32_to_bf16_bits(x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # NaN stays NaN, infinities stay infinite
    special = orc.f32_to_bf16_bits(np.array([np.nan, np.inf, -np.inf], np.float32))
    assert (special[0] & 0x7f80) == 0x7f80 and (special[0] & 0x7f) != 0
    assert special[1] == 0x7f80 and special[2] == 0xff80


def test_bf16_state_tile_roundtrip(orc):
    rng = np.random.default_rng(22)
    dk, dv = 12, 20
    r, c = np.ones(dk, np.float32), np.ones(dv, np.float32)
    vals = rng.standard_normal((dk, dv)) * 10.0
    assert orc.field_width(orc.BITS_BF16) == 16 and orc.tile_bytes(orc.BITS_BF16, dk, dv) == dk * dv * 2
    tile = orc.encode_tile(orc.BITS_BF16, dk, dv, vals, r, c)
    S = orc.decode_tile(orc.BITS_BF16, dk, dv, tile, r, c)
    want = orc.bf16_bits_to_f32(orc.f32_to_bf16_bits(vals.astype(np.float32))).astype(np.float64)
    assert np.array_equal(S, want)
    # field (i, j) is the bfloat16 of element (i, j) at the layout position
    for (i, j) in [(0, 0), (5, 7), (11, 19)]:
        assert orc.field_get(tile, 16, orc.elem_index(i, j, dv)) == \
            int(orc.f32_to_bf16_bits(np.array([vals[i, j]], np.float32))[0])
    off, slab = orc.pool_layout([orc.BITS_BF16, 4], 128, 128)
    assert list(off) == [0, 32768] and slab == 32768 + 8192
