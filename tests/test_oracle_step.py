"""Pins for the oracle's decode step.

Each test ties the oracle to something other than itself: exact rational
arithmetic, the dense-matrix recurrence, closed-form invariants of the gated
delta rule (the decay and key-direction correction channels described in
"线性注意力状态量化难题" section 时间维度), or the quantizer's definition
evaluated independently in numpy.  A plausible slip in the oracle -- a dropped
term, a sign, a transposed operand, a wrong index -- fails at least one."""
from fractions import Fraction as F

import numpy as np
import pytest


def _unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _f32(x):
    return np.asarray(x, np.float32)


def _fp32_tile(orc, S):
    dk, dv = S.shape
    one_r, one_c = np.ones(dk, np.float32), np.ones(dv, np.float32)
    return orc.encode_tile(32, dk, dv, S, one_r, one_c), one_r, one_c


# ------------------------------------------------------------ exact rational

def test_one_step_matches_exact_rational_dense_form(orc):
    """S' = alpha (I - beta k k^T) S + beta k v^T and o = S'^T q, evaluated with
    Fractions on fp32-exact inputs, against the oracle's FP32-state step."""
    rng = np.random.default_rng(1)
    dk, dv = 4, 6  # non-square: a transposed operand cannot pass
    S = _f32(rng.standard_normal((dk, dv)))
    q, k = _f32(rng.standard_normal(dk)), _f32(rng.standard_normal(dk))
    v = _f32(rng.standard_normal(dv))
    alpha, beta = np.float32(0.8125), np.float32(0.375)
    tile, r1, c1 = _fp32_tile(orc, S.astype(np.float64))
    new_tile, o = orc.step_tile(32, dk, dv, tile, r1, c1, q, k, v, alpha, beta)
    Sn = orc.decode_tile(32, dk, dv, new_tile, r1, c1)

    Sf = [[F(float(S[i, j])) for j in range(dv)] for i in range(dk)]
    kf, qf, vf = [F(float(x)) for x in k], [F(float(x)) for x in q], [F(float(x)) for x in v]
    a, b = F(float(alpha)), F(float(beta))
    A = [[a * ((1 if i == l else 0) - b * kf[i] * kf[l]) for l in range(dk)] for i in range(dk)]
    Sx = [[sum(A[i][l] * Sf[l][j] for l in range(dk)) + b * kf[i] * vf[j] for j in range(dv)]
          for i in range(dk)]
    ox = [sum(qf[i] * Sx[i][j] for i in range(dk)) for j in range(dv)]
    for i in range(dk):
        for j in range(dv):
            # stored state is the exact value rounded once to fp32
            assert Sn[i, j] == float(np.float32(float(Sx[i][j])))
    for j in range(dv):
        assert abs(float(o[j]) - float(ox[j])) <= 2 ** -23 * abs(float(ox[j])) + 1e-30


def test_bruteforce_matches_exact_rational(orc):
    rng = np.random.default_rng(2)
    dk, dv, T = 3, 5, 3
    S0 = _f32(rng.standard_normal((dk, dv))).astype(np.float64)
    q, k = _f32(rng.standard_normal((T, dk))), _f32(rng.standard_normal((T, dk)))
    v = _f32(rng.standard_normal((T, dv)))
    alpha = _f32(rng.uniform(0.5, 1, T))
    beta = _f32(rng.uniform(0, 1, T))
    ST, o = orc.bruteforce(S0, q, k, v, alpha, beta)
    S = [[F(float(S0[i, j])) for j in range(dv)] for i in range(dk)]
    for t in range(T):
        kf = [F(float(x)) for x in k[t]]
        a, b = F(float(alpha[t])), F(float(beta[t]))
        u = [sum(kf[i] * S[i][j] for i in range(dk)) for j in range(dv)]
        S = [[a * S[i][j] - a * b * kf[i] * u[j] + b * kf[i] * F(float(v[t, j])) for j in range(dv)]
             for i in range(dk)]
        ot = [sum(F(float(q[t, i])) * S[i][j] for i in range(dk)) for j in range(dv)]
        np.testing.assert_allclose(o[t], [float(x) for x in ot], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ST, [[float(x) for x in row] for row in S], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ unrolled recurrence

@pytest.mark.parametrize("dk,dv", [(16, 16), (8, 24)])
def test_fp32_path_matches_bruteforce_recurrence(orc, dk, dv):
    """FP32 state through T oracle steps vs the dense Phi-product recurrence."""
    rng = np.random.default_rng(dk + dv)
    T = 8
    S0 = _f32(rng.normal(0, 0.1, (dk, dv))).astype(np.float64)
    q, k = _f32(_unit(rng, T, dk)), _f32(_unit(rng, T, dk))
    v = _f32(rng.standard_normal((T, dv)))
    alpha = _f32(np.exp(-np.log1p(np.exp(rng.standard_normal(T)))))
    beta = _f32(rng.uniform(0, 1, T))
    ST, o_ref = orc.bruteforce(S0, q, k, v, alpha, beta)
    tile, r1, c1 = _fp32_tile(orc, S0)
    for t in range(T):
        tile, o = orc.step_tile(32, dk, dv, tile, r1, c1, q[t], k[t], v[t], alpha[t], beta[t])
        np.testing.assert_allclose(o, o_ref[t], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(orc.decode_tile(32, dk, dv, tile, r1, c1), ST, rtol=1e-5, atol=1e-6)


# ------------------------------------------------------------ closed-form invariants

def _quant_tile(orc, rng, bits, dk, dv):
    r = _f32(rng.uniform(0.5, 2.0, dk))
    c = _f32(rng.uniform(0.01, 0.05, dv))
    Q = 2 ** (bits - 1) - 1
    codes = rng.integers(-Q, Q + 1, (dk, dv))
    s = np.array([[orc.step_size(float(r[i]), float(c[j])) for j in range(dv)] for i in range(dk)])
    return orc.encode_tile(bits, dk, dv, codes * s, r, c), r, c, codes, s


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_I1_pure_decay(orc, bits):
    rng = np.random.default_rng(10 + bits)
    dk, dv = 16, 32
    tile, r, c, codes, s = _quant_tile(orc, rng, bits, dk, dv)
    q, k = _f32(_unit(rng, 1, dk)[0]), _f32(_unit(rng, 1, dk)[0])
    v = _f32(rng.standard_normal(dv))
    # beta = 0, alpha = 1: codes unchanged, bit-exact, over several steps
    t = tile
    for _ in range(5):
        t, o = orc.step_tile(bits, dk, dv, t, r, c, q, k, v, 1.0, 0.0)
        assert np.array_equal(t, tile)
        np.testing.assert_allclose(o, orc.readout_tile(bits, dk, dv, tile, r, c, q), rtol=0, atol=0)
    # beta = 0, alpha < 1: q' = quant(alpha * S) elementwise (numpy model of the quantizer)
    alpha = np.float32(0.7)
    t, o = orc.step_tile(bits, dk, dv, tile, r, c, q, k, v, alpha, 0.0)
    Q = 2 ** (bits - 1) - 1
    z = (float(alpha) * codes * s / s).astype(np.float32).astype(np.float64)
    want = np.clip(np.round(z), -Q, Q)  # numpy rounds half to even
    got = orc.decode_tile(bits, dk, dv, t, r, c) / s
    assert np.array_equal(np.round(got), want)


@pytest.mark.parametrize("bits", [4, 6, 8, 16, 32])
def test_I2_write_into_row(orc, bits):
    """alpha = beta = 1, k = e_m: row m becomes v, every other row is untouched."""
    rng = np.random.default_rng(20 + bits)
    dk, dv, m = 16, 16, 5
    if bits <= 8:
        tile, r, c, codes, s = _quant_tile(orc, rng, bits, dk, dv)
    else:
        S = rng.standard_normal((dk, dv))
        r, c = np.ones(dk, np.float32), np.ones(dv, np.float32)
        tile = orc.encode_tile(bits, dk, dv, S, r, c)
        s = np.ones((dk, dv))
    k = np.zeros(dk, np.float32)
    k[m] = 1
    q = _f32(rng.standard_normal(dk))
    Q = 2 ** (bits - 1) - 1 if bits <= 8 else None
    v = _f32(rng.uniform(-0.9, 0.9, dv) * (Q * s[m].min() if bits <= 8 else 3))
    before = orc.decode_tile(bits, dk, dv, tile, r, c)
    t, o = orc.step_tile(bits, dk, dv, tile, r, c, q, k, v, 1.0, 1.0)
    after = orc.decode_tile(bits, dk, dv, t, r, c)
    others = [i for i in range(dk) if i != m]
    assert np.array_equal(after[others], before[others])
    if bits <= 8:
        want = np.clip(np.round((v.astype(np.float64) / s[m]).astype(np.float32)), -Q, Q)
        assert np.array_equal(np.round(after[m] / s[m]), want)
    elif bits == 16:
        assert np.array_equal(after[m], v.astype(np.float16).astype(np.float64))
    else:
        assert np.array_equal(after[m], v.astype(np.float64))


def test_I3_associative_recall_fp32(orc):
    rng = np.random.default_rng(30)
    dk, dv = 16, 12
    K, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = K.T  # rows orthonormal
    V = rng.standard_normal((dk, dv))
    tile, r1, c1 = _fp32_tile(orc, np.zeros((dk, dv)))
    for t in range(dk):
        tile, _ = orc.step_tile(32, dk, dv, tile, r1, c1, np.zeros(dk), K[t], V[t], 1.0, 1.0)
    S = orc.decode_tile(32, dk, dv, tile, r1, c1)
    Kf = _f32(K).astype(np.float64)  # the step saw fp32 keys
    for t in range(dk):
        np.testing.assert_allclose(S.T @ Kf[t], V[t], rtol=1e-5, atol=2e-6)


def test_I4_delta_identity_and_I5_norm_bound(orc):
    rng = np.random.default_rng(40)
    dk, dv = 16, 24
    for trial in range(20):
        S = rng.standard_normal((dk, dv))
        k = _unit(rng, 1, dk)[0].astype(np.float64)
        v = rng.standard_normal(dv)
        alpha, beta = rng.uniform(0.05, 1.0), rng.uniform(0, 1)
        tile, r1, c1 = _fp32_tile(orc, S)
        S32 = orc.decode_tile(32, dk, dv, tile, r1, c1)
        k32, v32 = _f32(k), _f32(v)
        a32, b32 = np.float32(alpha), np.float32(beta)
        t, _ = orc.step_tile(32, dk, dv, tile, r1, c1, np.zeros(dk), k32, v32, a32, b32)
        Sn = orc.decode_tile(32, dk, dv, t, r1, c1)
        kk = k32.astype(np.float64)
        nk2 = kk @ kk
        # k^T S' = alpha (1 - beta |k|^2) k^T S + beta |k|^2 v^T
        lhs = kk @ Sn
        rhs = float(a32) * (1 - float(b32) * nk2) * (kk @ S32) + float(b32) * nk2 * v32
        np.testing.assert_allclose(lhs, rhs, rtol=1e-5, atol=1e-5)
        # |S'|_F <= alpha |S|_F + beta |k| |v|  (|k| = 1 up to fp32 rounding)
        bound = float(a32) * np.linalg.norm(S32) + float(b32) * np.sqrt(nk2) * np.linalg.norm(v32)
        assert np.linalg.norm(Sn) <= bound * (1 + 1e-6)


@pytest.mark.parametrize("bits", [4, 6, 8, 16])
def test_I7_readout_identity(orc, bits):
    """o = S'^T q equals alpha S^T q + beta (q.k)(v - alpha u), u = S^T k."""
    rng = np.random.default_rng(50 + bits)
    dk, dv = 32, 16
    if bits <= 8:
        tile, r, c, codes, s = _quant_tile(orc, rng, bits, dk, dv)
    else:
        r, c = np.ones(dk, np.float32), np.ones(dv, np.float32)
        tile = orc.encode_tile(16, dk, dv, rng.standard_normal((dk, dv)), r, c)
    q, k = _f32(_unit(rng, 1, dk)[0]), _f32(_unit(rng, 1, dk)[0])
    v = _f32(rng.standard_normal(dv))
    alpha, beta = np.float32(0.9), np.float32(0.6)
    S = orc.decode_tile(bits, dk, dv, tile, r, c)
    _, o = orc.step_tile(bits, dk, dv, tile, r, c, q, k, v, alpha, beta)
    qd, kd, vd = q.astype(float), k.astype(float), v.astype(float)
    u = S.T @ kd
    want = float(alpha) * (S.T @ qd) + float(beta) * (qd @ kd) * (vd - float(alpha) * u)
    np.testing.assert_allclose(o, want, rtol=2e-6, atol=1e-6)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_I8_code_domain_requantization(orc, bits):
    """New codes equal clamp(rne(alpha q + (beta k_i / r_i)(v_j - alpha u_j) / c_j)),
    except where that value sits within 1e-6 of a rounding boundary."""
    rng = np.random.default_rng(60 + bits)
    dk, dv = 32, 32
    Q = 2 ** (bits - 1) - 1
    tile, r, c, codes, s = _quant_tile(orc, rng, bits, dk, dv)
    q, k = _f32(_unit(rng, 1, dk)[0]), _f32(_unit(rng, 1, dk)[0])
    v = _f32(rng.standard_normal(dv) * 0.3)
    alpha, beta = np.float32(0.95), np.float32(0.5)
    S = orc.decode_tile(bits, dk, dv, tile, r, c)
    t, _ = orc.step_tile(bits, dk, dv, tile, r, c, q, k, v, alpha, beta)
    new = np.round(orc.decode_tile(bits, dk, dv, t, r, c) / s).astype(int)
    u = S.T @ k.astype(float)
    a_i = float(beta) * k.astype(float) / r.astype(float)
    b_j = (v.astype(float) - float(alpha) * u) / c.astype(float)
    z = float(alpha) * codes + np.outer(a_i, b_j)
    want = np.clip(np.round(z), -Q, Q).astype(int)
    near = np.abs(np.abs(z - np.floor(z)) - 0.5) < 1e-6
    assert np.array_equal(new[~near], want[~near])
    assert (z.min() < -Q or z.max() > Q) or bits == 8  # the clamp is exercised for 4/6 bit


def test_P3_pivot_is_fp16_of_fp32_path(orc):
    rng = np.random.default_rng(70)
    dk, dv = 16, 16
    S = rng.standard_normal((dk, dv)).astype(np.float16).astype(np.float64)
    r, c = np.ones(dk, np.float32), np.ones(dv, np.float32)
    t16 = orc.encode_tile(16, dk, dv, S, r, c)
    t32 = orc.encode_tile(32, dk, dv, S, r, c)
    q, k = _f32(_unit(rng, 1, dk)[0]), _f32(_unit(rng, 1, dk)[0])
    v = _f32(rng.standard_normal(dv))
    n16, o16 = orc.step_tile(16, dk, dv, t16, r, c, q, k, v, 0.9, 0.4)
    n32, o32 = orc.step_tile(32, dk, dv, t32, r, c, q, k, v, 0.9, 0.4)
    assert np.array_equal(o16, o32)
    S32 = orc.decode_tile(32, dk, dv, n32, r, c)
    assert np.array_equal(orc.decode_tile(16, dk, dv, n16, r, c),
                          S32.astype(np.float16).astype(np.float64))


def test_bf16_state_is_bf16_of_fp32_path(orc):
    """The BF16-state step equals the FP32-state step rounded to bfloat16
    (torch's round-half-even conversion), and reads out the same o."""
    import torch
    rng = np.random.default_rng(71)
    dk, dv = 16, 16
    S = torch.from_numpy(rng.standard_normal((dk, dv)).astype(np.float32)).bfloat16().double().numpy()
    r, c = np.ones(dk, np.float32), np.ones(dv, np.float32)
    B = orc.BITS_BF16
    tb, t32 = orc.encode_tile(B, dk, dv, S, r, c), orc.encode_tile(32, dk, dv, S, r, c)
    q, k = _f32(_unit(rng, 1, dk)[0]), _f32(_unit(rng, 1, dk)[0])
    v = _f32(rng.standard_normal(dv))
    nb, ob = orc.step_tile(B, dk, dv, tb, r, c, q, k, v, 0.9, 0.4)
    n32, o32 = orc.step_tile(32, dk, dv, t32, r, c, q, k, v, 0.9, 0.4)
    assert np.array_equal(ob, o32)
    S32 = torch.from_numpy(orc.decode_tile(32, dk, dv, n32, r, c).astype(np.float32))
    assert np.array_equal(orc.decode_tile(B, dk, dv, nb, r, c), S32.bfloat16().double().numpy())
    # write into a row, as I2: row m becomes bf16(v), other rows untouched
    m = 3
    kk = np.zeros(dk, np.float32)
    kk[m] = 1
    t2, _ = orc.step_tile(B, dk, dv, tb, r, c, q, kk, v, 1.0, 1.0)
    after = orc.decode_tile(B, dk, dv, t2, r, c)
    assert np.array_equal(np.delete(after, m, 0), np.delete(S, m, 0))
    assert np.array_equal(after[m], torch.from_numpy(v).bfloat16().double().numpy())


def test_nonfinite_inputs_follow_the_stated_rule(orc):
    rng = np.random.default_rng(80)
    dk, dv = 16, 16
    tile, r, c, codes, s = _quant_tile(orc, rng, 8, dk, dv)
    q, k = _f32(_unit(rng, 1, dk)[0]), _f32(_unit(rng, 1, dk)[0])
    v = _f32(rng.standard_normal(dv))
    t, o = orc.step_tile(8, dk, dv, tile, r, c, q, k, v, np.nan, 0.5)
    assert np.all(np.round(orc.decode_tile(8, dk, dv, t, r, c) / s) == 0)  # NaN -> code 0
    assert np.all(np.isnan(o))
    # out-of-range values saturate to +-Q by sign (a huge finite gate; an infinite
    # one would make 0 * inf = NaN in the beta term)
    t, o = orc.step_tile(8, dk, dv, tile, r, c, q, k, v, 1e30, 0.0)
    got = np.round(orc.decode_tile(8, dk, dv, t, r, c) / s)
    assert np.all(got[codes > 0] == 127) and np.all(got[codes < 0] == -127)
    assert np.all(got[codes == 0] == 0)


# ------------------------------------------------------------ pool level

def test_pool_step_equals_per_tile_steps_with_slot_indirection(orc):
    rng = np.random.default_rng(90)
    dk = dv = 16
    bits = np.array([8, 4, 16, 6, 32], np.uint8)
    H = bits.size
    off, slab = orc.pool_layout(bits, dk, dv)
    n_slots = 5
    pool = rng.integers(0, 256, n_slots * slab, dtype=np.uint8)
    r = _f32(rng.uniform(0.5, 2, (H, dk)))
    c = _f32(rng.uniform(0.01, 0.05, (H, dv)))
    # make fp16/fp32 tiles hold finite values
    for p in range(n_slots):
        for h in (2, 4):
            t = orc.encode_tile(int(bits[h]), dk, dv, rng.standard_normal((dk, dv)), r[h], c[h])
            pool[p * slab + off[h]: p * slab + off[h] + t.size] = t
    slots = np.array([3, 0, 4], np.int32)
    n = slots.size
    q, k = _f32(_unit(rng, n * H, dk)), _f32(_unit(rng, n * H, dk))
    v = _f32(rng.standard_normal((n * H, dv)))
    alpha, beta = _f32(rng.uniform(0.5, 1, n * H)), _f32(rng.uniform(0, 1, n * H))
    ref = pool.copy()
    o = orc.step_pool(pool, bits, dk, dv, r, c, slots, q, k, v, alpha, beta, n_threads=3)
    for ni, p in enumerate(slots):
        for h in range(H):
            lo = p * slab + off[h]
            tb = orc.tile_bytes(int(bits[h]), dk, dv)
            t, oo = orc.step_tile(int(bits[h]), dk, dv, ref[lo:lo + tb], r[h], c[h], q[ni * H + h],
                                  k[ni * H + h], v[ni * H + h], alpha[ni * H + h], beta[ni * H + h])
            assert np.array_equal(pool[lo:lo + tb], t)
            assert np.array_equal(o[ni, h], oo)
    # slots not in the batch (1, 2) and tile padding are untouched
    for p in (1, 2):
        assert np.array_equal(pool[p * slab:(p + 1) * slab], ref[p * slab:(p + 1) * slab])
    # empty batch is a no-op
    before = pool.copy()
    orc.step_pool(pool, bits, dk, dv, r, c, np.zeros(0, np.int32), np.zeros(0), np.zeros(0),
                  np.zeros(0), np.zeros(0), np.zeros(0))
    assert np.array_equal(pool, before)
    # readout_pool is the non-mutating S^T q
    o2 = orc.readout_pool(pool, bits, dk, dv, r, c, slots, q)
    for ni, p in enumerate(slots):
        for h in range(H):
            lo = p * slab + off[h]
            tb = orc.tile_bytes(int(bits[h]), dk, dv)
            assert np.array_equal(o2[ni, h], orc.readout_tile(int(bits[h]), dk, dv, pool[lo:lo + tb],
                                                               r[h], c[h], q[ni * H + h]))
    assert np.array_equal(pool, before)


def test_store_pool_matches_encode(orc):
    rng = np.random.default_rng(91)
    dk = dv = 16
    bits = np.array([4, 6, 8, 16, 32], np.uint8)
    H = bits.size
    off, slab = orc.pool_layout(bits, dk, dv)
    pool = np.zeros(2 * slab, np.uint8)
    r = _f32(rng.uniform(0.5, 2, (H, dk)))
    c = _f32(rng.uniform(0.01, 0.05, (H, dv)))
    S = _f32(rng.normal(0, 1, (1, H, dk, dv)))
    orc.store_pool(pool, bits, dk, dv, r, c, np.array([1], np.int32), S)
    assert not pool[:slab].any()
    for h in range(H):
        t = orc.encode_tile(int(bits[h]), dk, dv, S[0, h].astype(np.float64), r[h], c[h])
        assert np.array_equal(pool[slab + off[h]: slab + off[h] + t.size], t)


def test_load_after_store_is_within_half_a_step(orc):
    """load(store(S)) differs from S by at most half a step in range (codes),
    rounds to binary16 (pivots), and is the identity for FP32 states."""
    rng = np.random.default_rng(92)
    dk, dv = 16, 12
    bits = np.array([4, 6, 8, 16, 32], np.uint8)
    H = bits.size
    off, slab = orc.pool_layout(bits, dk, dv)
    pool = np.zeros(3 * slab, np.uint8)
    r = _f32(rng.uniform(0.5, 2, (H, dk)))
    c = _f32(rng.uniform(0.01, 0.05, (H, dv)))
    S = _f32(rng.normal(0, 0.3, (2, H, dk, dv)))
    slots = np.array([2, 0], np.int32)
    orc.store_pool(pool, bits, dk, dv, r, c, slots, S)
    L = orc.load_pool(pool, bits, dk, dv, r, c, slots)
    for h in range(H):
        b = int(bits[h])
        if b <= 8:
            s = (r[h][:, None].astype(np.float64) * c[h][None, :]).astype(np.float32).astype(np.float64)
            Q = 2 ** (b - 1) - 1
            inr = np.abs(S[:, h]) <= Q * s
            err = np.abs(L[:, h].astype(np.float64) - S[:, h])
            assert np.all(err[inr] <= (s / 2 * (1 + 1e-6) + np.zeros_like(err))[inr])
            assert np.all(np.abs(L[:, h]) <= Q * s * (1 + 1e-6))
        elif b == 16:
            assert np.array_equal(L[:, h], S[:, h].astype(np.float16).astype(np.float32))
        else:
            assert np.array_equal(L[:, h], S[:, h])


# ------------------------------------------------------------ per-channel gate

def test_kda_one_step_exact_rational(orc):
    rng = np.random.default_rng(100)
    dk, dv = 4, 5
    S = _f32(rng.standard_normal((dk, dv)))
    q, k = _f32(rng.standard_normal(dk)), _f32(rng.standard_normal(dk))
    v = _f32(rng.standard_normal(dv))
    a = _f32(rng.uniform(0.3, 1.0, dk))
    beta = np.float32(0.625)
    tile, r1, c1 = _fp32_tile(orc, S.astype(np.float64))
    nt, o = orc.step_tile_kda(32, dk, dv, tile, r1, c1, q, k, v, a, beta)
    Sn = orc.decode_tile(32, dk, dv, nt, r1, c1)
    Sf = [[F(float(S[i, j])) for j in range(dv)] for i in range(dk)]
    kf, qf, vf, af = ([F(float(x)) for x in y] for y in (k, q, v, a))
    b = F(float(beta))
    A = [[((1 if i == l else 0) - b * kf[i] * kf[l]) * af[l] for l in range(dk)] for i in range(dk)]
    Sx = [[sum(A[i][l] * Sf[l][j] for l in range(dk)) + b * kf[i] * vf[j] for j in range(dv)]
          for i in range(dk)]
    for i in range(dk):
        for j in range(dv):
            assert Sn[i, j] == float(np.float32(float(Sx[i][j])))
    ox = [sum(qf[i] * Sx[i][j] for i in range(dk)) for j in range(dv)]
    for j in range(dv):
        assert abs(float(o[j]) - float(ox[j])) <= 2 ** -23 * abs(float(ox[j])) + 1e-30


def test_kda_matches_bruteforce_and_reduces_to_scalar_gate(orc):
    rng = np.random.default_rng(101)
    dk, dv, T = 16, 12, 6
    S0 = _f32(rng.normal(0, 0.2, (dk, dv))).astype(np.float64)
    q, k = _f32(_unit(rng, T, dk)), _f32(_unit(rng, T, dk))
    v = _f32(rng.standard_normal((T, dv)))
    a = _f32(rng.uniform(0.5, 1.0, (T, dk)))
    beta = _f32(rng.uniform(0, 1, T))
    ST, o_ref = orc.bruteforce_kda(S0, q, k, v, a, beta)
    tile, r1, c1 = _fp32_tile(orc, S0)
    for t in range(T):
        tile, o = orc.step_tile_kda(32, dk, dv, tile, r1, c1, q[t], k[t], v[t], a[t], beta[t])
        np.testing.assert_allclose(o, o_ref[t], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(orc.decode_tile(32, dk, dv, tile, r1, c1), ST, rtol=1e-5, atol=1e-6)
    # every channel equal: the scalar gated delta rule (dense form, separate code)
    a_s = _f32(rng.uniform(0.5, 1.0, T))
    ST1, o1 = orc.bruteforce_kda(S0, q, k, v, np.repeat(a_s[:, None], dk, 1), beta)
    ST2, o2 = orc.bruteforce(S0, q, k, v, a_s, beta)
    np.testing.assert_allclose(ST1, ST2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    # and the quantized per-channel step with equal channels equals the scalar step
    for bits in (4, 6, 8, 16):
        tq, rq, cq, codes, s = _quant_tile(orc, rng, bits, dk, dv) if bits <= 8 else (
            orc.encode_tile(16, dk, dv, rng.standard_normal((dk, dv)), r1, c1), r1, c1, None, None)
        al = np.float32(0.8125)
        t1, o1 = orc.step_tile_kda(bits, dk, dv, tq, rq, cq, q[0], k[0], v[0], np.full(dk, al, np.float32), beta[0])
        t2, o2 = orc.step_tile(bits, dk, dv, tq, rq, cq, q[0], k[0], v[0], al, beta[0])
        np.testing.assert_allclose(o1, o2, rtol=1e-6, atol=1e-7)
        d1, d2 = orc.decode_tile(bits, dk, dv, t1, rq, cq), orc.decode_tile(bits, dk, dv, t2, rq, cq)
        assert np.mean(d1 != d2) <= 0.01  # identical up to rounding-boundary flips


def test_kda_decay_only_rows(orc):
    """beta = 0: every row decays by its own channel gate."""
    rng = np.random.default_rng(102)
    dk, dv = 8, 8
    S = rng.standard_normal((dk, dv))
    tile, r1, c1 = _fp32_tile(orc, S)
    a = _f32(rng.uniform(0.1, 1.0, dk))
    nt, _ = orc.step_tile_kda(32, dk, dv, tile, r1, c1, np.zeros(dk), np.zeros(dk), np.zeros(dv), a, 0.0)
    S32 = orc.decode_tile(32, dk, dv, tile, r1, c1)
    want = (a.astype(np.float64)[:, None] * S32).astype(np.float32).astype(np.float64)
    assert np.array_equal(orc.decode_tile(32, dk, dv, nt, r1, c1), want)


def test_kda_pool_matches_tiles_and_threads(orc):
    """The pool-level per-channel step equals tile-by-tile steps, for any thread count."""
    rng = np.random.default_rng(103)
    bits = np.array([4, 6, 8, 16, 32], np.uint8)
    H, dk, dv, n_req = 5, 8, 12, 3
    r = _f32(rng.uniform(0.01, 0.02, (H, dk)))
    c = _f32(rng.uniform(0.5, 1.5, (H, dv)))
    off, slab = orc.pool_layout(bits, dk, dv)
    slots = np.array([2, 0, 3], np.int32)
    pool = rng.integers(0, 256, 4 * slab).astype(np.uint8)
    q, k = _f32(rng.standard_normal((n_req, H, dk))), _f32(rng.standard_normal((n_req, H, dk)))
    v = _f32(rng.standard_normal((n_req, H, dv)))
    a = _f32(rng.uniform(0.3, 1.0, (n_req, H, dk)))
    b = _f32(rng.uniform(0, 1, (n_req, H)))
    # random bytes are valid codes for 4/6/8 bits; give 16/32-bit heads finite values
    S = rng.standard_normal((dk, dv))
    for p in range(4):
        for h in (3, 4):
            t = orc.encode_tile(int(bits[h]), dk, dv, S, r[h], c[h])
            pool[p * slab + off[h]:p * slab + off[h] + t.size] = t
    want = pool.copy()
    o_want = np.empty((n_req, H, dv), np.float32)
    for n, p in enumerate(slots):
        for h in range(H):
            o0 = p * slab + off[h]
            nb = dk * dv * int(bits[h]) // 8
            t, o_want[n, h] = orc.step_tile_kda(int(bits[h]), dk, dv, want[o0:o0 + nb], r[h], c[h],
                                                q[n, h], k[n, h], v[n, h], a[n, h], b[n, h])
            want[o0:o0 + nb] = t
    for threads in (1, 4):
        got = pool.copy()
        o = orc.step_pool_kda(got, bits, dk, dv, r, c, slots, q, k, v, a, b, n_threads=threads)
        assert np.array_equal(got, want)
        assert np.array_equal(o, o_want)


def test_per_slot_factors_follow_the_slot(orc):
    """With a scale stride S every slot p has its own factors at (p*S + h); a
    stored code decodes to code * fl32(r_pi c_pj) of its own slot (checked in
    numpy), and the pool calls equal the tile calls on the slot's factors."""
    rng = np.random.default_rng(93)
    dk, dv = 16, 12
    bits = np.array([4, 6, 8, 16, 32], np.uint8)
    H, S = bits.size, bits.size + 2
    n_slots = 4
    off, slab = orc.pool_layout(bits, dk, dv)
    pool = np.zeros(n_slots * slab, np.uint8)
    r = _f32(rng.uniform(0.5, 2.0, (n_slots * S, dk)))
    c = _f32(rng.uniform(0.01, 0.05, (n_slots * S, dv)))
    slots = np.array([3, 1], np.int32)
    X = np.empty((slots.size, H, dk, dv), np.float32)
    codes = {}
    for n, p in enumerate(slots):
        for h in range(H):
            b = int(bits[h])
            if b <= 8:
                Q = 2 ** (b - 1) - 1
                codes[n, h] = rng.integers(-Q, Q + 1, (dk, dv))
                s = (r[p * S + h][:, None].astype(np.float64) * c[p * S + h][None, :]).astype(np.float32)
                X[n, h] = codes[n, h] * s.astype(np.float64)
            else:
                X[n, h] = rng.standard_normal((dk, dv))
    assert orc.store_pool(pool, bits, dk, dv, r, c, slots, X, scale_stride=S) == 0
    L = orc.load_pool(pool, bits, dk, dv, r, c, slots, scale_stride=S)
    for n, p in enumerate(slots):
        for h in range(H):
            b = int(bits[h])
            if b <= 8:
                s = (r[p * S + h][:, None].astype(np.float64) * c[p * S + h][None, :]).astype(np.float32)
                assert np.array_equal(L[n, h], (codes[n, h] * s.astype(np.float64)).astype(np.float32))
            elif b == 16:
                assert np.array_equal(L[n, h], X[n, h].astype(np.float16).astype(np.float32))
            else:
                assert np.array_equal(L[n, h], X[n, h])
    q, k = _f32(_unit(rng, slots.size * H, dk)), _f32(_unit(rng, slots.size * H, dk))
    v = _f32(rng.standard_normal((slots.size * H, dv)))
    alpha = _f32(rng.uniform(0.5, 1, slots.size * H))
    beta = _f32(rng.uniform(0, 1, slots.size * H))
    ref = pool.copy()
    o = orc.step_pool(pool, bits, dk, dv, r, c, slots, q, k, v, alpha, beta, scale_stride=S)
    o2 = orc.readout_pool(pool, bits, dk, dv, r, c, slots, q, scale_stride=S)
    for n, p in enumerate(slots):
        for h in range(H):
            b, lo, t = int(bits[h]), p * slab + off[h], n * H + h
            tb = orc.tile_bytes(b, dk, dv)
            tt, oo = orc.step_tile(b, dk, dv, ref[lo:lo + tb], r[p * S + h], c[p * S + h], q[t],
                                   k[t], v[t], alpha[t], beta[t])
            assert np.array_equal(pool[lo:lo + tb], tt)
            assert np.array_equal(o[n, h], oo)
            assert np.array_equal(o2[n, h], orc.readout_tile(b, dk, dv, tt, r[p * S + h],
                                                              c[p * S + h], q[t]))


def test_nonfinite_values_are_reported(orc):
    """The step reports a tile when a value it stores from is not finite: for a
    code, the fp32 quotient the code is decided on (so a finite update over a
    vanishing step size counts); for an FP16/FP32 element, the value itself (a
    finite value that overflows binary16 does not count).  A non-finite query
    touches only the readout and is not reported."""
    rng = np.random.default_rng(81)
    dk, dv = 16, 16
    tile, r, c, codes, s = _quant_tile(orc, rng, 8, dk, dv)
    q, k = _f32(_unit(rng, 1, dk)[0]), _f32(_unit(rng, 1, dk)[0])
    v = _f32(rng.standard_normal(dv))
    t0, o0, bad = orc.step_tile(8, dk, dv, tile, r, c, q, k, v, 0.9, 0.5, return_flag=True)
    assert not bad
    _, _, bad = orc.step_tile(8, dk, dv, tile, r, c, q, k, v, np.nan, 0.5, return_flag=True)
    assert bad
    vb = v.copy()
    vb[3] = np.inf
    t, _, bad = orc.step_tile(8, dk, dv, tile, r, c, q, k, vb, 0.9, 0.5, return_flag=True)
    assert bad
    got = np.round(orc.decode_tile(8, dk, dv, t, r, c) / s)
    # column 3 saturates by the sign of k_i (beta > 0); the other columns are unaffected
    assert np.array_equal(got[:, 3], np.where(k > 0, 127, -127))
    assert np.array_equal(np.delete(got, 3, 1),
                          np.delete(np.round(orc.decode_tile(8, dk, dv, t0, r, c) / s), 3, 1))
    qb = q.copy()
    qb[0] = np.nan
    t, o, bad = orc.step_tile(8, dk, dv, tile, r, c, qb, k, v, 0.9, 0.5, return_flag=True)
    assert not bad and np.array_equal(t, t0) and np.all(np.isnan(o))
    # a step size of 1e-40 (a binary32 subnormal): the update is finite, the quotient is not
    rt, ct = np.full(dk, 1e-20, np.float32), np.full(dv, 1e-20, np.float32)
    tt = orc.encode_tile(8, dk, dv, np.zeros((dk, dv)), rt, ct)
    t, _, bad = orc.step_tile(8, dk, dv, tt, rt, ct, q, k, v, 0.9, 0.5, return_flag=True)
    assert bad
    x = 0.5 * k[:, None].astype(np.float64) * v[None, :]
    got = np.array([[orc.field_get(t, 8, orc.elem_index(i, j, dv)) for j in range(dv)]
                    for i in range(dk)]).astype(np.int64) - 128
    assert np.array_equal(got, np.where(x > 0, 127, np.where(x < 0, -127, 0)))
    # FP16 / FP32 elements: reported on the fp32 value; 1e5 overflows binary16 only
    one_r, one_c = np.ones(dk, np.float32), np.ones(dv, np.float32)
    big = np.zeros((dk, dv))
    big[1, 2] = 1e5
    t16, bad = orc.encode_tile(16, dk, dv, big, one_r, one_c, return_flag=True)
    assert not bad and orc.field_get(t16, 16, orc.elem_index(1, 2, dv)) == 0x7C00
    big[1, 2] = 1e39
    _, bad = orc.encode_tile(32, dk, dv, big, one_r, one_c, return_flag=True)
    assert bad
    big[1, 2] = np.nan
    _, bad = orc.encode_tile(16, dk, dv, big, one_r, one_c, return_flag=True)
    assert bad


def test_pool_counts_reported_tiles(orc):
    rng = np.random.default_rng(82)
    dk = dv = 16
    bits = np.array([4, 8, 16, 32], np.uint8)
    H = bits.size
    off, slab = orc.pool_layout(bits, dk, dv)
    r = _f32(rng.uniform(0.5, 2, (H, dk)))
    c = _f32(rng.uniform(0.01, 0.05, (H, dv)))
    S0 = _f32(rng.normal(0, 0.2, (3, H, dk, dv)))
    pool = np.zeros(3 * slab, np.uint8)
    slots = np.array([2, 0, 1], np.int32)
    assert orc.store_pool(pool, bits, dk, dv, r, c, slots, S0) == 0
    S1 = S0.copy()
    S1[1, 2, 0, 0] = np.inf
    S1[2, 0, 5, 5] = np.nan
    assert orc.store_pool(pool.copy(), bits, dk, dv, r, c, slots, S1) == 2
    n = slots.size
    q, k = _f32(_unit(rng, n * H, dk)), _f32(_unit(rng, n * H, dk))
    v = _f32(rng.standard_normal((n * H, dv)))
    alpha, beta = _f32(rng.uniform(0.5, 1, n * H)), _f32(rng.uniform(0, 1, n * H))
    _, bad = orc.step_pool(pool.copy(), bits, dk, dv, r, c, slots, q, k, v, alpha, beta,
                           return_flagged=True)
    assert bad == 0
    alpha[1 * H + 3] = np.nan  # request 1, head 3
    beta[2 * H + 0] = np.inf   # request 2, head 0
    q[0, 0] = np.nan           # readout only
    _, bad = orc.step_pool(pool.copy(), bits, dk, dv, r, c, slots, q, k, v, alpha, beta,
                           return_flagged=True)
    assert bad == 2
    ab = _f32(rng.uniform(0.5, 1, (n * H, dk)))
    _, bad = orc.step_pool_kda(pool.copy(), bits, dk, dv, r, c, slots, q, k, v, ab,
                               _f32(rng.uniform(0, 1, n * H)), return_flagged=True)
    assert bad == 0
    ab[4, 7] = np.nan
    _, bad = orc.step_pool_kda(pool.copy(), bits, dk, dv, r, c, slots, q, k, v, ab,
                               _f32(rng.uniform(0, 1, n * H)), return_flagged=True)
    assert bad == 1
