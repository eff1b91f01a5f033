"""GPU parity of the per-key-channel-gate step (sq_decode_step_kda) against
the oracle's per-channel step, teacher-forced as in test_gpu_parity.py, over
every kernel the step can take: the fused d = 128 launch (4/6/8-bit codes and
FP16 pivots), the FP32-state launch, and the any-shape kernel."""
import numpy as np
import pytest
import torch

from gpu_harness import Case, KdaCase, Tally, host_f32, run_teacher_forced
from quantized_recurrent_state_gated_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    from quantized_recurrent_state_gated_amd import sq as m
    return m


def test_kda_tiny_all_steps(sq, orc):
    w = I.WORKLOADS["tiny"]
    run_teacher_forced(KdaCase(sq, orc, w), w.steps, "kda-tiny")


def test_kda_layer(sq, orc):
    w = I.scaled(I.WORKLOADS["layer"], steps=64)
    run_teacher_forced(KdaCase(sq, orc, w), w.steps, "kda-layer")


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_kda_d128_every_width(sq, orc, qkv):
    w = I.Workload("kmix", 3, 12, 128, 128, 4, {4: 2, 6: 2, 8: 2, 16: 2, 32: 2, I.BITS_BF16: 2}, qkv_dtype=qkv,
                   seed=199)
    run_teacher_forced(KdaCase(sq, orc, w, n_slots=5, slots=[4, 1, 2]), w.steps, f"kda-mix-{qkv}")


@pytest.mark.parametrize("dk,dv", [(12, 20), (64, 128), (256, 32)])
def test_kda_other_shapes(sq, orc, dk, dv):
    w = I.Workload("kshape", 2, 6, dk, dv, 3, {4: 1, 6: 1, 8: 1, 16: 1, 32: 1, I.BITS_BF16: 1}, seed=dk * 7 + dv)
    run_teacher_forced(KdaCase(sq, orc, w), w.steps, f"kda-shape{dk}x{dv}")


def test_kda_with_equal_channels_is_the_scalar_step(sq, orc):
    """alpha_i = alpha for every channel: the per-channel step and
    sq_decode_step agree to the parity tolerances (the two kernels round in
    a different order, so bit identity is not expected)."""
    w = I.Workload("keq", 3, 12, 128, 128, 3, {4: 2, 6: 2, 8: 2, 16: 2, 32: 2, I.BITS_BF16: 2}, seed=211)
    a, b = Case(sq, orc, w), Case(sq, orc, w)
    assert np.array_equal(a.host(), b.host())
    tally = Tally()
    for t in range(w.steps):
        si = I.step_inputs(w, t)
        o1 = a.step(si)
        o2 = torch.empty_like(o1)
        al = si.alpha.cuda()[..., None].expand(w.n_req, w.n_heads, w.dk).contiguous()
        sq.sq_decode_step_kda(b.pool, b.slots_d, si.q.cuda(), si.k.cuda(), si.v.cuda(), al,
                              si.beta.cuda(), o2)
        pa, pb = a.host(), b.host()
        from gpu_harness import compare_pools
        compare_pools(tally, pb, pa, a.bits, a.off, a.slab, a.slots, w.dk, w.dv)
        tally.add_o(o2.cpu().numpy(), o1.cpu().numpy())
        b.dev.copy_(a.dev)  # teacher-forced: both continue from the same bytes
    tally.check()


def test_kda_zero_write_decays_each_row(sq, orc):
    """beta = 0: every key row decays by its own gate; on FP32 heads the new
    state is exactly fl32(alpha_i S_ij); o = S'^T q."""
    w = I.Workload("kdecay", 2, 6, 128, 128, 1, {4: 1, 6: 1, 8: 1, 16: 1, 32: 1, I.BITS_BF16: 1}, seed=17)
    case = KdaCase(sq, orc, w)
    pre = case.host()
    si = case.inputs(0)
    si.beta.zero_()
    case.step(si)
    post = case.host()
    ref, _ = case.oracle_step(pre, si)
    tally = Tally()
    case.compare(tally, post, ref)
    tally.check()
    h = int(np.nonzero(case.bits == 32)[0][0])
    lo, tb = int(case.off[h]), orc.tile_bytes(32, 128, 128)
    for n, p in enumerate(case.slots):
        base = int(p) * case.slab + lo
        S0 = orc.decode_tile(32, 128, 128, pre[base:base + tb], case.r[h], case.c[h])
        S1 = orc.decode_tile(32, 128, 128, post[base:base + tb], case.r[h], case.c[h])
        want = (host_f32(si.alpha)[n, h].astype(np.float32)[:, None] * S0.astype(np.float32))
        assert np.array_equal(S1.astype(np.float32), want)


def test_kda_host_errors(sq, orc):
    w = I.scaled(I.WORKLOADS["layer"], 2, 6, 1)
    case = KdaCase(sq, orc, w)
    si = case.inputs(0)
    q, k, v = si.q.cuda(), si.k.cuda(), si.v.cuda()
    a, b = si.alpha.cuda(), si.beta.cuda()
    pre = case.host()
    rc = sq._lib.sq_decode_step_kda(case.pool.handle, case.slots_d.data_ptr(), 2, q.data_ptr(),
                                    k.data_ptr(), v.data_ptr(), 1, a.data_ptr() + 4, b.data_ptr(),
                                    None, None)
    assert rc == sq.SQ_ERR_INVALID  # misaligned alpha
    rc = sq._lib.sq_decode_step_kda(case.pool.handle, case.slots_d.data_ptr(), 2, q.data_ptr(),
                                    k.data_ptr(), v.data_ptr(), 1, None, b.data_ptr(), None, None)
    assert rc == sq.SQ_ERR_INVALID
    empty = torch.zeros(0, dtype=torch.int32, device="cuda")
    z = torch.zeros(0, device="cuda")
    sq.sq_decode_step_kda(case.pool, empty, z, z, z, z, z, None)
    assert np.array_equal(case.host(), pre)


def test_kda_mid_size_launch(sq, orc):
    """The per-channel gate through the 256-thread launch (1,024-16,383 tiles)."""
    w = I.Workload("kmid", 4, 300, 128, 128, 2, {4: 96, 6: 100, 8: 96, 16: 4, 32: 2, I.BITS_BF16: 2},
                   seed=52)
    assert 1024 <= w.n_req * w.n_heads < 16384
    run_teacher_forced(KdaCase(sq, orc, w), w.steps, "kda-mid")


@pytest.mark.parametrize("n_req", [3, 167])
def test_kda_head_groups_of_unequal_size(sq, orc, n_req):
    """The per-channel gate over n_req x 100 heads (XCD head groups of 12 and
    13); 167 requests (16,700 tiles) take the two-tiles-per-workgroup launch."""
    w = I.Workload(f"kh100x{n_req}", n_req, 100, 128, 128, 2,
                   {4: 30, 6: 30, 8: 30, 16: 4, 32: 3, I.BITS_BF16: 3}, seed=100 + n_req)
    slots = list(range(n_req + 1))[::-1][:n_req]
    run_teacher_forced(KdaCase(sq, orc, w, n_slots=n_req + 1, slots=slots), w.steps,
                       f"kda-h100x{n_req}")
