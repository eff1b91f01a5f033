"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every step is teacher-forced: the oracle starts from the GPU's own pre-step
bytes with identical inputs, and the two post-step states and readouts are
compared to the tolerances in gpu_harness.  Sizes here span several tiles and
every width class; the full-size workloads are in test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

from gpu_harness import Case, KdaCase, Tally, host_f32, run_teacher_forced, say, unpack_fields
from quantized_recurrent_state_gated_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    from quantized_recurrent_state_gated_amd import sq as m
    return m


# ------------------------------------------------------------------ store

@pytest.mark.parametrize("name,shape", [("tiny", None), ("layer", (3, 12)), ("any", (2, 5))])
def test_store_bit_exact(sq, orc, name, shape):
    if name == "any":
        w = I.Workload("any", 2, 6, 12, 20, 1, {4: 1, 6: 1, 8: 1, 16: 1, 32: 1, I.BITS_BF16: 1}, seed=77)
    else:
        w = I.WORKLOADS[name] if shape is None else I.scaled(I.WORKLOADS[name], *shape)
    say(f"store {w.name} {w.n_req}x{w.n_heads} d={w.dk}x{w.dv}")
    case = Case(sq, orc, w, n_slots=w.n_req + 1, slots=np.arange(w.n_req)[::-1] + 1)
    ref = case.host()
    case.dev.zero_()
    S0 = torch.from_numpy(case.S0).cuda()
    sq.sq_pool_store(case.pool, case.slots_d, S0)
    got = case.host()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dk,dv", [(128, 128), (12, 20)])
def test_load_bit_exact(sq, orc, dk, dv):
    w = I.Workload("load", 2, 6, dk, dv, 2, {4: 1, 6: 1, 8: 1, 16: 1, 32: 1, I.BITS_BF16: 1}, seed=dk + dv)
    case = Case(sq, orc, w, n_slots=4, slots=[3, 1])
    case.step(I.step_inputs(w, 0))  # load a state that has been through a step
    host = case.host()
    S = torch.empty(w.n_req, w.n_heads, dk, dv, device="cuda")
    sq.sq_pool_load(case.pool, case.slots_d, S)
    want = orc.load_pool(host, case.bits, dk, dv, case.r, case.c, case.slots)
    got = S.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # store(load(x)) reproduces the tiles bit for bit
    before = case.host().copy()
    case.dev.zero_()
    sq.sq_pool_store(case.pool, case.slots_d, S)
    after = case.host()
    for p in case.slots:
        assert np.array_equal(after[p * case.slab:(p + 1) * case.slab],
                              before[p * case.slab:(p + 1) * case.slab])


# ------------------------------------------------------------------ step parity

def test_tiny_all_steps(sq, orc):
    w = I.WORKLOADS["tiny"]
    run_teacher_forced(Case(sq, orc, w), w.steps, "tiny")


def test_tiny_literal_scales_degenerate(sq, orc):
    """The tiny recipe's column factors read literally as steps (0.5..2): an
    N(0, 0.1^2) state then quantizes to all-zero codes; the step must still
    agree with the oracle (codes move only where updates exceed half a step)."""
    w = I.WORKLOADS["tiny"]
    r, c = I.scales(w)
    case = Case(sq, orc, w, scales=(r.numpy(), c.numpy() * 127.0))
    pre = case.host()
    fields = unpack_fields(pre[None, : orc.tile_bytes(8, 16, 16)], 8)
    assert np.all(fields == 128)  # every code is zero
    run_teacher_forced(case, w.steps, "tiny-literal", check_changes=False)


def test_layer_all_steps(sq, orc):
    w = I.WORKLOADS["layer"]
    run_teacher_forced(Case(sq, orc, w), w.steps, "layer")


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_d128_every_width(sq, orc, qkv):
    w = I.Workload("mix", 3, 12, 128, 128, 4, {4: 2, 6: 2, 8: 2, 16: 2, 32: 2, I.BITS_BF16: 2}, qkv_dtype=qkv,
                   seed=99)
    run_teacher_forced(Case(sq, orc, w, n_slots=5, slots=[4, 1, 2]), w.steps, f"mix-{qkv}")


@pytest.mark.parametrize("dk,dv", [(16, 16), (12, 20), (128, 64), (64, 128), (256, 32), (4, 4), (256, 256)])
def test_other_shapes(sq, orc, dk, dv):
    w = I.Workload("shape", 2, 6, dk, dv, 3, {4: 1, 6: 1, 8: 1, 16: 1, 32: 1, I.BITS_BF16: 1}, seed=dk * 1000 + dv)
    run_teacher_forced(Case(sq, orc, w), w.steps, f"shape{dk}x{dv}")


def test_single_width_pools(sq, orc):
    for bits in (4, 6, 8, 16, 32, I.BITS_BF16):
        w = I.Workload(f"only{bits}", 2, 3, 128, 128, 2, {bits: 3}, seed=bits)
        run_teacher_forced(Case(sq, orc, w), w.steps, w.name)


# ------------------------------------------------------------------ invariants on the GPU

def test_pure_decay_keeps_codes_and_readout(sq, orc):
    """beta = 0, alpha = 1: codes are unchanged bit for bit, o = S^T q equals
    sq_readout, for every width.  The two are different kernel instances, free
    to contract different multiply-add pairs; a code tile's readout comes out
    of the excess form Y - OFF sum(g), whose terms are up to OFF (128 at
    8 bits) times the result, so the two agree to a few hundred fp32 ulps of
    the head's largest readout, not to one."""
    w = I.Workload("decay", 2, 12, 128, 128, 3, {4: 2, 6: 2, 8: 2, 16: 2, 32: 2, I.BITS_BF16: 2}, seed=5)
    case = Case(sq, orc, w)
    start = case.host()
    for t in range(w.steps):
        si = I.step_inputs(w, t)
        si.alpha.fill_(1.0)
        si.beta.zero_()
        o = case.step(si)
        assert np.array_equal(case.host(), start)
        o2 = torch.empty_like(o)
        sq.sq_readout(case.pool, case.slots_d, si.q.cuda(), o2)
        torch.cuda.synchronize()
        a, b = o.cpu().numpy(), o2.cpu().numpy()
        lim = 4e-5 * np.abs(b).max(axis=-1, keepdims=True) + 1e-6
        assert np.all(np.abs(a - b) <= lim), float((np.abs(a - b) / lim).max())
        o_ref = orc.readout_pool(start, case.bits, w.dk, w.dv, case.r, case.c, case.slots,
                                 host_f32(si.q))
        t2 = Tally()
        t2.add_o(o2.cpu().numpy(), o_ref)
        t2.check()


def test_write_into_row(sq, orc):
    """alpha = beta = 1, k = e_m: only row m changes."""
    w = I.Workload("row", 1, 6, 128, 128, 1, {4: 1, 6: 1, 8: 1, 16: 1, 32: 1, I.BITS_BF16: 1}, seed=6)
    case = Case(sq, orc, w)
    pre = case.host()
    si = I.step_inputs(w, 0)
    m = 37
    si.alpha.fill_(1.0)
    si.beta.fill_(1.0)
    k = torch.zeros_like(si.k)
    k[..., m] = 1.0
    si.k = k
    case.step(si)
    post = case.host()
    for h in range(w.n_heads):
        b = int(case.bits[h])
        tb = orc.tile_bytes(b, 128, 128)
        lo = int(case.off[h])
        S_pre = orc.decode_tile(b, 128, 128, pre[lo:lo + tb], case.r[h], case.c[h])
        S_post = orc.decode_tile(b, 128, 128, post[lo:lo + tb], case.r[h], case.c[h])
        others = np.arange(128) != m
        assert np.array_equal(S_post[others], S_pre[others])
        assert not np.array_equal(S_post[m], S_pre[m])
    ref, _ = case.oracle_step(pre, si)
    tally = Tally()
    case.compare(tally, post, ref)
    tally.check()


def test_determinism_and_checkpoint_restore(sq, orc):
    """Two runs from one snapshot are bit-identical (no atomics, fixed order);
    restoring the snapshot and replaying reproduces pool and readouts."""
    w = I.scaled(I.WORKLOADS["layer"], 4, 24, 6)
    case = Case(sq, orc, w)
    for t in range(2):
        case.step(I.step_inputs(w, t))
    snap = case.dev.clone()
    runs = []
    for _ in range(2):
        case.dev.copy_(snap)
        outs = [case.step(I.step_inputs(w, t)).cpu() for t in range(2, w.steps)]
        runs.append((case.host().copy(), outs))
    assert np.array_equal(runs[0][0], runs[1][0])
    for a, b in zip(runs[0][1], runs[1][1]):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ edge cases

def test_empty_batch_is_noop(sq, orc):
    w = I.scaled(I.WORKLOADS["layer"], 2, 6, 1)
    case = Case(sq, orc, w)
    pre = case.host()
    empty = torch.zeros(0, dtype=torch.int32, device="cuda")
    z = torch.zeros(0, device="cuda")
    sq.sq_decode_step(case.pool, empty, z, z, z, z, z, None)
    sq.sq_readout(case.pool, empty, z, z)
    sq.sq_pool_store(case.pool, empty, z)
    assert np.array_equal(case.host(), pre)


def test_subset_of_slots_and_no_readout(sq, orc):
    """A batch touching 3 of 7 slots in scrambled order, o not requested:
    untouched slots keep their bytes."""
    w = I.scaled(I.WORKLOADS["layer"], 3, 12, 2)
    case = Case(sq, orc, w, n_slots=7, slots=[6, 2, 4])
    for t in range(w.steps):
        si = I.step_inputs(w, t)
        pre = case.host()
        case.step(si, want_o=False)
        post = case.host()
        for p in (0, 1, 3, 5):
            assert np.array_equal(post[p * case.slab:(p + 1) * case.slab],
                                  pre[p * case.slab:(p + 1) * case.slab])
        ref, _ = case.oracle_step(pre, si)
        tally = Tally()
        case.compare(tally, post, ref)
        tally.check()


def test_host_errors_with_a_live_pool(sq, orc):
    w = I.scaled(I.WORKLOADS["layer"], 2, 6, 1)
    case = Case(sq, orc, w)
    si = I.step_inputs(w, 0)
    q, k, v = si.q.cuda(), si.k.cuda(), si.v.cuda()
    a, b = si.alpha.cuda(), si.beta.cuda()
    with pytest.raises(sq.SqError) as e:  # the library's own check: more requests than slots
        too_many = torch.zeros(3, dtype=torch.int32, device="cuda")
        sq._check(sq._lib.sq_decode_step(case.pool.handle, too_many.data_ptr(), 3, q.data_ptr(),
                                         k.data_ptr(), v.data_ptr(), 1, a.data_ptr(), b.data_ptr(),
                                         None, None), "too many requests")
    assert e.value.status == sq.SQ_ERR_INVALID
    with pytest.raises(sq.SqError) as e:  # the binding's: q sized for 2 requests, 3 slot ids
        sq.sq_decode_step(case.pool, too_many, q, k, v, a, b)
    assert e.value.status == sq.SQ_ERR_INVALID
    with pytest.raises(sq.SqError):
        rc = sq._lib.sq_decode_step(case.pool.handle, case.slots_d.data_ptr(), 2, q.data_ptr() + 2,
                                    k.data_ptr(), v.data_ptr(), 1, a.data_ptr(), b.data_ptr(),
                                    None, None)
        sq._check(rc, "misaligned q")
    assert sq._lib.sq_decode_step(case.pool.handle, case.slots_d.data_ptr(), 2, q.data_ptr(),
                                  k.data_ptr(), v.data_ptr(), 7, a.data_ptr(), b.data_ptr(), None,
                                  None) == sq.SQ_ERR_INVALID
    off, nb = sq.sq_pool_tile_offset(case.pool, 1, 3)
    assert off == case.slab + int(case.off[3]) and nb == orc.tile_bytes(int(case.bits[3]), 128, 128)
    with pytest.raises(sq.SqError):
        sq.sq_pool_tile_offset(case.pool, 2, 0)


def test_check_slots(sq, orc):
    """sq_check_slots flags ids out of range (1) and repeated ids (2), and
    successive calls on one pool stay independent (generation stamps)."""
    w = I.scaled(I.WORKLOADS["layer"], 2, 6, 1)
    case = Case(sq, orc, w, n_slots=9, slots=[3, 5])
    res = torch.full((1,), -7, dtype=torch.int32, device="cuda")

    def check(ids):
        t = torch.tensor(ids, dtype=torch.int32, device="cuda")
        sq.sq_check_slots(case.pool, t, res)
        torch.cuda.synchronize()
        return int(res.item())

    assert check([3, 5]) == 0
    assert check([0, 1, 2, 3, 4, 5, 6, 7, 8]) == 0
    assert check([8, 0, 8]) == 2
    assert check([3, 5]) == 0  # stamps from the previous calls do not leak
    assert check([9]) == 1 and check([-1, 2]) == 1
    assert check([4, 9, 4]) == 3
    assert check(list(range(9))[::-1]) == 0
    assert check([]) == 0
    big = torch.arange(9, dtype=torch.int32, device="cuda").repeat(300)  # 2700 ids, many blocks
    sq.sq_check_slots(case.pool, big, res)
    torch.cuda.synchronize()
    assert int(res.item()) == 2
    pre = case.host()
    assert check([0, 1]) == 0
    assert np.array_equal(case.host(), pre)  # the check never touches the pool


def _plant_nonfinite(si, H, kda=False):
    """Non-finite inputs whose stored result is unique (the same in any
    evaluation order), one kind per request: 0 NaN gate (every head), 1 NaN
    write strength / NaN key element, 2 NaN and +-Inf value elements (one
    column each), 3 NaN query element (readout only), 4 untouched."""
    nan, inf = float("nan"), float("inf")
    for h in range(H):
        if kda:
            si.alpha[0, h, (7 * h) % si.alpha.shape[-1]] = nan
        else:
            si.alpha[0, h] = nan
    for h in range(0, H, 3):
        si.beta[1, h] = nan
    for h in range(1, H, 3):
        si.k[1, h, (5 * h) % si.k.shape[-1]] = nan
    dv = si.v.shape[-1]
    for h in range(H):
        si.v[2, h, (3 * h) % dv] = (nan, inf, -inf)[h % 3]
    for h in range(0, H, 2):
        si.q[3, h, h % si.q.shape[-1]] = nan
    return si


def _nonfinite_case(sq, orc, w, kda=False, **kw):
    """Step once with planted non-finite inputs; compare every tile (codes
    exactly as the NaN -> 0 / +-Inf -> +-Q rule decides them) and every
    readout against the oracle, and the sticky flag against the oracle's
    count of tiles that stored from a non-finite value."""
    case = (KdaCase if kda else Case)(sq, orc, w, **kw)
    assert sq.sq_pool_last_device_error(case.pool) == sq.SQ_OK
    pre = case.host()
    si = _plant_nonfinite(case.inputs(0), w.n_heads, kda)
    o = case.step(si)
    flag = sq.sq_pool_last_device_error(case.pool)
    post = case.host()
    ref, o_ref, n_bad = case.oracle_step(pre, si, return_flagged=True)
    tally = Tally()
    case.compare(tally, post, ref)
    tally.add_o(o.cpu().numpy(), o_ref)
    say(f"[nonfinite {w.name}{' kda' if kda else ''}] {tally.summary()} oracle_flagged={n_bad} "
        f"flag={flag}")
    tally.check()
    assert tally.nonfinite > 0
    assert n_bad > 0 and flag == sq.SQ_ERR_DEVICE
    assert sq.sq_pool_last_device_error(case.pool) == sq.SQ_OK  # read and cleared
    # a clean step from the clean state leaves the flag clear (the FP16/BF16/FP32
    # tiles stepped above now hold non-finite values, which a further step
    # would report again)
    case.dev.copy_(torch.from_numpy(pre))
    case.step(case.inputs(1))
    assert sq.sq_pool_last_device_error(case.pool) == sq.SQ_OK
    return post, case


@pytest.mark.parametrize("shape", ["d128", "d128_mid", "odd"])
def test_non_finite_inputs_follow_the_rule(sq, orc, shape):
    """Caller errors with a defined result: a NaN quotient stores code 0, +-Inf
    the bound +-Q, FP16/BF16/FP32 elements the non-finite value; the pool's
    sticky flag reports it.  Every tile and every readout is compared."""
    mix = {4: 2, 6: 2, 8: 2, 16: 2, 32: 2, I.BITS_BF16: 2}
    if shape == "d128":
        w = I.Workload("nonfinite", 5, 12, 128, 128, 1, mix, seed=31)
    elif shape == "d128_mid":  # the 256-thread launch of the d = 128 step
        w = I.Workload("nonfinite_mid", 5, 240, 128, 128, 1,
                       {4: 60, 6: 100, 8: 60, 16: 8, 32: 6, I.BITS_BF16: 6}, seed=32)
    else:
        w = I.Workload("nonfinite_odd", 5, 12, 12, 20, 1, mix, seed=33)
    post, case = _nonfinite_case(sq, orc, w, n_slots=6, slots=[4, 0, 5, 2, 1])
    # request 0 (NaN gate): every code is 0, every unquantized element NaN
    for h in range(w.n_heads):
        b = int(case.bits[h])
        lo = int(case.slots[0]) * case.slab + int(case.off[h])
        f = unpack_fields(post[None, lo:lo + orc.tile_bytes(b, w.dk, w.dv)], b)
        if b <= 8:
            assert np.all(f == 2 ** (b - 1)), (h, b)


def test_non_finite_inputs_follow_the_rule_channel_gate(sq, orc):
    w = I.Workload("nonfinite_kda", 5, 12, 128, 128, 1,
                   {4: 2, 6: 2, 8: 2, 16: 2, 32: 2, I.BITS_BF16: 2}, seed=34)
    _nonfinite_case(sq, orc, w, kda=True, n_slots=5, slots=[3, 4, 0, 1, 2])


def test_non_finite_store(sq, orc):
    """sq_pool_store of NaN / +-Inf: codes 0 / +-Q, the value itself in FP16,
    BF16 and FP32 tiles, bit-exact with the oracle's store; the flag is set."""
    w = I.Workload("store_nf", 2, 6, 128, 128, 1, {4: 1, 6: 1, 8: 1, 16: 1, 32: 1, I.BITS_BF16: 1},
                   seed=35)
    case = Case(sq, orc, w)
    S = case.S0.copy()
    S[0, :, 0, :3] = [float("nan"), float("inf"), -float("inf")]
    S[1, :, 5, 7] = float("nan")
    case.dev.zero_()
    sq.sq_pool_store(case.pool, case.slots_d, torch.from_numpy(S).cuda())
    flag = sq.sq_pool_last_device_error(case.pool)
    got = case.host()
    want = np.zeros_like(got)
    n_bad = orc.store_pool(want, case.bits, w.dk, w.dv, case.r, case.c, case.slots, S)
    assert n_bad == 2 * w.n_heads and flag == sq.SQ_ERR_DEVICE
    tally = Tally()
    case.compare(tally, got, want)
    tally.check()
    for p in case.slots:  # every code tile bit-exact
        for h in range(w.n_heads):
            b = int(case.bits[h])
            if b <= 8:
                lo, tb = int(p) * case.slab + int(case.off[h]), orc.tile_bytes(b, w.dk, w.dv)
                assert np.array_equal(got[lo:lo + tb], want[lo:lo + tb]), (p, h)


# ------------------------------------------------------------------ per-slot scales

@pytest.mark.parametrize("dk,dv", [(128, 128), (12, 20)])
def test_per_slot_scales(sq, orc, dk, dv):
    """scale_slot_stride S > 0: every slot has its own row and column factors
    at vector p * S + h.  Store, steps, readout and load follow the slot's own
    factors (teacher-forced against the oracle at the same stride)."""
    mix = {4: 2, 6: 2, 8: 2, 16: 1, 32: 1, I.BITS_BF16: 1}
    w = I.Workload(f"stride{dk}x{dv}", 3, 9, dk, dv, 3, mix, seed=dk + 3 * dv)
    n_slots, slots, S = 5, [4, 1, 3], 9 + 3
    case = Case(sq, orc, w, n_slots=n_slots, slots=slots, scale_stride=S)
    # the store through the library matches the oracle's per-slot encoding
    ref = case.host()
    case.dev.zero_()
    sq.sq_pool_store(case.pool, case.slots_d, torch.from_numpy(case.S0).cuda())
    assert np.array_equal(case.host(), ref)
    run_teacher_forced(case, w.steps, f"stride {dk}x{dv}")
    host = case.host()
    si = I.step_inputs(w, 7)
    o = torch.empty(w.n_req, w.n_heads, dv, device="cuda")
    sq.sq_readout(case.pool, case.slots_d, si.q.cuda(), o)
    o_ref = orc.readout_pool(host, case.bits, dk, dv, case.r, case.c, case.slots, host_f32(si.q),
                             scale_stride=S)
    t = Tally()
    t.add_o(o.cpu().numpy(), o_ref)
    t.check()
    L = torch.empty(w.n_req, w.n_heads, dk, dv, device="cuda")
    sq.sq_pool_load(case.pool, case.slots_d, L)
    want = orc.load_pool(host, case.bits, dk, dv, case.r, case.c, case.slots, scale_stride=S)
    assert np.array_equal(L.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert sq.sq_pool_last_device_error(case.pool) == sq.SQ_OK


def test_per_slot_scales_channel_gate(sq, orc):
    w = I.Workload("stride_kda", 3, 9, 128, 128, 2, {4: 2, 6: 2, 8: 2, 16: 1, 32: 1, I.BITS_BF16: 1},
                   seed=91)
    case = KdaCase(sq, orc, w, n_slots=4, slots=[2, 3, 0], scale_stride=9)
    run_teacher_forced(case, w.steps, "stride kda")


def test_two_pools_on_two_streams(sq, orc):
    """The library keeps no global state: two pools stepped concurrently on two
    streams, from two host threads, end bit-identical to the same steps run
    one after the other on the default stream."""
    import threading

    w = I.scaled(I.WORKLOADS["layer"], 3, 12, 8)
    cases = [Case(sq, orc, w), Case(sq, orc, I.scaled(w, name="other"), slots=[2, 0, 1])]
    inits = [c.dev.clone() for c in cases]
    ins = [[I.step_inputs(w, t + 10 * k, "cuda") for t in range(w.steps)] for k in range(2)]

    def run(k, stream):
        c = cases[k]
        with torch.cuda.stream(stream):
            for si in ins[k]:
                sq.sq_decode_step(c.pool, c.slots_d, si.q, si.k, si.v, si.alpha, si.beta, None,
                                  stream)

    for k in range(2):
        run(k, torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = [c.dev.clone() for c in cases]
    for c, i0 in zip(cases, inits):
        c.dev.copy_(i0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    th = [threading.Thread(target=run, args=(k, streams[k])) for k in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    for c, wnt in zip(cases, want):
        assert torch.equal(c.dev, wnt)


def test_saturating_updates(sq, orc):
    """Writes far outside the scales' range: most codes of the written rows
    clamp to +-Q, and the clamp decision matches the oracle's."""
    w = I.Workload("sat", 2, 12, 128, 128, 3, {4: 2, 6: 2, 8: 2, 16: 2, 32: 2, I.BITS_BF16: 2},
                   seed=41)
    case = Case(sq, orc, w)
    tally = Tally()
    saturated = 0
    for t in range(w.steps):
        si = I.step_inputs(w, t)
        si.v = (si.v.float() * 200.0).to(si.v.dtype)
        si.beta.fill_(1.0)
        pre = case.host()
        o = case.step(si)
        post = case.host()
        ref, o_ref = case.oracle_step(pre, si)
        case.compare(tally, post, ref)
        tally.add_o(o.cpu().numpy(), o_ref)
        for h in range(w.n_heads):
            b = int(case.bits[h])
            if b <= 8:
                tb = orc.tile_bytes(b, 128, 128)
                f = unpack_fields(post[None, int(case.off[h]):int(case.off[h]) + tb], b)
                saturated += int(((f == 1) | (f == 2 ** b - 1)).sum())
    tally.check()
    assert saturated > 1000  # the clamp path was exercised


def test_mid_size_launch_takes_256_threads(sq, orc):
    """1,024-16,383 tiles take the 256-thread launch of the d = 128 step
    (four blocks per thread): same parity bar, every width, scrambled slots."""
    w = I.Workload("mid", 4, 400, 128, 128, 3,
                   {4: 96, 6: 196, 8: 96, 16: 4, 32: 4, I.BITS_BF16: 4}, seed=51)
    assert 1024 <= w.n_req * w.n_heads < 16384
    run_teacher_forced(Case(sq, orc, w, n_slots=6, slots=[5, 0, 3, 1]), w.steps, "mid")


@pytest.mark.parametrize("n_req,H", [(3, 100), (8, 150), (111, 150), (421, 40)])
def test_head_groups_of_unequal_size(sq, orc, n_req, H):
    """Pools of 64 or more heads split the heads of every request into 8 XCD
    groups; with H not a multiple of 8 the groups differ in size (12/13 and
    18/19 heads) and the rounded-up grid has surplus workgroups.  Every tile
    must still be stepped exactly once: 300 tiles (128-thread launch), 1,200
    tiles (256-thread launch), and 16,650 and 16,840 tiles (two tiles per
    workgroup; an odd tile count per XCD leaves the last workgroup half
    empty, and 40 heads take the contiguous-eighths order), every width,
    scrambled slots."""
    mix = {4: H // 4, 6: H // 4, 8: H // 4, 16: 2, 32: 2}
    mix[I.BITS_BF16] = H - sum(mix.values())
    w = I.Workload(f"h{H}", n_req, H, 128, 128, 2, mix, seed=H)
    slots = list(range(n_req + 1))[::-1][:n_req]
    run_teacher_forced(Case(sq, orc, w, n_slots=n_req + 1, slots=slots), w.steps, f"h{H}")


BOUNDARY_MIXES = {  # n_req x H = the tile count of the launch; about 1:2:1 + 1.4 % pivots
    (3, 341): {4: 84, 6: 168, 8: 83, 16: 4, 32: 1, I.BITS_BF16: 1},   # 1,023: 128 threads per tile
    (2, 512): {4: 126, 6: 252, 8: 126, 16: 6, 32: 1, I.BITS_BF16: 1},  # 1,024: 256 threads per tile
    (43, 381): {4: 94, 6: 188, 8: 93, 16: 4, 32: 1, I.BITS_BF16: 1},   # 16,383: 256 threads per tile
    (64, 256): {4: 63, 6: 126, 8: 62, 16: 3, 32: 1, I.BITS_BF16: 1},   # 16,384: two tiles per workgroup
}


BOUNDARY_CASES = [(shape, "bf16") for shape in BOUNDARY_MIXES] + [((2, 512), "f32"), ((64, 256), "f32")]


@pytest.mark.parametrize("kda", [False, True], ids=["scalar_gate", "channel_gate"])
@pytest.mark.parametrize("shape,qkv", BOUNDARY_CASES, ids=lambda c: f"{c[0] * c[1]}_tiles"
                         if isinstance(c, tuple) else c)
def test_launch_size_boundaries(sq, orc, shape, qkv, kda):
    """One step on each side of the two tile counts where the d = 128 launch
    changes shape (1,024 and 16,384 tiles), every tile compared with the
    oracle (whole-pool byte comparison; only differing code tiles unpacked);
    fp32 q/k/v as well as bf16 for the two larger launch shapes."""
    from gpu_harness import compare_pools_fast
    n_req, H = shape
    w = I.Workload(f"edge{n_req * H}", n_req, H, 128, 128, 1, BOUNDARY_MIXES[shape], qkv_dtype=qkv,
                   seed=n_req + H)
    assert sum(BOUNDARY_MIXES[shape].values()) == H
    case = (KdaCase if kda else Case)(sq, orc, w, n_slots=n_req + 1, slots=list(range(1, n_req + 1)))
    si = case.inputs(0)
    pre = case.host()
    if not kda:  # the readout-only instance of the same launch shape, before the step
        o_r = torch.empty(n_req, H, w.dv, device="cuda")
        sq.sq_readout(case.pool, case.slots_d, si.q.cuda(), o_r)
        t_r = Tally()
        t_r.add_o(o_r.cpu().numpy(), orc.readout_pool(pre, case.bits, w.dk, w.dv, case.r, case.c,
                                                      case.slots, host_f32(si.q), n_threads=16))
        t_r.check()
        assert np.array_equal(case.host(), pre)
    o = case.step(si)
    post = case.host()
    ref, o_ref = case.oracle_step(pre, si)
    tally = Tally()
    compare_pools_fast(tally, post, ref, case.bits, case.off, case.slab, case.slots, w.dk, w.dv)
    tally.add_o(o.cpu().numpy(), o_ref)
    say(f"edge {n_req}x{H} kda={kda}: {tally.summary()}")
    tally.check()
    assert tally.tiles == n_req * H
    assert np.array_equal(post[:case.slab], pre[:case.slab])  # slot 0 is not in the batch


@pytest.mark.parametrize("dk,dv", [(12, 20), (64, 128), (256, 32)])
def test_readout_other_shapes(sq, orc, dk, dv):
    """sq_readout through the any-shape kernel, every width: o = S^T q of the
    stored state, the pool unchanged."""
    w = I.Workload("ro", 3, 6, dk, dv, 1, {4: 1, 6: 1, 8: 1, 16: 1, 32: 1, I.BITS_BF16: 1},
                   seed=dk * 7 + dv)
    case = Case(sq, orc, w, n_slots=4, slots=[3, 0, 2])
    case.step(I.step_inputs(w, 0))  # read a state that has been through a step
    start = case.host()
    si = I.step_inputs(w, 1)
    o = torch.empty(w.n_req, w.n_heads, dv, device="cuda")
    sq.sq_readout(case.pool, case.slots_d, si.q.cuda(), o)
    torch.cuda.synchronize()
    assert np.array_equal(case.host(), start)
    o_ref = orc.readout_pool(start, case.bits, dk, dv, case.r, case.c, case.slots, host_f32(si.q))
    t = Tally()
    t.add_o(o.cpu().numpy(), o_ref)
    say(f"[readout {dk}x{dv}] {t.summary()}")
    t.check()
