"""The step is a pure function of its inputs: run twice from the same pool
bytes with the same inputs, it writes the same bytes and the same readout,
bit for bit.  Checked for the scalar and the per-channel gate at the three
launch sizes of the d = 128 kernels (under 1,024 tiles, 1,024-16,383 tiles,
16,384 tiles and more), several steps in a row, so that a result that
depends on timing (a register read or overwritten too early, a race between
the waves of a tile) shows up as a difference between the two runs.  Every
head width is present, FP32- and BF16-state heads included."""
import numpy as np
import pytest
import torch

from gpu_harness import Case, KdaCase
from quantized_recurrent_state_gated_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    from quantized_recurrent_state_gated_amd import sq as m
    return m


def _run(case, ins, kda):
    step = case.sq.sq_decode_step_kda if kda else case.sq.sq_decode_step
    outs = []
    for si in ins:
        o = torch.empty(case.w.n_req, case.w.n_heads, case.w.dv, device="cuda")
        step(case.pool, case.slots_d, si.q, si.k, si.v, si.alpha, si.beta, o)
        outs.append(o)
    torch.cuda.synchronize()
    return case.dev.cpu().numpy(), torch.stack(outs).cpu().numpy()


SHAPES = {  # tiles: (requests, heads per width, steps)
    "96_tiles": (4, {4: 5, 6: 8, 8: 5, 16: 2, 32: 2, I.BITS_BF16: 2}, 4),
    "2400_tiles": (40, {4: 14, 6: 26, 8: 14, 16: 2, 32: 2, I.BITS_BF16: 2}, 3),
    "16800_tiles": (70, {4: 60, 6: 110, 8: 60, 16: 4, 32: 3, I.BITS_BF16: 3}, 2),
}


@pytest.mark.parametrize("kda", [False, True], ids=["scalar_gate", "channel_gate"])
@pytest.mark.parametrize("shape", list(SHAPES))
def test_two_runs_write_the_same_bytes(sq, orc, kda, shape):
    n_req, counts, steps = SHAPES[shape]
    w = I.Workload(f"rep{shape}", n_req, sum(counts.values()), 128, 128, steps, counts, seed=77 + n_req)
    case = (KdaCase if kda else Case)(sq, orc, w)
    ins = []
    for t in range(steps):
        si = I.step_inputs(w, t, "cuda")
        if kda:
            si.alpha = I.channel_gates(w, t, "cuda")
        ins.append(si)
    init = case.dev.clone()
    first = _run(case, ins, kda)
    for rep in range(2):
        case.dev.copy_(init)
        torch.cuda.synchronize()
        again = _run(case, ins, kda)
        assert np.array_equal(again[0], first[0]), f"run {rep + 2}: pool bytes differ"
        assert np.array_equal(again[1].view(np.uint32), first[1].view(np.uint32)), \
            f"run {rep + 2}: readout differs"
    assert not np.array_equal(first[0], init.cpu().numpy())  # the steps did update the pool
