"""The step under HIP graph capture: sq_decode_step, sq_decode_step_kda and
sq_check_slots make no allocation, copy, memset or synchronization, so a
serving loop can capture several steps once and replay them.  Every replay is
checked bit for bit against the same steps run eagerly (the kernels are
deterministic), with the program's own eager work and synchronizations between
replays."""
import numpy as np
import pytest
import torch

from gpu_harness import Case
from quantized_recurrent_state_gated_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    from quantized_recurrent_state_gated_amd import sq as m
    return m


def _inputs(w, steps, kda):
    out = []
    for t in range(steps):
        si = I.step_inputs(w, t, "cuda")
        if kda:
            si.alpha = I.channel_gates(w, t, "cuda")
        out.append(si)
    return out


@pytest.mark.parametrize("kda", [False, True])
def test_graph_replay_matches_eager(sq, orc, kda):
    w = I.scaled(I.WORKLOADS["layer"], 4, 24, 6)
    case = Case(sq, orc, w)
    init = case.dev.clone()
    ins = _inputs(w, w.steps, kda)
    step = sq.sq_decode_step_kda if kda else sq.sq_decode_step
    outs = [torch.empty(w.n_req, w.n_heads, w.dv, device="cuda") for _ in range(w.steps)]
    flag = torch.full((1,), -1, dtype=torch.int32, device="cuda")

    def run():
        sq.sq_check_slots(case.pool, case.slots_d, flag)
        for si, o in zip(ins, outs):
            step(case.pool, case.slots_d, si.q, si.k, si.v, si.alpha, si.beta, o)

    # eager reference
    run()
    torch.cuda.synchronize()
    want_state = case.dev.clone()
    want_o = [o.clone() for o in outs]
    assert int(flag.item()) == 0

    # capture (on torch's capture stream: the binding passes the current stream)
    case.dev.copy_(init)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        case.dev.copy_(init)
        for o in outs:
            o.fill_(float("nan"))
        flag.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(case.dev, want_state), f"replay {rep}: state"
        for t, (o, ref) in enumerate(zip(outs, want_o)):
            assert torch.equal(o, ref), f"replay {rep}: o of step {t}"
        assert int(flag.item()) == 0, f"replay {rep}: slot check"
        # eager work between replays
        sq.sq_readout(case.pool, case.slots_d, ins[0].q, outs[0])
        torch.cuda.synchronize()


def test_graph_replayed_slot_check_still_flags_repeats(sq, orc):
    w = I.scaled(I.WORKLOADS["layer"], 2, 6, 1)
    case = Case(sq, orc, w, n_slots=5, slots=[1, 3])
    ids = torch.tensor([4, 0, 4], dtype=torch.int32, device="cuda")
    flag = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sq.sq_check_slots(case.pool, ids, flag)
    for _ in range(3):
        flag.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert int(flag.item()) == 2
        ids[2] = 1  # a valid batch on the next replay
        g.replay()
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        ids[2] = 4
