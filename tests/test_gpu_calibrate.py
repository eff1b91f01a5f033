"""calibrate() end to end on the GPU: the FP32-state calibration decode runs
through the HIP step and sq_pool_load, the spatial fit and the allocation
run on the result, and the tables it returns drive a pool that steps at the
parity bar against the oracle."""
import numpy as np
import pytest

from gpu_harness import Case, run_teacher_forced
from quantized_recurrent_state_gated_amd import calibrate as C
from quantized_recurrent_state_gated_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    from quantized_recurrent_state_gated_amd import sq as m
    return m


def test_calibrate_end_to_end(sq, orc):
    w = I.scaled(I.WORKLOADS["layer"], 3, 16, 4)
    budget, n_piv = 6.0, 1
    out = C.calibrate(w, budget, n_piv, steps=64, stride=16, n_req=3, iters=2)
    bits, r, c, rep = out["bits"], out["r"], out["c"], out["report"]
    assert bits.shape == (w.n_heads,) and int((bits == 16).sum()) == n_piv
    assert set(int(b) for b in bits) <= {4, 6, 8, 16}
    q = bits[bits <= 8].astype(int)
    assert q.sum() <= round(budget * q.size)                 # within the bit budget
    assert rep["weighted_distortion"] <= rep["weighted_distortion_maxabs"] * (1 + 1e-9)
    assert bool((r > 0).all()) and bool((c > 0).all())
    # the tables are usable as they are: a pool with these widths and factors
    case = Case(sq, orc, w, bits=bits, scales=(r.cpu().numpy(), c.cpu().numpy()))
    run_teacher_forced(case, w.steps, "calibrated")
