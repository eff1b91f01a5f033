"""sq_check_slots_noalloc, the slot check that allocates nothing: its stamps
live in a fixed device array inside the library.  Checked against
sq_check_slots (the pool-table version) call by call, over two calls in a row
with the second one smaller, and again after many calls; host-side argument
errors are checked without a GPU."""
import ctypes

import numpy as np
import pytest
import torch



@pytest.fixture(scope="module")
def sq():
    from quantized_recurrent_state_gated_amd import sq as m
    return m


def test_noalloc_host_errors(sq):
    lib = sq._lib
    res = ctypes.c_void_p(0x1000)
    assert lib.sq_check_slots_noalloc(None, 0, 4, None, None) == sq.SQ_ERR_INVALID
    assert lib.sq_check_slots_noalloc(None, -1, 4, res, None) == sq.SQ_ERR_INVALID
    assert lib.sq_check_slots_noalloc(None, 2, 4, res, None) == sq.SQ_ERR_INVALID
    assert lib.sq_check_slots_noalloc(None, 0, 0, res, None) == sq.SQ_ERR_INVALID
    assert lib.sq_check_slots_noalloc(None, 0, 4, ctypes.c_void_p(0x1002), None) == sq.SQ_ERR_INVALID
    assert lib.sq_check_slots_noalloc(None, 0, 65537, res, None) == sq.SQ_ERR_UNSUPPORTED


def _pool(sq, n_slots):
    """A small pool (one 16 x 16 INT8 head per slot) with n_slots slots."""
    bits = np.array([8], np.uint8)
    r = torch.ones(1, 16, device="cuda")
    c = torch.ones(1, 16, device="cuda")
    state = torch.zeros(sq.sq_pool_bytes(n_slots, 1, 16, 16, bits), dtype=torch.uint8,
                        device="cuda")
    return sq.sq_pool_alloc(n_slots, 1, 16, 16, bits, r, c, state), state, r, c


@pytest.mark.gpu
def test_noalloc_matches_pool_check(sq):
    """Two calls in a row, the second with a smaller batch and fewer slots,
    each compared with sq_check_slots on a pool of the same slot count; then
    a long run of mixed calls, so that the shared array is reused."""
    rng = np.random.default_rng(20261203)
    pools = {}

    def both(ids, n_slots):
        if n_slots not in pools:
            pools[n_slots] = _pool(sq, n_slots)
        pool = pools[n_slots][0]
        t = torch.tensor(ids, dtype=torch.int32, device="cuda")
        a = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        b = torch.full((1,), -9, dtype=torch.int32, device="cuda")
        sq.sq_check_slots(pool, t, a)
        sq.sq_check_slots_noalloc(t, n_slots, b)
        torch.cuda.synchronize()
        return int(a.item()), int(b.item())

    # first call: a large valid batch, then a smaller one with a repeat
    ids = rng.permutation(3000)[:2500].tolist()
    assert both(ids, 3000) == (0, 0)
    assert both([5, 7, 5], 40) == (2, 2)
    # the stamps the first call left must not leak into later ones
    assert both(ids[:40], 3000) == (0, 0)
    assert both([1, 2, 3], 4) == (0, 0)
    cases = [([], 10), ([9], 10), ([10], 10), ([-1, 3], 10), ([4, 11, 4], 10),
             (list(range(65536))[::-1], 65536), ([65535, 0, 65535], 65536)]
    for ids_, n in cases:
        a, b = both(ids_, n)
        assert a == b, (ids_[:8], n, a, b)
    for it in range(60):
        n = int(rng.integers(1, 5000))
        m = int(rng.integers(0, min(n, 3000) + 1))
        ids_ = rng.integers(0, n, m) if it % 3 == 0 else rng.permutation(n)[:m]
        if it % 5 == 0 and m:
            ids_ = ids_.copy()
            ids_[0] = n + int(rng.integers(0, 3))  # out of range
        a, b = both(ids_.tolist(), n)
        assert a == b, (it, n, m, a, b)
