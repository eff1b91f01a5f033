"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (one sq_decode_step over the whole batch).

The pools are initialised on the GPU with sq_pool_store; sampled tiles of the
store are checked bit-exact against the oracle's encoding of the same fp32
states.  On checked steps, sampled tiles (every head of one request plus a
random set covering every width) are copied back before and after the step
and the oracle steps them, teacher-forced, with the same inputs."""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

from gpu_harness import Tally, host_f32, say
from quantized_recurrent_state_gated_amd import inputs as I

pytestmark = pytest.mark.gpu
THREADS = 16


@pytest.fixture(scope="module")
def sq():
    from quantized_recurrent_state_gated_amd import sq as m
    return m


class DevicePool:
    def __init__(self, sq, w):
        self.sq, self.w = sq, w
        self.bits = I.head_bits(w)
        self.r, self.c = I.scales(w, device="cuda")
        nbytes = sq.sq_pool_bytes(w.n_req, w.n_heads, w.dk, w.dv, self.bits)
        self.state = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.pool = sq.sq_pool_alloc(w.n_req, w.n_heads, w.dk, w.dv, self.bits, self.r, self.c,
                                     self.state)
        self.slots = torch.arange(w.n_req, dtype=torch.int32, device="cuda")
        for p in range(w.n_req):
            sq.sq_pool_store(self.pool, self.slots[p:p + 1], I.initial_state(w, p, "cuda"))
        torch.cuda.synchronize()
        self.rh, self.ch = self.r.cpu().numpy(), self.c.cpu().numpy()

    def tile_bytes(self, tiles):
        """uint8 copies of tiles [(n, h)] (slot n holds request n)."""
        out = []
        for n, h in tiles:
            off, nb = self.sq.sq_pool_tile_offset(self.pool, int(n), int(h))
            out.append(self.state[off:off + nb])
        return [t.cpu().numpy() for t in out]


def sample(w, bits, rng, n_random):
    tiles = [(int(rng.integers(w.n_req)), h) for h in range(w.n_heads)]
    tiles += [(int(rng.integers(w.n_req)), int(rng.integers(w.n_heads))) for _ in range(n_random)]
    for b in sorted(set(int(x) for x in bits)):  # every width, several requests
        hs = np.nonzero(bits == b)[0]
        tiles += [(int(rng.integers(w.n_req)), int(rng.choice(hs))) for _ in range(8)]
    return sorted(set(tiles))


def check_store(orc, dp, tiles):
    w = dp.w
    got = dp.tile_bytes(tiles)
    by_req = {}
    for (n, h), g in zip(tiles, got):
        by_req.setdefault(n, []).append((h, g))
    for n, lst in by_req.items():
        S0 = I.initial_state(w, n, "cuda").cpu().numpy()
        for h, g in lst:
            want = orc.encode_tile(int(dp.bits[h]), w.dk, w.dv, S0[h].astype(np.float64), dp.rh[h],
                                   dp.ch[h])
            assert np.array_equal(g, want), f"store tile ({n}, {h}) bits {dp.bits[h]}"


def check_step(orc, dp, tiles, si, pre, post, o, tally, kda=False):
    w = dp.w
    q, k, v = host_f32(si.q), host_f32(si.k), host_f32(si.v)
    al, be = si.alpha.cpu().numpy(), si.beta.cpu().numpy()
    o_gpu = o.cpu().numpy()

    def one(i):
        n, h = tiles[i]
        step = orc.step_tile_kda if kda else orc.step_tile
        return step(int(dp.bits[h]), w.dk, w.dv, pre[i], dp.rh[h], dp.ch[h], q[n, h], k[n, h],
                    v[n, h], al[n, h], be[n, h])

    with cf.ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(one, range(len(tiles))))
    for b in sorted(set(int(x) for x in dp.bits)):
        idx = [i for i, (n, h) in enumerate(tiles) if dp.bits[h] == b]
        tally.add_tiles(np.stack([post[i] for i in idx]), np.stack([res[i][0] for i in idx]), b)
    tally.add_o(np.stack([o_gpu[n, h] for n, h in tiles]), np.stack([r[1] for r in res]))


def run_fullsize(sq, orc, name, check_steps, n_random=2048, all_tiles_at=(), kda=False):
    """kda: step with sq_decode_step_kda and per-channel gates I.channel_gates."""
    w = I.WORKLOADS[name]
    say(f"[{name}{' kda' if kda else ''}] init {w.n_req} x {w.n_heads}")
    dp = DevicePool(sq, w)
    rng = np.random.default_rng(7)
    tiles = sample(w, dp.bits, rng, n_random)
    check_store(orc, dp, tiles)
    say(f"[{name}] store bit-exact on {len(tiles)} sampled tiles")
    o = torch.empty(w.n_req, w.n_heads, w.dv, device="cuda")
    tally = Tally()
    every = [(n, h) for n in range(w.n_req) for h in range(w.n_heads)]
    for t in range(max(check_steps) + 1):
        si = I.step_inputs(w, t, "cuda")
        if kda:
            si.alpha = I.channel_gates(w, t, "cuda")
        check = t in check_steps
        sel = every if t in all_tiles_at else tiles
        if check:
            pre = dp.tile_bytes(sel)
        step = sq.sq_decode_step_kda if kda else sq.sq_decode_step
        step(dp.pool, dp.slots, si.q, si.k, si.v, si.alpha, si.beta, o)
        if check:
            torch.cuda.synchronize()
            post = dp.tile_bytes(sel)
            check_step(orc, dp, sel, si, pre, post, o, tally, kda)
            say(f"[{name}] step {t} ({len(sel)} tiles): {tally.summary()}")
    tally.check()


def test_serving_full_size(sq, orc):
    run_fullsize(sq, orc, "serving", check_steps=(0, 1, 63))


def test_highconc_full_size(sq, orc):
    run_fullsize(sq, orc, "highconc", check_steps=(0, 1, 31))


def test_drift_full_length(sq, orc):
    """2048 steps; every tile checked at steps 0, 1, 1024, 2047, a sample of
    tiles every 128 steps."""
    steps = tuple(range(0, 2048, 128)) + (1, 1024, 2047)
    run_fullsize(sq, orc, "drift", check_steps=steps, n_random=256, all_tiles_at=(0, 1, 1024, 2047))


def test_serving_full_size_channel_gate(sq, orc):
    """The per-key-channel-gate step at the serving size, in the launch bench.py times."""
    run_fullsize(sq, orc, "serving", check_steps=(0, 1, 31), kda=True)


def test_highconc_full_size_channel_gate(sq, orc):
    """The per-key-channel-gate step at 256 x 2304 heads (88 % 4-bit)."""
    run_fullsize(sq, orc, "highconc", check_steps=(0, 1, 15), kda=True)


def test_serving_readout_full_size(sq, orc):
    """sq_readout over the whole serving pool after two steps: o = S^T q from
    the stored state, on sampled tiles of every width; the pool is unchanged."""
    w = I.WORKLOADS["serving"]
    say(f"[serving readout] init {w.n_req} x {w.n_heads}")
    dp = DevicePool(sq, w)
    for t in range(2):
        si = I.step_inputs(w, t, "cuda")
        sq.sq_decode_step(dp.pool, dp.slots, si.q, si.k, si.v, si.alpha, si.beta, None)
    si = I.step_inputs(w, 2, "cuda")
    rng = np.random.default_rng(11)
    tiles = sample(w, dp.bits, rng, 2048)
    before = dp.tile_bytes(tiles)
    o = torch.empty(w.n_req, w.n_heads, w.dv, device="cuda")
    sq.sq_readout(dp.pool, dp.slots, si.q, o)
    torch.cuda.synchronize()
    after = dp.tile_bytes(tiles)
    assert all(np.array_equal(a, b) for a, b in zip(before, after)), "readout wrote the pool"
    q, o_gpu = host_f32(si.q), o.cpu().numpy()

    def one(i):
        n, h = tiles[i]
        return orc.readout_tile(int(dp.bits[h]), w.dk, w.dv, before[i], dp.rh[h], dp.ch[h], q[n, h])

    with cf.ThreadPoolExecutor(THREADS) as ex:
        ref = list(ex.map(one, range(len(tiles))))
    tally = Tally()
    tally.add_o(np.stack([o_gpu[n, h] for n, h in tiles]), np.stack(ref))
    say(f"[serving readout] {len(tiles)} tiles: {tally.summary()}")
    assert tally.o_worst <= 1.0, tally.summary()
