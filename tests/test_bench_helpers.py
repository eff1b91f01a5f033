"""Host-side helpers of bench.py: the counter summary, the stale-profile rule
and the saturated-code report (on CPU tensors with an oracle-built pool)."""
import csv
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _pmc_csv(path, rows):
    """rows: (kernel, counter, value); a new dispatch starts at each kernel's
    first counter of the pass."""
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        wr.writeheader()
        seen, did = set(), 0
        for name, counter, val in rows:
            if (name, counter) in seen or not seen:
                did += 1
                seen = set()
            seen.add((name, counter))
            wr.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": val})


def test_pmc_summary_counts_bytes_by_request_size_and_picks_exact_kernels(tmp_path, monkeypatch):
    step = "void sqk::" + bench.STEP_KERNEL + "(sqk::FusedArgs)"
    kda = "void sqk::" + bench.KDA_KERNEL + "(sqk::FusedArgs)"
    f32 = "void sqk::k_step128_f32<unsigned short, true, false>(sqk::StepArgs)"
    copy = "__amd_rocclr_copyBuffer"
    conv = "void at::native::vectorized_elementwise_kernel<4, at::native::copy_kernel_impl>"
    r32, r64, r128, rall = bench.READ_COUNTERS
    w64, wall, bub = bench.WRITE_COUNTERS
    rd, wr = [], []
    # step: three dispatches (median taken); reads 10 x 32 B + 20 x 64 B + 100 x 128 B
    for n128 in (99, 100, 101):
        rd += [(step, r32, 10), (step, r64, 20), (step, r128, n128), (step, rall, 130 + n128 - 100)]
        wr += [(step, w64, 200), (step, wall, 204), (step, bub, n128)]
    rd += [(kda, r32, 0), (kda, r64, 0), (kda, r128, 50), (kda, rall, 50)]
    wr += [(kda, w64, 100), (kda, wall, 100), (kda, bub, 50)]
    gib128 = (1 << 30) // 128
    for v in (3, gib128):  # a small blit and the 1 GiB copy: the largest is taken
        rd += [(copy, r32, 0), (copy, r64, 0), (copy, r128, v), (copy, rall, v)]
        wr += [(copy, w64, 2 * v), (copy, wall, 2 * v), (copy, bub, v)]
    for other in (f32, conv):
        rd += [(other, c, 9e9) for c in bench.READ_COUNTERS]
        wr += [(other, c, 9e9) for c in bench.WRITE_COUNTERS]
    _pmc_csv(tmp_path / "r.csv", rd)
    _pmc_csv(tmp_path / "w.csv", wr)
    monkeypatch.setattr(bench, "traffic_file", lambda wl: str(tmp_path / f"traffic_{wl}.json"))
    assert bench.pmc_summary(str(tmp_path / "r.csv"), str(tmp_path / "w.csv"), "highconc") == 0
    t = json.load(open(tmp_path / "traffic_highconc.json"))
    assert t["workload"] == "highconc"
    assert all(c.endswith("--copy-calibration --workload highconc") for c in t["commands"])
    assert t["step"]["fetch_bytes_per_launch"] == 10 * 32 + 20 * 64 + 100 * 128
    assert t["step"]["write_bytes_per_launch"] == 200 * 64 + 4 * 32
    assert t["step"]["dispatches"] == [3, 3]
    assert t["step"]["reads_by_size_sum_to_all"] and t["step"]["tcc_bubble_reads"] == 100
    assert t["channel_gate_step"]["hbm_bytes_per_launch"] == 50 * 128 + 100 * 64
    assert t["copy"]["fetch_bytes_per_launch"] == 1 << 30
    assert t["copy"]["write_bytes_per_launch"] == 1 << 30
    # the profile is used only for the kernel source and the workload it was taken on
    sha = t["kernel_source_sha"]
    assert bench.traffic_from_profile(sha, "highconc") == t["step"]["hbm_bytes_per_launch"]
    assert bench.traffic_from_profile("0" * 16, "highconc") is None
    assert bench.traffic_from_profile(sha, "serving") is None
    assert bench.traffic_from_profile(sha, "highconc", "channel_gate_step") is not None


class _FakeSq:
    def __init__(self, off, bits, dk, dv):
        self.off, self.bits, self.dk, self.dv = off, bits, dk, dv

    def sq_pool_tile_offset(self, pool, slot, head):
        assert slot == 0
        return int(self.off[head]), self.dk * self.dv * int(self.bits[head]) // 8


class _W:
    n_req = 3


def test_saturation_counts_codes_at_the_range_ends(orc):
    bits = np.array([4, 6, 8, 6, 16], np.uint8)
    dk = dv = 8
    off, slab = orc.pool_layout(bits, dk, dv)
    rng = np.random.default_rng(5)
    pool = np.zeros(3 * slab, np.uint8)
    want = {}
    for b in (4, 6, 8):
        Q = 2 ** (b - 1) - 1
        sat = tot = 0
        for h in np.nonzero(bits == b)[0]:
            for p in range(3):
                codes = rng.integers(-Q, Q + 1, (dk, dv))
                sat += int((np.abs(codes) == Q).sum())
                tot += codes.size
                r, c = np.ones(dk, np.float32), np.ones(dv, np.float32)
                t = orc.encode_tile(b, dk, dv, codes.astype(np.float64), r, c)
                pool[p * slab + off[h]:p * slab + off[h] + t.size] = t
        want[str(b)] = sat / tot
    got = bench.saturation(_FakeSq(off, bits, dk, dv), _W(), bits, None, torch.from_numpy(pool))
    assert got.keys() == want.keys()
    for b in want:
        assert abs(got[b] - want[b]) < 1e-12, (b, got[b], want[b])


def test_cpu_baseline_times_full_steps_on_n_threads_and_one(orc):
    from quantized_recurrent_state_gated_amd import inputs as I
    w = I.scaled(I.WORKLOADS["layer"], 4, 6, 1)
    bits = I.head_bits(w)
    r, c = (x.numpy() for x in I.scales(w))
    off, slab = orc.pool_layout(bits, w.dk, w.dv)
    pool = np.zeros(w.n_req * slab, np.uint8)
    S0 = torch.stack([I.initial_state(w, p) for p in range(w.n_req)]).numpy()
    orc.store_pool(pool, bits, w.dk, w.dv, r, c, np.arange(w.n_req, dtype=np.int32), S0)
    before = pool.copy()
    w2 = I.scaled(I.WORKLOADS["layer"], 2, 3, 1)
    w2 = type(w2)(**{**w2.__dict__, "name": "other"})
    bits2 = I.head_bits(w2)
    r2, c2 = (x.numpy() for x in I.scales(w2))
    _, slab2 = orc.pool_layout(bits2, w2.dk, w2.dv)
    pool2 = np.zeros(w2.n_req * slab2, np.uint8)
    out = bench.cpu_baseline(w, bits, pool, r, c, [I.step_inputs(w, t) for t in range(2)], 2,
                             "two threads", (w2, bits2, pool2, r2, c2, [I.step_inputs(w2, 0)]))
    assert np.array_equal(pool, before)  # the caller's image is not stepped
    assert out["kind"] == "oracle" and out["cores"] == 2 and out["value"] > 0
    assert out["cores_why"] == "two threads"
    assert out["sample"].startswith(f"2 full decode steps of {w.name} ({w.n_req} requests")
    assert out["one_core"]["value"] > 0
    assert out["one_core"]["sample"].startswith(f"{w.n_req // 2} of {w.n_req} requests")
    assert out["other"]["value"] > 0 and out["other"]["sample"].startswith("1 full decode step")


def test_cpu_threads_follow_the_stated_share(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "16")
    n, why = bench.cpu_threads()
    assert n == 16 and "OMP_NUM_THREADS=16" in why
    monkeypatch.delenv("OMP_NUM_THREADS")
    n, why = bench.cpu_threads()
    assert n == len(os.sched_getaffinity(0)) and "affinity" in why
    assert bench.cpu_threads(3)[0] == 3
