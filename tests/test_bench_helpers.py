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


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, val in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val})


def test_pmc_summary_scales_by_the_copy_and_picks_exact_kernels(tmp_path, monkeypatch):
    step = "void sqk::" + bench.STEP_KERNEL + "(sqk::FusedArgs)"
    kda = "void sqk::" + bench.KDA_KERNEL + "(sqk::FusedArgs)"
    f32 = "void sqk::k_step128_f32<unsigned short, true, false>(sqk::StepArgs)"
    copy = "__amd_rocclr_copyBuffer"
    gib = 1 << 20  # KiB in 1 GiB
    conv = "void at::native::vectorized_elementwise_kernel<4, at::native::copy_kernel_impl>"
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE",
             [(copy, 3), (copy, gib / 2), (step, 1000), (step, 1002), (step, 998), (kda, 1100),
              (f32, 9e9), (conv, 5e9)])
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE",
             [(copy, 2), (copy, gib), (step, 2000), (step, 2000), (kda, 2000), (f32, 9e9),
              (conv, 5e9)])
    monkeypatch.setattr(bench, "traffic_file", lambda wl: str(tmp_path / f"traffic_{wl}.json"))
    assert bench.pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "highconc") == 0
    t = json.load(open(tmp_path / "traffic_highconc.json"))
    assert t["workload"] == "highconc"
    assert all(c.endswith("--copy-calibration --workload highconc") for c in t["commands"])
    assert t["fetch_factor"] == 2.0 and t["write_factor"] == 1.0
    assert t["step"]["fetch_bytes_per_launch"] == 2.0 * 1000 * 1024  # median, scaled
    assert t["step"]["write_bytes_per_launch"] == 2000 * 1024
    assert t["step"]["dispatches"] == [3, 2]
    assert t["channel_gate_step"]["hbm_bytes_per_launch"] == (2.0 * 1100 + 2000) * 1024
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


def test_cpu_baseline_times_the_oracle_on_n_threads_and_one(orc):
    from quantized_recurrent_state_gated_amd import inputs as I
    w = I.scaled(I.WORKLOADS["layer"], 4, 6, 1)
    bits = I.head_bits(w)
    r, c = (x.numpy() for x in I.scales(w))
    off, slab = orc.pool_layout(bits, w.dk, w.dv)
    pool = np.zeros(w.n_req * slab, np.uint8)
    S0 = torch.stack([I.initial_state(w, p) for p in range(w.n_req)]).numpy()
    orc.store_pool(pool, bits, w.dk, w.dv, r, c, np.arange(w.n_req, dtype=np.int32), S0)
    si = I.step_inputs(w, 0)
    out = bench.cpu_baseline(w, bits, lambda n: pool[: n * slab].copy(), r, c, si, 2, 1e3)
    assert out["kind"] == "oracle" and out["cores"] == 2 and out["value"] > 0
    assert out["sample"].startswith(f"{w.n_req} of {w.n_req} requests")  # capped at the workload
    assert out["one_core"]["value"] > 0
    assert out["one_core"]["sample"].startswith(f"{w.n_req // 2} of {w.n_req} requests")
