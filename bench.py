#!/usr/bin/env python3
"""Throughput of the fused quantized gated delta-rule decode step on one MI355X.

Workload: the STEPQuant pages' serving point -- 70 concurrent requests x 2304
recurrent heads ("K1 論文詳解" 背景; "线性注意力状态量化难题" 时间维度), d_k = d_v
= 128, per-head 4/6/8-bit codes averaging 6 bits plus 32 FP16 pivot heads
(1.39 %), bf16 q/k/v, synthetic seeded inputs.  One step = one call of
sq_decode_step over the whole batch (one kernel launch): every tile is read,
updated, read out, requantized and written back in place.

Prints ONE JSON line: heads*tokens/s, ms per step, algorithmic HBM GB/s, the
roofline of the step kernel, and the CPU oracle timed on a bounded sample of
the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized state-update heads·tokens/s + achieved HBM GB/s (70 req × 2304 heads)"
HBM_PEAK_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "quantized_recurrent_state_gated_amd", "csrc", "sq_kernels.hip")


def traffic_file(workload: str) -> str:
    """Counter-measured HBM bytes of the step launches of one workload."""
    return os.path.join(ROOT, "profiles", f"traffic_step128_{workload}.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_bytes_per_step(w, bits) -> int:
    """State read + write of every tile, plus per head-token q, k, v (bf16),
    alpha, beta (fp32) and o (fp32)."""
    from quantized_recurrent_state_gated_amd.inputs import field_width

    d2 = w.dk * w.dv
    state = sum(2 * d2 * field_width(b) // 8 for b in bits) * w.n_req
    io = w.n_req * w.n_heads * (2 * (2 * w.dk + w.dv) + 8 + 4 * w.dv)
    return state + io


# rocprofv3 kernel names of the two timed step instances (bf16 q/k/v; launches
# of 16,384 tiles or more, two tiles per workgroup)
STEP_KERNEL = "k_step128x2<unsigned short, true, false, 5>"
KDA_KERNEL = "k_step128x2<unsigned short, true, true, 5>"


def step_kernel(n_tiles: int, kda: bool = False) -> str:
    """The d = 128 step instance a launch of n_tiles 4/6/8/16-bit tiles takes
    (bf16 q/k/v): two tiles per workgroup from 16,384 tiles, four waves per
    tile from 1,024, else two."""
    g = "true" if kda else "false"
    if n_tiles >= 16384:
        return f"k_step128x2<unsigned short, true, {g}, 5>"
    if n_tiles >= 1024:
        return f"k_step128<unsigned short, true, {g}, 256, 8>"
    return f"k_step128<unsigned short, true, {g}, 128, 5>"


def traffic_from_profile(sha: str, workload: str, which: str = "step"):
    """HBM bytes per launch measured by rocprofv3 counters for this exact kernel
    source and workload, scaled by the copy-kernel calibration; None if absent
    or stale."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != sha or t.get("workload") != workload or which not in t:
        return None
    return t[which].get("hbm_bytes_per_launch")


COPY_BYTES = 1 << 30  # the calibration copy of --copy-calibration

# gfx950 L2-to-memory request counters, by request size (rocprofv3 -L):
# reads of 32, 64 and 128 bytes, all reads; writes of 64 bytes, all writes
# (a write is 32 or 64 bytes); TCC_BUBBLE counts 128-byte reads as well.
READ_COUNTERS = ("TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B", "TCC_EA0_RDREQ_128B", "TCC_EA0_RDREQ")
WRITE_COUNTERS = ("TCC_EA0_WRREQ_64B", "TCC_EA0_WRREQ", "TCC_BUBBLE")
PMC_KERNELS = {"step": STEP_KERNEL, "channel_gate_step": KDA_KERNEL,
               "copy": "copyBuffer"}  # the runtime's blit kernel of the 1 GiB copy


def _pmc_dispatches(path, counters):
    """{kernel key: [{counter: value} per dispatch, in dispatch order]} from a
    rocprofv3 --pmc csv; dispatches missing a counter are dropped."""
    import csv
    by = {k: {} for k in PMC_KERNELS}
    for r in csv.DictReader(open(path)):
        c = r["Counter_Name"]
        if c not in counters:
            continue
        for key, name in PMC_KERNELS.items():
            if name in r["Kernel_Name"]:
                by[key].setdefault(int(r["Dispatch_Id"]), {})[c] = float(r["Counter_Value"])
    return {k: [d[i] for i in sorted(d) if len(d[i]) == len(counters)] for k, d in by.items() if d}


def pmc_summary(read_csv: str, write_csv: str, workload: str) -> int:
    """HBM bytes per launch from gfx950's per-request-size counters: reads =
    32 n32 + 64 n64 + 128 n128, writes = 64 n64 + 32 (n - n64), per dispatch;
    the median over the step's dispatches.  No scale factor: the 1 GiB
    calibration copy (the largest blit dispatch) is reported beside as a check."""
    import statistics
    rd = _pmc_dispatches(read_csv, READ_COUNTERS)
    wr = _pmc_dispatches(write_csv, WRITE_COUNTERS)

    def rbytes(d):
        return 32 * d[READ_COUNTERS[0]] + 64 * d[READ_COUNTERS[1]] + 128 * d[READ_COUNTERS[2]]

    def wbytes(d):
        return 64 * d[WRITE_COUNTERS[0]] + 32 * (d[WRITE_COUNTERS[1]] - d[WRITE_COUNTERS[0]])

    def one(key):
        r, w = rd[key], wr[key]
        if key == "copy":
            r, w = [max(r, key=rbytes)], [max(w, key=wbytes)]
        read = statistics.median(rbytes(d) for d in r)
        write = statistics.median(wbytes(d) for d in w)
        return {"kernel": PMC_KERNELS[key], "fetch_bytes_per_launch": read,
                "write_bytes_per_launch": write, "hbm_bytes_per_launch": read + write,
                "dispatches": [len(r), len(w)],
                "raw_median": {c: statistics.median(d[c] for d in r) for c in READ_COUNTERS} |
                              {c: statistics.median(d[c] for d in w) for c in WRITE_COUNTERS},
                # every dispatch: the sized read counts add up to all reads, and
                # every write is a 64-byte one or the rest (32-byte)
                "reads_by_size_sum_to_all": all(
                    d[READ_COUNTERS[0]] + d[READ_COUNTERS[1]] + d[READ_COUNTERS[2]] ==
                    d[READ_COUNTERS[3]] for d in r),
                "tcc_bubble_reads": statistics.median(d[WRITE_COUNTERS[2]] for d in w)}

    wl = "" if workload == "serving" else f" --workload {workload}"
    cmd = ("python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-fp32-baseline "
           f"--no-copy-ceiling --copy-calibration{wl}")
    out = {"kernel_source_sha": kernel_source_sha(), "workload": workload,
           "method": "per-request-size L2-to-memory counters, bytes per dispatch, no scale factor",
           "commands": [f"rocprofv3 --pmc {' '.join(READ_COUNTERS)} --output-format csv "
                        f"-d <dir> -o <name> -- {cmd}",
                        f"rocprofv3 --pmc {' '.join(WRITE_COUNTERS)} --output-format csv "
                        f"-d <dir> -o <name> -- {cmd}"]}
    for key in ("step", "channel_gate_step", "copy"):
        if key in rd and key in wr:
            out[key] = one(key)
    if "copy" in out:
        out["copy"]["expected_bytes_each_way"] = COPY_BYTES
    path = traffic_file(workload)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


CLOCK_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU",
                  "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES")
N_XCDS, N_SES, N_SIMDS = 8, 32, 256 * 4


def clock_summary(csv_path: str, kernel: str = STEP_KERNEL) -> int:
    """Per dispatch of `kernel` in a rocprofv3 --pmc run of CLOCK_COUNTERS:
    duration; counted clock rates (GRBM_GUI_ACTIVE is summed over the 8 XCDs,
    SQ_CYCLES over the 32 shader engines); VALU wave-instructions issued; and
    those per SIMD per 4 counted cycles (a wave64 VALU instruction occupies a
    16-lane SIMD for 4 cycles)."""
    import csv
    by = {}
    for r in csv.DictReader(open(csv_path)):
        if kernel not in r["Kernel_Name"] or r["Counter_Name"] not in CLOCK_COUNTERS:
            continue
        d = by.setdefault(int(r["Dispatch_Id"]),
                          {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    print("| launch | µs | GRBM_GUI_ACTIVE per XCD per µs | SQ_CYCLES per SE per µs | "
          "VALU wave-instructions | VALU per SIMD per 4 counted cycles |")
    print("|---|---|---|---|---|---|")
    for i, (_, d) in enumerate(sorted(by.items())):
        us = d["ns"] / 1e3
        cyc = d["SQ_CYCLES"] / N_SES
        share = d["SQ_INSTS_VALU"] * 4 / (N_SIMDS * cyc) if cyc else float("nan")
        print(f"| {i + 1} | {us:.1f} | {d['GRBM_GUI_ACTIVE'] / N_XCDS / us:.0f} | {cyc / us:.0f} | "
              f"{d['SQ_INSTS_VALU']:.4g} | {share:.2f} |")
    return 0


def trace_summary(stats_csv: str) -> int:
    import csv
    for r in csv.DictReader(open(stats_csv)):
        if "k_step128" in r["Name"] and "_f32" not in r["Name"]:
            print(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                  f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {r['Percentage']} |")
    return 0


def unquantized_baseline(sq, I, w, dev, stream, ins, quant_ms, fmt=32, steps=16, warmup=10):
    """The same step with every head holding an unquantized state: FP32 (the
    'FP32 state' baseline of the pages' efficiency comparison) or bfloat16
    (fmt = 144), timed on the same inputs; context for the quantized step, not
    part of the metric."""
    import numpy as np
    import torch

    bits = np.full(w.n_heads, fmt, np.uint8)
    nbytes = sq.sq_pool_bytes(w.n_req, w.n_heads, w.dk, w.dv, bits)
    ones_r = torch.ones(w.n_heads, w.dk, device=dev)
    ones_c = torch.ones(w.n_heads, w.dv, device=dev)
    state = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    pool = sq.sq_pool_alloc(w.n_req, w.n_heads, w.dk, w.dv, bits, ones_r, ones_c, state)
    slots = torch.arange(w.n_req, dtype=torch.int32, device=dev)
    for p in range(w.n_req):
        sq.sq_pool_store(pool, slots[p:p + 1], I.initial_state(w, p, dev))
    o = torch.empty(w.n_req, w.n_heads, w.dv, device=dev)

    def step(t):
        x = ins[t % len(ins)]
        sq.sq_decode_step(pool, slots, x.q, x.k, x.v, x.alpha, x.beta, o, stream)

    for t in range(warmup):
        step(t)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for t in range(steps):
        step(warmup + t)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    byts = algorithmic_bytes_per_step(w, bits)
    del pool, state
    torch.cuda.empty_cache()
    out = {"ms_per_step": ms, "hbm_gbps": byts / (ms / 1e3) / 1e9, "pool_bytes": nbytes,
           "speedup_of_quantized_step": ms / quant_ms}
    if fmt == 32:
        out["pages_context"] = "2.91x state-update speedup at 6 bits on NVIDIA A800"
    return out


def channel_gate_step(sq, I, w, bits, pool, slots, dev, stream, n_in, quant_ms, steps=32,
                      warmup=40):
    """The per-key-channel-gate (KDA) step, sq_decode_step_kda, on the same pool
    and inputs with alpha [n_req][H][d_k] resident in HBM: the second model
    family's step at the same shape.  Reported beside the metric, not in it."""
    import torch

    ins = []
    for t in range(n_in):
        si = I.step_inputs(w, t, dev)
        si.alpha = I.channel_gates(w, t, dev)
        ins.append(si)
    o = torch.empty(w.n_req, w.n_heads, w.dv, device=dev)

    def step(t):
        x = ins[t % n_in]
        sq.sq_decode_step_kda(pool, slots, x.q, x.k, x.v, x.alpha, x.beta, o, stream)

    # the timed launches follow the warm-up in stream order with no host
    # synchronization between them, so the GPU never idles in between
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for t in range(warmup):
        step(t)
    evs[0].record(stream)
    for t in range(steps):
        step(warmup + t)
        evs[t + 1].record(stream)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    # the scalar gate's 4 bytes per head-token become 4 d_k bytes
    byts = algorithmic_bytes_per_step(w, bits) + w.n_req * w.n_heads * 4 * (w.dk - 1)
    gbps = byts / (ms / 1e3) / 1e9
    return {"value": w.n_req * w.n_heads / (ms / 1e3), "unit": "heads*tokens/s",
            "traffic": traffic_from_profile(kernel_source_sha(), w.name, "channel_gate_step"),
            "ms_per_step": ms, "hbm_gbps": gbps, "frac": gbps / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": byts, "time_vs_scalar_gate_step": ms / quant_ms,
            "kernel": step_kernel(w.n_req * w.n_heads, kda=True)}


def saturation(sq, w, bits, pool, state):
    """Fraction of stored codes at the ends of the symmetric range (+-Q) per
    width, read from the pool bytes after the timed steps: a proxy for the
    requantizer's clamp rate (a code at +-Q was clamped or rounded onto the
    bound).  torch integer ops on the bytes; diagnostic only."""
    import numpy as np
    import torch

    slab = state.numel() // w.n_req
    rows = state[: w.n_req * slab].view(w.n_req, slab)
    out = {}
    for b in (4, 6, 8):
        hs = np.nonzero(bits == b)[0]
        if hs.size == 0:
            continue
        offs = [sq.sq_pool_tile_offset(pool, 0, int(h)) for h in hs]
        nb = offs[0][1]
        idx = torch.tensor([o for o, _ in offs], device=state.device)[:, None] + \
            torch.arange(nb, device=state.device)[None, :]
        t = rows[:, idx].to(torch.int32)  # [n_req][heads of width b][tile bytes]
        if b == 8:
            f = t
        elif b == 4:
            f = torch.stack([t & 15, t >> 4], -1)
        else:
            g = t.view(w.n_req, hs.size, -1, 3)
            word = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
            f = torch.stack([(word >> sh) & 63 for sh in (0, 6, 12, 18)], -1)
        out[str(b)] = float(((f == 1) | (f == (1 << b) - 1)).double().mean())
        del t, f
    return out


def small_batch_graph(sq, I, dev, steps=16, reps=20):
    """The layer workload (8 requests x 48 heads, 384 tiles: cache-resident and
    launch-bound) stepped eagerly and as a HIP graph of `steps` captured
    steps; per-step times of both.  Context for the small-batch regime."""
    import torch

    w = I.WORKLOADS["layer"]
    bits = I.head_bits(w)
    r, c = I.scales(w, device=dev)
    nbytes = sq.sq_pool_bytes(w.n_req, w.n_heads, w.dk, w.dv, bits)
    state = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    pool = sq.sq_pool_alloc(w.n_req, w.n_heads, w.dk, w.dv, bits, r, c, state)
    slots = torch.arange(w.n_req, dtype=torch.int32, device=dev)
    for p in range(w.n_req):
        sq.sq_pool_store(pool, slots[p:p + 1], I.initial_state(w, p, dev))
    ins = [I.step_inputs(w, t, dev) for t in range(steps)]
    o = torch.empty(w.n_req, w.n_heads, w.dv, device=dev)

    def run():
        for x in ins:
            sq.sq_decode_step(pool, slots, x.q, x.k, x.v, x.alpha, x.beta, o)

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * steps)

    eager = timed(run)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    graph = timed(g.replay)
    del g, pool, state
    torch.cuda.empty_cache()
    return {"workload": f"layer: {w.n_req} requests x {w.n_heads} heads ({w.tiles} tiles)",
            "eager_ms_per_step": eager, "graph_ms_per_step": graph,
            "steps_per_graph": steps, "speedup": eager / graph}


def copy_ceiling(dev, stream, nbytes=2 << 30, reps=10):
    """Device-to-device copy rate measured in the same process (torch copy_,
    i.e. the runtime's blit kernel): bytes read + written per second.  A
    practical bandwidth ceiling for a read-and-write stream, next to the
    nominal peak."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"gbps": 2 * nbytes / (ms / 1e3) / 1e9, "bytes_per_copy": nbytes, "ms_per_copy": ms,
            "what": "device-to-device copy (torch copy_), read + write bytes per second"}


def cpu_model() -> str:
    """The host CPU's model name as lscpu reports it (else /proc/cpuinfo)."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=30).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads(requested=None):
    """(threads, reason): the requested count; else the job's CPU share as the
    environment states it (OMP_NUM_THREADS); else every core in the affinity mask."""
    aff = len(os.sched_getaffinity(0))
    if requested:
        return int(requested), f"--cpu-threads {requested} ({aff} cores in the affinity mask)"
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env), (f"OMP_NUM_THREADS={env}: the job's CPU share ({aff} cores in the "
                          f"affinity mask, shared with other jobs)")
    return aff, f"every core in the affinity mask ({aff})"


def oracle_steps(w, bits, pool, r, c, inputs, n_req, threads):
    """Wall time of the oracle stepping requests 0..n_req-1 of a host pool once
    per input in `inputs` (in place)."""
    import numpy as np
    import oracle

    slots = np.arange(n_req, dtype=np.int32)
    total = 0.0
    for si in inputs:
        q, k, v = (x[:n_req].float().cpu().numpy() for x in (si.q, si.k, si.v))
        al, be = si.alpha[:n_req].cpu().numpy(), si.beta[:n_req].cpu().numpy()
        t0 = time.perf_counter()
        oracle.step_pool(pool, bits, w.dk, w.dv, r, c, slots, q, k, v, al, be, n_threads=threads,
                         want_o=True)
        total += time.perf_counter() - t0
    return total


def cpu_baseline(w, bits, host_pool, r, c, inputs, n_threads, why, other=None):
    """The oracle, as it stands: len(inputs) full decode steps of workload w on
    n_threads threads (every tile of every request), then one thread on
    1/n_threads of the requests for one step.  other = (workload, bits, host
    pool, r, c, inputs): one full step of a second workload on n_threads."""
    pool = host_pool.copy()
    t = oracle_steps(w, bits, pool, r, c, inputs, w.n_req, n_threads)
    n_steps = len(inputs)
    out = {"value": n_steps * w.n_req * w.n_heads / t, "unit": "heads*tokens/s",
           "cores": n_threads, "cores_why": why, "kind": "oracle", "cpu": cpu_model(),
           "sample": f"{n_steps} full decode steps of {w.name} ({w.n_req} requests x {w.n_heads} "
                     f"heads = {w.n_req * w.n_heads} tiles per step), {t:.1f} s wall on "
                     f"{n_threads} threads",
           "s_per_step": t / n_steps}
    if n_threads > 1:
        n1 = max(1, w.n_req // n_threads)
        pool = host_pool.copy()
        t1 = oracle_steps(w, bits, pool, r, c, inputs[:1], n1, 1)
        out["one_core"] = {"value": n1 * w.n_heads / t1, "unit": "heads*tokens/s",
                           "sample": f"{n1} of {w.n_req} requests x all {w.n_heads} heads, one "
                                     f"step ({n1 * w.n_heads} tiles, {t1:.1f} s on 1 thread)"}
    if other is not None:
        w2, bits2, pool2, r2, c2, in2 = other
        t2 = oracle_steps(w2, bits2, pool2, r2, c2, in2, w2.n_req, n_threads)
        out[w2.name] = {"value": len(in2) * w2.n_req * w2.n_heads / t2, "unit": "heads*tokens/s",
                        "s_per_step": t2 / len(in2),
                        "sample": f"{len(in2)} full decode step(s) of {w2.name} ({w2.n_req} x "
                                  f"{w2.n_heads} = {w2.n_req * w2.n_heads} tiles), {t2:.1f} s "
                                  f"wall on {n_threads} threads"}
    return out


def host_pool_of(sq, I, name, dev):
    """A workload's pool, initialised on the GPU from its seeded initial
    states, copied to host memory; returns (workload, bits, pool, r, c)."""
    import torch

    w = I.WORKLOADS[name]
    bits = I.head_bits(w)
    r, c = I.scales(w, device=dev)
    nbytes = sq.sq_pool_bytes(w.n_req, w.n_heads, w.dk, w.dv, bits)
    state = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    pool = sq.sq_pool_alloc(w.n_req, w.n_heads, w.dk, w.dv, bits, r, c, state)
    slots = torch.arange(w.n_req, dtype=torch.int32, device=dev)
    for p in range(w.n_req):
        sq.sq_pool_store(pool, slots[p:p + 1], I.initial_state(w, p, dev))
    host = state.cpu().numpy()
    sq.sq_pool_free(pool)
    return w, bits, host, r.cpu().numpy(), c.cpu().numpy()


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256,
                    help="timed steps (enough that the warm-up launches are a small part of a kernel trace)")
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed steps first: after an idle spell launch times jump and take "
                         "~25-30 launches to settle")
    ap.add_argument("--workload", default="serving", choices=["serving", "highconc", "layer", "drift"])
    ap.add_argument("--distinct-inputs", type=int, default=16,
                    help="distinct pre-generated step inputs, cycled over the timed steps")
    ap.add_argument("--cpu-threads", type=int, default=None,
                    help="oracle threads (default: OMP_NUM_THREADS, else every core in the affinity mask)")
    ap.add_argument("--cpu-steps", type=int, default=2,
                    help="full decode steps of the workload the CPU oracle times")
    ap.add_argument("--cpu-other", default="highconc",
                    help="a second workload the CPU oracle times one full step of ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp32-baseline", action="store_true",
                    help="skip timing the unquantized FP32- and BF16-state steps at the same shape")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip timing a device-to-device copy as a practical bandwidth ceiling")
    ap.add_argument("--small-batch", action="store_true",
                    help="also time the small layer workload eagerly and as a HIP graph (it runs "
                         "the same kernel, so it is off by default to keep kernel traces clean)")
    ap.add_argument("--no-kda", action="store_true",
                    help="skip timing the per-key-channel-gate step at the same shape")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("READ_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs of `bench.py --copy-calibration` "
                         "(the read-request and the write-request counters, by size) into "
                         "profiles/ and exit")
    ap.add_argument("--clock-summary", metavar="PMC_CSV",
                    help="per-launch clock and VALU table from a rocprofv3 --pmc run of "
                         "GRBM_GUI_ACTIVE SQ_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU "
                         "SQ_WAVE_CYCLES, and exit")
    ap.add_argument("--trace-summary", metavar="KERNEL_STATS_CSV",
                    help="print the step kernel's row of a rocprofv3 --stats csv and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary, args.workload)
    if args.trace_summary:
        return trace_summary(args.trace_summary)
    if args.clock_summary:
        return clock_summary(args.clock_summary)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the step is measured on one GPU only (--gpus 1); it would shard by request "
              "slot or by head with no exchange, and multi-GPU runs are not implemented",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from quantized_recurrent_state_gated_amd import inputs as I
    from quantized_recurrent_state_gated_amd import sq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = I.WORKLOADS[args.workload]
    bits = I.head_bits(w)
    log(f"[bench] workload {w.name}: {w.n_req} req x {w.n_heads} heads, d={w.dk}, "
        f"bits { {int(b): int((bits == b).sum()) for b in sorted(set(bits))} }")

    t0 = time.time()
    r, c = I.scales(w, device=dev)
    nbytes = sq.sq_pool_bytes(w.n_req, w.n_heads, w.dk, w.dv, bits)
    state = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    pool = sq.sq_pool_alloc(w.n_req, w.n_heads, w.dk, w.dv, bits, r, c, state)
    slots = torch.arange(w.n_req, dtype=torch.int32, device=dev)
    for p in range(w.n_req):
        sq.sq_pool_store(pool, slots[p:p + 1], I.initial_state(w, p, dev))
    torch.cuda.synchronize()
    log(f"[bench] pool {nbytes / 1e9:.3f} GB initialised in {time.time() - t0:.1f} s")

    n_in = max(1, min(args.distinct_inputs, args.steps))
    ins = [I.step_inputs(w, t, dev) for t in range(n_in)]
    o = torch.empty(w.n_req, w.n_heads, w.dv, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {n_in} distinct step inputs resident in HBM")

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 x 1 GiB device copies done")

    stream = torch.cuda.current_stream()

    def step(t):
        x = ins[t % n_in]
        sq.sq_decode_step(pool, slots, x.q, x.k, x.v, x.alpha, x.beta, o, stream)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")

    # events around every launch, on the stream the kernel runs on
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for t in range(args.steps):
        step(args.warmup + t)
        evs[t + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = sorted(evs[t].elapsed_time(evs[t + 1]) for t in range(args.steps))
    gpu_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = gpu_ms / args.steps
    log(f"[bench] {args.steps} timed steps: {gpu_ms:.3f} ms events, {wall * 1e3:.3f} ms wall")

    head_tokens = w.n_req * w.n_heads
    value = head_tokens * args.steps / (gpu_ms / 1e3)
    bpstep = algorithmic_bytes_per_step(w, bits)
    gbps = bpstep / (ms_per_step / 1e3) / 1e9
    sha = kernel_source_sha()
    traffic = traffic_from_profile(sha, w.name)
    stats = I.pool_stats(w)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "heads*tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.n_req} requests x {w.n_heads} heads, d_k=d_v={w.dk}, "
                        f"4/6/8-bit codes (mean {stats['mean_bits_nonpivot']:.3f}) + FP16 pivots, "
                        f"{w.qkv_dtype} q/k/v, one fused decode step per launch",
            "n_req": w.n_req, "n_heads": w.n_heads, "d_k": w.dk, "d_v": w.dv,
            "head_bits": {str(int(b)): int((bits == b).sum()) for b in sorted(set(bits))},
            "pool_bytes": stats["pool_bytes"],
            "state_compression_vs_fp32": stats["fp32_pool_bytes"] / stats["pool_bytes"],
        },
        "hbm_gbps": gbps,
        "roofline": {
            "bound": "hbm",
            "achieved": gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "traffic": traffic,
            "kernel": step_kernel(w.n_req * w.n_heads) + " (one launch = one decode step over all tiles)",
            "algorithmic_bytes_per_launch": bpstep,
            "avg_launch_ms": ms_per_step,
            "launch_ms_min_median_max": [per[0], per[len(per) // 2], per[-1]],
            "kernel_source_sha": sha,
        },
        "cpu_baseline": None,
    }

    result["saturated_code_fraction"] = saturation(sq, w, bits, pool, state)
    log(f"[bench] codes at +-Q after the timed steps: {result['saturated_code_fraction']}")

    if not args.no_copy_ceiling:
        cc = copy_ceiling(dev, stream)
        result["roofline"]["copy_ceiling_gbps"] = cc["gbps"]
        result["roofline"]["frac_of_copy_ceiling"] = gbps / cc["gbps"]
        result["copy_ceiling"] = cc
        log(f"[bench] D2D copy ceiling: {cc['gbps']:.0f} GB/s; step at {gbps / cc['gbps']:.3f} of it")

    if args.small_batch:
        result["small_batch_graph"] = small_batch_graph(sq, I, dev)
        log(f"[bench] layer workload: {result['small_batch_graph']['eager_ms_per_step'] * 1e3:.1f} us "
            f"eager, {result['small_batch_graph']['graph_ms_per_step'] * 1e3:.1f} us in a graph")

    if not args.no_kda:
        result["channel_gate_step"] = channel_gate_step(sq, I, w, bits, pool, slots, dev, stream,
                                                        n_in, ms_per_step)
        log(f"[bench] per-channel-gate step: {result['channel_gate_step']['ms_per_step']:.3f} ms "
            f"({result['channel_gate_step']['frac']:.3f} of HBM peak)")

    if not args.no_fp32_baseline:
        for key, fmt in (("fp32_state_baseline", 32), ("bf16_state_baseline", I.BITS_BF16)):
            result[key] = unquantized_baseline(sq, I, w, dev, stream, ins, ms_per_step, fmt)
            log(f"[bench] {key}: {result[key]['ms_per_step']:.3f} ms "
                f"({result[key]['speedup_of_quantized_step']:.2f}x)")

    if not args.no_cpu_baseline:
        del ins
        torch.cuda.synchronize()
        log("[bench] CPU oracle baseline ...")
        n_cpu, why = cpu_threads(args.cpu_threads)
        host = state.cpu().numpy()
        other = None
        if args.cpu_other and args.cpu_other != w.name:
            w2, bits2, pool2, r2, c2 = host_pool_of(sq, I, args.cpu_other, dev)
            other = (w2, bits2, pool2, r2, c2, [I.step_inputs(w2, 0)])
            torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(
            w, bits, host, r.cpu().numpy(), c.cpu().numpy(),
            [I.step_inputs(w, t) for t in range(args.cpu_steps)], n_cpu, why, other)
        log(f"[bench] CPU oracle: {result['cpu_baseline']['value']:.3e} heads*tokens/s "
            f"on {n_cpu} threads")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
