#!/usr/bin/env python3
"""Throughput of the FlashAttention-2 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ref] [--pass fwd|bwd]
                    [--impl fa2|fa1] [--batch-sweep]

Without --warmup / --steps, W fills about 0.4 s and K about 0.25 s of
launches; the JSON line reports the W and K actually run.  The GPU's clock
dips after load begins: at [4,32,2048,64] the first ~6 launches (1.2 ms)
run at ~175 us, launches from ~1.2 ms to ~8 ms at 200-225 us, and the clock
settles after ~25 ms of load at ~163 us per launch.  A short run such as
--warmup 5 --steps 20 (~5 ms of load) times exactly that dip and reads
25-30 % below the settled rate; nothing here shortens or skips it.

A step is one fa2_fwd call: the whole hot path (load Q, stream K/V tiles,
two MFMA contractions, online softmax, normalised O and LSE) over one batch
of seeded synthetic fp16 inputs already resident in HBM.  Prints ONE JSON
line on stdout; progress goes to stderr.

value      TFLOP/s with FLOPs = 4*B*H*N^2*d (halved when causal), wall clock
           over K steps between two device synchronisations;
roofline   the kernel's average launch time from HIP events on the stream it
           is launched on, against MI355X's dense fp16 MFMA peak;
           ``traffic`` is the HBM bytes per launch measured by rocprofv3
           counters for this exact kernel source (null if the source changed
           since they were taken);
cpu_baseline  the float64 CPU oracle timed on the host cores on a bounded
           sample of the same workload (a reported baseline, not a target).

--pass bwd times the backward pass instead: a step is one fa2_bwd call (the
dQ kernel, then the dK/dV kernel) on the forward's O and LSE and a seeded
upstream gradient; FLOPs = 10*B*H*N^2*d (five products of 2*N^2*d: S, dP,
dV, dK, dQ; halved when causal), the roofline unit is the whole call, and
the CPU baseline is the float64 gradient oracle.

A decoding workload (Nq query rows against N keys, e.g. decode_64k) is
timed through fa2_fwd_splitkv with the library's split count: value and
roofline are HBM GB/s of algorithmic bytes (Q, K, V read once, O and LSE
written once) against 8 TB/s, parity is every row against the oracle.

--impl fa1 times the FlashAttention-1-order comparator (fa1_fwd, d = 64)
on the workload instead of fa2_fwd.  --batch-sweep times both, causal and
not, at [B, 32, 2048, 64] for B = 1, 2, 4, 8, 16 (the batch experiment of
"Implementing FlashAttention 1 and 2 forward in Triton") and prints one JSON
line with every point and the FA2 / FA1 speed ratios.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FA2 fwd TFLOP/s and % of MI355X fp16 MFMA peak, [4,32,2048,64]"
METRIC_BWD = "FA2 bwd TFLOP/s and % of MI355X fp16 MFMA peak"
METRIC_DECODE = "FA2 split-KV decode HBM GB/s (Q, K, V read, O, LSE written) and % of MI355X HBM peak"
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP16_TFLOPS = 2516.6   # MI355X dense fp16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
_CSRC = os.path.join(ROOT, "exact_attention_fwd_amd", "csrc")
# The device sources of each measured path: its HBM counters stay valid while
# these are unchanged.
KERNEL_SOURCES = {
    "fwd": [os.path.join(_CSRC, f) for f in ("fa2_fwd_gfx950.hip", "fa2_device.h")],
    "bwd": [os.path.join(_CSRC, f) for f in ("fa2_bwd_gfx950.hip", "fa2_device.h")],
    "fa1": [os.path.join(_CSRC, f) for f in ("fa1_fwd_gfx950.hip", "fa2_device.h")],
    "decode": [os.path.join(_CSRC, f) for f in ("fa2_splitkv_gfx950.hip", "fa2_device.h")],
}
# rocprofv3 kernel-name fragments of each path (a call may launch several).
KERNEL_NAMES = {"fwd": ("fa2_fwd_kernel",), "bwd": ("fa2_bwd_dq_kernel", "fa2_bwd_dkdv"),
                "fa1": ("fa1_fwd_kernel",), "decode": ("splitkv_partial_kernel", "lse_merge_kernel")}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha(path: str = "fwd") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[path]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_key(path: str, workload: str) -> str:
    return workload if path == "fwd" else f"{path}:{workload}"


def measured_traffic(path: str, workload: str):
    """HBM bytes per call from the committed counter summary, if they were
    taken on the current source of that path's kernels."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    w = t.get("workloads", {}).get(traffic_key(path, workload))
    if w is None or w.get("kernel_sha256") != kernel_sha(path):
        return None
    return w.get("hbm_bytes_per_launch")


def algorithmic_bytes(path: str, w) -> float:
    """HBM bytes a call must move at least: inputs read once, outputs written
    once (workspaces excluded)."""
    if path == "bwd":   # q, k, v, o, dO, LSE in; dQ, dK, dV out
        return w.B * w.H * w.N * (16.0 * w.d + 4)
    return w.hbm_bytes()


def summarize_counters(directory: str) -> dict:
    """profiles/traffic.json from rocprofv3 --pmc runs laid out as
    <dir>/copy_<C>/ (bench.py --copy-calibration 512) and
    <dir>/pmc_<path>_<workload>_<C>/ (bench.py --pass/--impl/--workload),
    C in FETCH_SIZE, WRITE_SIZE.  Each counter is scaled by the factor that
    makes it read the true bytes of the plain copy; a call's bytes are the
    sums over its kernels of the median per-dispatch values."""
    import csv
    import glob
    import statistics

    from exact_attention_fwd_amd.workloads import WORKLOADS

    def values(sub, names):
        out = {}
        for f in glob.glob(os.path.join(directory, sub, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    for n in names:
                        if n in r["Kernel_Name"]:
                            out.setdefault(n, []).append(float(r["Counter_Value"]))
        return out

    copy_kib = 512 * 1024
    cf = statistics.median(values("copy_FETCH_SIZE", ("copyBuffer",))["copyBuffer"])
    cw = statistics.median(values("copy_WRITE_SIZE", ("copyBuffer",))["copyBuffer"])
    ff, wf = copy_kib / cf, copy_kib / cw
    res = {"note": "HBM bytes per call from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, "
                   "median over dispatches, summed over the kernels of one call), each scaled by the "
                   "factor that makes the same counter read the true bytes of a plain 512 MiB device "
                   "copy (bench.py --copy-calibration 512).  An entry is valid only while the sha256 "
                   "of its path's kernel sources matches.",
           "calibration": {"copy_bytes": copy_kib * 1024, "fetch_size_kib": cf, "write_size_kib": cw,
                           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "workloads": {}}
    for d in sorted(glob.glob(os.path.join(directory, "pmc_*_FETCH_SIZE"))):
        stem = os.path.basename(d)[len("pmc_"):-len("_FETCH_SIZE")]
        path, wname = stem.split("_", 1)
        names = KERNEL_NAMES[path]
        fv = values(f"pmc_{stem}_FETCH_SIZE", names)
        wv = values(f"pmc_{stem}_WRITE_SIZE", names)
        fk = sum(statistics.median(v) for v in fv.values())
        wk = sum(statistics.median(v) for v in wv.values())
        rd, wr = fk * 1024 * ff, wk * 1024 * wf
        alg = algorithmic_bytes(path, WORKLOADS[wname])
        res["workloads"][traffic_key(path, wname)] = {
            "kernel_sha256": kernel_sha(path), "kernels": sorted(fv),
            "fetch_factor": round(ff, 4), "write_factor": round(wf, 4), "fetch_size_kib": fk,
            "write_size_kib": wk, "hbm_read_bytes": int(rd), "hbm_write_bytes": int(wr),
            "hbm_bytes_per_launch": int(rd + wr), "algorithmic_bytes": int(alg),
            "ratio_to_algorithmic": round((rd + wr) / alg, 4)}
    return res


def cpu_baseline(w, q, k, v, budget_s: float):
    """Time the oracle on whole (b, h) heads, as many as fit ~budget_s (the
    median of three runs), or on the sampled rows of a long workload (one
    run)."""
    import numpy as np

    from exact_attention_fwd_amd.workloads import sample_rows
    from oracle import attention_fp64
    from oracle.attention import oracle_threads

    threads = oracle_threads()
    per_row_flops = 4.0 * w.N * w.d / (2 if w.causal else 1)
    if w.sampled_rows:
        rows = np.stack([np.stack([sample_rows(w.N, b, h, w.sampled_rows) for h in range(w.H)])
                         for b in range(w.B)])
        t0 = time.perf_counter()
        attention_fp64(q, k, v, w.scale, causal=w.causal, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
        flops = rows.size * per_row_flops
        sample = f"{w.sampled_rows} seeded query rows per (b,h) of {w.name}, all {w.B * w.H} heads"
    else:
        # whole heads, the first n of them; n sized from a one-head probe
        t0 = time.perf_counter()
        attention_fp64(q[:1, :1], k[:1, :1], v[:1, :1], w.scale, causal=w.causal, threads=1)
        one = max(time.perf_counter() - t0, 1e-4)
        n_heads = int(min(w.B * w.H, max(threads, budget_s * threads / one)))
        n_heads = max(1, n_heads)
        qf, kf, vf = (x.reshape(1, w.B * w.H, w.N, w.d)[:, :n_heads] for x in (q, k, v))
        runs = []
        for _ in range(3):   # whole-head workloads: the median of three runs
            t0 = time.perf_counter()
            attention_fp64(qf, kf, vf, w.scale, causal=w.causal, threads=threads)
            runs.append(time.perf_counter() - t0)
        dt = sorted(runs)[1]
        flops = n_heads * w.N * per_row_flops
        sample = (f"{n_heads} of {w.B * w.H} heads of {w.name}, every query row; median of 3 runs "
                  f"({', '.join(f'{r:.3f}' for r in runs)} s)")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3)}


def measured_ceilings(torch, dev, seconds: float = 0.25) -> dict:
    """The box's practical ceilings, measured with library kernels (run after
    the timed region, so they cannot warm the GPU for it):
    dense fp16 matmul TFLOP/s (torch.matmul, hipBLASLt, 8192^3, fp32
    accumulation), device-to-device copy GB/s (bytes read + written) and a
    read-only stream GB/s (torch.sum over 1 GiB of fp16)."""
    stream = torch.cuda.current_stream(dev)

    def timed(fn, warm=3):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize(dev)
        n = max(5, int(seconds / max(time.perf_counter() - t0, 1e-6)))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) * 1e-3 / n

    g = torch.Generator(device=dev).manual_seed(0)
    n = 8192
    a = torch.randn((n, n), device=dev, dtype=torch.float16, generator=g)
    b = torch.randn((n, n), device=dev, dtype=torch.float16, generator=g)
    c = torch.empty((n, n), device=dev, dtype=torch.float16)
    t_mm = timed(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    nbytes = 1 << 30
    src = torch.ones(nbytes // 2, device=dev, dtype=torch.float16)
    dst = torch.empty_like(src)
    t_cp = timed(lambda: dst.copy_(src))
    t_sum = timed(lambda: torch.sum(src, dtype=torch.float32))
    # a memory-bound matrix-vector product reads the 1 GiB matrix once
    mat = src.view(32768, 16384)
    x = torch.ones(16384, device=dev, dtype=torch.float16)
    y = torch.empty(32768, device=dev, dtype=torch.float16)
    t_mv = timed(lambda: torch.mv(mat, x, out=y))
    del src, dst, mat, x, y
    return {"fp16_matmul_tflops": 2.0 * n ** 3 / t_mm / 1e12,
            "copy_gbs": 2.0 * nbytes / t_cp / 1e9,
            "read_gbs": nbytes / min(t_sum, t_mv) / 1e9,
            "read_gbs_sum": nbytes / t_sum / 1e9, "read_gbs_mv": nbytes / t_mv / 1e9,
            "how": "torch.matmul fp16 [8192x8192]x[8192x8192] (hipBLASLt); copy_ of 1 GiB fp16 "
                   "(bytes read + written); read stream = the faster of torch.sum over and "
                   "torch.mv with a [32768x16384] fp16 matrix of that 1 GiB; HIP events, after "
                   "the timed region"}


def lds_probe(torch, iters: int = 2000, reps: int = 20) -> dict:
    """LDS read bandwidth of one CU for the forward's two LDS read
    instructions (ds_read_b128 for K, ds_read_b64_tr_b16 for V) at 4, 8 and
    16 waves per CU: one workgroup per CU, every wave reading a 64 KiB LDS
    block over and over (libfa2probe.so).  Bytes per clock per CU use the
    shader clock that wave 0 of workgroup 0 measured over its loop."""
    import ctypes

    from exact_attention_fwd_amd import _build

    if not os.path.exists(_build.PROBE_PATH):
        raise RuntimeError(f"{_build.PROBE_PATH} is not built (python -m exact_attention_fwd_amd._build)")
    lib = ctypes.CDLL(_build.PROBE_PATH)
    lib.fa2probe_lds_read.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(ctypes.c_double)]
    lib.fa2probe_lds_read.restype = ctypes.c_int
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    points = []
    for mode, name in ((0, "ds_read_b128"), (1, "ds_read_b64_tr_b16")):
        for waves in (4, 8, 16):
            out = (ctypes.c_double * 3)()
            rc = lib.fa2probe_lds_read(mode, 64 * waves, n_cu, iters, reps, out)
            if rc != 0:
                raise RuntimeError(f"fa2probe_lds_read({name}, {waves} waves) failed: {rc}")
            ms, nbytes, ghz = out[0], out[1], out[2]
            rate = nbytes / (ms * 1e-3)
            points.append({"instruction": name, "waves_per_cu": waves, "ms": round(ms, 4),
                           "tb_s": round(rate / 1e12, 2), "clock_ghz": round(ghz, 3),
                           "bytes_per_clk_per_cu": round(rate / (ghz * 1e9) / n_cu, 1)})
            log(f"[lds] {name} {waves} waves/CU: {rate / 1e12:.1f} TB/s at {ghz:.2f} GHz, "
                f"{points[-1]['bytes_per_clk_per_cu']} B/clk/CU")
    return {"metric": "LDS read bandwidth per CU", "unit": "bytes/clk/CU", "cus": n_cu,
            "points": points,
            "how": f"one workgroup of 64*waves threads per CU; each wave reads a 64 KiB LDS block "
                   f"{iters} x 16 times (conflict-free consecutive lane segments); {reps} launches "
                   f"timed with HIP events after 3 untimed; clock from s_memtime / s_memrealtime "
                   f"of wave 0"}


def valu_probe(torch, iters: int = 4000) -> dict:
    """VALU issue rate (libfa2probe.so): shader-clock cycles per instruction
    for 16 independent chains of v_add_f32, v_fma_f32, v_exp_f32, and the
    mixes exp2 + add and exp2 + add + mul (cycles per group), at 1 to 4 waves
    per SIMD (one workgroup of 256 to 1024 threads per CU).  A SIMD serves
    its waves unevenly (the oldest runs ahead), so the per-SIMD rate comes
    from the longest wave loop of each workgroup, not from the mean."""
    import ctypes

    from exact_attention_fwd_amd import _build

    if not os.path.exists(_build.PROBE_PATH):
        raise RuntimeError(f"{_build.PROBE_PATH} is not built (python -m exact_attention_fwd_amd._build)")
    lib = ctypes.CDLL(_build.PROBE_PATH)
    lib.fa2probe_valu_issue.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_double)]
    lib.fa2probe_valu_issue.restype = ctypes.c_int
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    names = ("v_add_f32", "v_fma_f32", "v_exp_f32", "exp2+add", "exp2+add+mul")
    points = []
    for waves_per_simd in (1, 2, 3, 4):
        for kind, name in enumerate(names):
            out = (ctypes.c_double * 2)()
            rc = lib.fa2probe_valu_issue(kind, 256 * waves_per_simd, n_cu, iters, out)
            if rc != 0:
                raise RuntimeError(f"fa2probe_valu_issue({name}, {waves_per_simd}) failed: {rc}")
            points.append({"kind": name, "waves_per_simd": waves_per_simd,
                           "cycles_per_wave": round(out[0], 2), "cycles_per_simd": round(out[1], 2)})
            log(f"[valu] {name} {waves_per_simd} waves/SIMD: {out[0]:.2f} cycles per wave, "
                f"{out[1]:.2f} per SIMD")
    return {"metric": "VALU issue rate", "unit": "shader cycles per instruction (or group)",
            "points": points,
            "how": f"one workgroup per CU, 16 independent chains per wave, {iters} x 16 elements, "
                   f"s_memtime around each wave's loop; per wave: the mean of the waves' loop "
                   f"times; per SIMD: the longest loop of each workgroup's waves over the "
                   f"elements per SIMD, mean over workgroups"}


STEP_MODEL_MODES = ("mfma only", "sequential: S^T, softmax, P V", "pipelined, registers",
                    "pipelined, operands from LDS", "pipelined, operands from LDS, barrier per 2 tiles",
                    "sequential, operands from LDS",
                    "pipelined, LDS operands, barriers, K/V staged through registers",
                    "pipelined, LDS operands, barriers, K/V staged by direct loads to LDS")


def step_model_ceiling(torch, d: int, iters: int = 4096, reps: int = 3):
    """TFLOP/s of the step model's full variant (K/V staged through registers,
    two waves per SIMD, random operands) at head dim d, or None when the
    probe library is not built or the probe fails."""
    import ctypes

    from exact_attention_fwd_amd import _build

    if not os.path.exists(_build.PROBE_PATH):
        log(f"[bench] {_build.PROBE_PATH} is not built: no step-model ceiling")
        return None
    lib = ctypes.CDLL(_build.PROBE_PATH)
    lib.fa2probe_step_model.argtypes = [ctypes.c_int] * 7 + [ctypes.POINTER(ctypes.c_double)]
    lib.fa2probe_step_model.restype = ctypes.c_int
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    out = (ctypes.c_double * 4)()
    rc = lib.fa2probe_step_model(d, 6, 2, 1, n_cu * 2, iters, reps, out)
    if rc != 0:
        # context for the bench line, not part of it: report and go on
        log(f"[bench] fa2probe_step_model({d}) failed ({rc}): no step-model ceiling")
        return None
    return out[1]


def step_probe(torch, iters: int = 4096, rounds: int = 2, reps: int = 3) -> dict:
    """A ceiling for the forward's key step at d = 64 and d = 128
    (libfa2probe.so): per wave the MFMAs of one 64-key tile against 32
    queries (d/4 of them) and the softmax VALU work between them, with
    no output written, in variants that add the kernel's parts one at a time
    (STEP_MODEL_MODES) up to the K/V staging from HBM, at the waves per SIMD
    the registers allow; once with random fp16 operands like the forward's
    N(0, 1) inputs and once with small smooth ones (the clock under an MFMA
    load depends on the operand bits that toggle).
    TFLOP/s count the MFMA work only, like the forward's rate; one workgroup
    per CU, `rounds` workgroups per CU in turn."""
    import ctypes

    from exact_attention_fwd_amd import _build

    if not os.path.exists(_build.PROBE_PATH):
        raise RuntimeError(f"{_build.PROBE_PATH} is not built (python -m exact_attention_fwd_amd._build)")
    lib = ctypes.CDLL(_build.PROBE_PATH)
    lib.fa2probe_step_model.argtypes = [ctypes.c_int] * 7 + [ctypes.POINTER(ctypes.c_double)]
    lib.fa2probe_step_model.restype = ctypes.c_int
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    max_waves = {64: (4, 4, 3, 2, 2, 3, 2, 2), 128: (3, 3, 2, 2, 2, 2, 2, 2)}
    points = []
    for data in ("random", "smooth"):
        for d in (64, 128):
            for mode, name in enumerate(STEP_MODEL_MODES):
                for w in range(1, max_waves[d][mode] + 1):
                    if w == 1 and (mode >= 6 or (d == 128 and mode == 4)):
                        continue
                    out = (ctypes.c_double * 4)()
                    rc = lib.fa2probe_step_model(d, mode, w, int(data == "random"), n_cu * rounds, iters,
                                                 reps, out)
                    if rc != 0:
                        raise RuntimeError(f"fa2probe_step_model({d}, {mode}, {w}, {data}) failed: {rc}")
                    points.append({"data": data, "d": d, "mode": name, "waves_per_simd": w,
                                   "ms": round(out[0], 4), "tflops": round(out[1], 1),
                                   "clock_ghz": round(out[2], 3), "mfma_busy": round(out[3], 3)})
                    log(f"[step] {data} d={d} {name}, {w} waves/SIMD: {out[1]:.1f} TFLOP/s, "
                        f"{out[2]:.2f} GHz, MFMA busy {out[3]:.3f}")
    return {"metric": "key-step model", "unit": "TFLOP/s (MFMA work)", "points": points,
            "how": f"{n_cu * rounds} workgroups of 256 x waves-per-SIMD threads, one per CU at a time, "
                   f"{iters} tiles per wave, {reps} launches timed after one untimed"}


def bwd_flops(w) -> float:
    """10*B*H*N^2*d: S = Q K^T, dP = dO V^T, dV = P^T dO, dK = dS^T Q and
    dQ = dS K, 2*N^2*d each per head; halved when causal."""
    f = 10.0 * w.B * w.H * w.N * w.N * w.d
    return f / 2 if w.causal else f


def upstream_grad(w):
    """The seeded upstream gradient dO of a workload, N(0, 1) in fp16."""
    from exact_attention_fwd_amd.workloads import make_qkv
    return make_qkv(w.B, w.H, w.N, w.d, 1.0, w.seed + 7919)[0]


def cpu_baseline_bwd(w, q, k, v, do, budget_s: float):
    """Time the gradient oracle on whole heads, as many as fit ~budget_s."""
    from oracle import attention_bwd_fp64
    from oracle.attention import oracle_threads

    threads = oracle_threads()
    t0 = time.perf_counter()
    attention_bwd_fp64(q[:1, :1], k[:1, :1], v[:1, :1], do[:1, :1], w.scale, causal=w.causal,
                       threads=1)
    one = max(time.perf_counter() - t0, 1e-4)
    n_heads = max(1, int(min(w.B * w.H, max(threads, budget_s * threads / one))))
    sl = (x.reshape(1, w.B * w.H, w.N, w.d)[:, :n_heads] for x in (q, k, v, do))
    t0 = time.perf_counter()
    attention_bwd_fp64(*sl, w.scale, causal=w.causal, threads=threads)
    dt = time.perf_counter() - t0
    flops = n_heads * bwd_flops(w) / (w.B * w.H)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_heads} of {w.B * w.H} heads of {w.name}, all gradients",
            "seconds": round(dt, 3)}


def time_calls(step, sync, warmup=None, steps=None):
    """Warm up (default ~0.4 s) and time (default ~0.25 s) back-to-back calls;
    returns (steps, warmup, seconds per call)."""
    n_probe = 5
    sync()
    tp0 = time.perf_counter()
    for _ in range(n_probe):
        step()
    sync()
    t_one = max((time.perf_counter() - tp0) / n_probe, 1e-6)
    warmup = max(20, math.ceil(0.4 / t_one)) if warmup is None else warmup
    steps = max(10, math.ceil(0.25 / t_one)) if steps is None else steps
    for _ in range(max(0, warmup - n_probe)):
        step()
    sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    sync()
    return steps, warmup, (time.perf_counter() - t0) / steps


def _load_fwd(path):
    """fa2_fwd of a library build at ``path`` (its own handle)."""
    import ctypes
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL)
    lib.fa2_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.fa2_fwd.restype = ctypes.c_int
    return lib


def tile_sweep_configs(d: int, causal: bool):
    """The forward's compile-time tile choices worth timing at head dim d:
    waves per workgroup (4 or 8 where the row's chunks divide evenly), K/V
    tiles in LDS per tensor (2 or 4; 2 at d = 256), LDS operand reads ahead
    of the MFMAs (3, 4, 5) and, in 8-wave groups, the raised priority of the
    younger half (on, off).  Each is a dict of the FA2_FWD_* macros."""
    out = []
    for waves in ((4, 8) if d in (64, 128) else (0,)):
        for bufs in ((2, 4) if d != 256 else (2,)):
            for ahead in (3, 4, 5):
                for prio in ((1, 0) if waves == 8 else (1,)):
                    out.append({"FA2_FWD_WAVES": waves, "FA2_FWD_KV_BUFS": bufs,
                                "FA2_FWD_AHEAD": ahead, "FA2_FWD_PRIO": prio})
    return out


def tile_sweep(args, w, torch):
    """Offline sweep of the forward's tile choices: rebuild the library once
    per configuration (parallel hipcc jobs into a temporary folder), check
    each build's output bit for bit against the in-tree one, and time them
    in interleaved rounds (HIP events, each round ~0.3 s of warm-up and
    ~0.2 s timed per configuration, the order reversed every other round)."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    import exact_attention_fwd_amd as fa2
    from exact_attention_fwd_amd import _build
    from exact_attention_fwd_amd.workloads import make_qkv

    cfgs = tile_sweep_configs(w.d, w.causal)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.sigma, w.seed)
    tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    with tempfile.TemporaryDirectory() as td:
        def mk(i):
            return _build.build(out=os.path.join(td, f"libfa2_{i}.so"),
                                defines=tuple(f"{k}={v}" for k, v in cfgs[i].items()))
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            paths = list(ex.map(mk, range(len(cfgs))))
        log(f"[sweep] built {len(paths)} libraries in {time.perf_counter() - t0:.0f} s")
        libs = [_load_fwd(p) for p in paths]
        ref_o, ref_l = fa2.fwd(tq, tk, tv, scale=w.scale, causal=w.causal)
        outs = []
        for lib in libs:
            o = torch.empty_like(tq)
            lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
            st = lib.fa2_fwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), w.B, w.H, w.N, w.d, w.scale, int(w.causal),
                             stream.cuda_stream)
            if st != fa2.FA2_OK:
                raise RuntimeError(f"sweep build failed to launch: {fa2.fa2_status_string(st)}")
            outs.append((o, lse))
        torch.cuda.synchronize(dev)
        same = [bool(torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
                     and torch.equal(l.view(torch.int32), ref_l.view(torch.int32))) for o, l in outs]
        times = [[] for _ in libs]
        for r in range(args.sweep_rounds):
            order = range(len(libs)) if r % 2 == 0 else reversed(range(len(libs)))
            for i in order:
                o, lse = outs[i]
                a = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.N, w.d, w.scale, int(w.causal), stream.cuda_stream)

                def step(lib=libs[i], a=a):
                    lib.fa2_fwd(*a)
                _, _, sec = time_calls(step, lambda: torch.cuda.synchronize(dev), warmup=None, steps=None)
                times[i].append(sec)
        flops = w.flops()
        rows = []
        for c, t, sm in zip(cfgs, times, same):
            med = sorted(t)[len(t) // 2]
            rows.append({**c, "ms": round(med * 1e3, 5), "tflops": round(flops / med / 1e12, 1),
                         "runs_ms": [round(x * 1e3, 5) for x in t], "bit_identical": sm})
        best = min(rows, key=lambda r: r["ms"])
        print(json.dumps({"metric": "forward tile sweep, TFLOP/s per configuration", "workload": w.name,
                          "configs": rows, "best": best}), flush=True)


def split_sweep(args, w, torch, fa2):
    """Split key/value forward of a decoding workload at each key-range
    count: HBM GB/s of algorithmic bytes per count."""
    from exact_attention_fwd_amd.workloads import make_decode_inputs

    q, k, v = make_decode_inputs(w)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    out = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.nq), dtype=torch.float32, device=dev)
    auto = fa2.fa2_splitkv_splits(w.B, w.H, w.nq, w.N, w.d, 0)
    points = []
    for req in (1, 2, 4, 8, 16, 32, 64, 128, 0):
        n = fa2.fa2_splitkv_splits(w.B, w.H, w.nq, w.N, w.d, req)
        wsb = fa2.fa2_splitkv_workspace_bytes(w.B, w.H, w.nq, w.N, w.d, req)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        a = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), lse.data_ptr(),
             ws.data_ptr(), wsb, w.B, w.H, w.nq, w.N, w.d, w.scale, req, stream.cuda_stream)

        def step(a=a):
            if fa2.fa2_fwd_splitkv(*a) != fa2.FA2_OK:
                raise RuntimeError("fa2_fwd_splitkv failed")
        _, _, sec = time_calls(step, lambda: torch.cuda.synchronize(dev))
        points.append({"requested": req, "n_splits": n, "auto": req == 0, "us": round(sec * 1e6, 2),
                       "gbs": round(w.hbm_bytes() / sec / 1e9, 1)})
        log(f"[split-sweep] {points[-1]}")
    print(json.dumps({"metric": "split key/value forward HBM GB/s per key-range count",
                      "workload": w.name, "auto_splits": auto, "points": points}), flush=True)


def batch_sweep(torch, fa2):
    """FA2 vs the FA1 loop order at [B, 32, 2048, 64], B = 1 .. 16."""
    from exact_attention_fwd_amd.workloads import make_qkv

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    H, N, d = 32, 2048, 64
    points = []
    for B in (1, 2, 4, 8, 16):
        tq, tk, tv = (torch.from_numpy(x).to(dev) for x in make_qkv(B, H, N, d, 1.0, 0))
        out = torch.empty_like(tq)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        ws_bytes = fa2.fa1_workspace_bytes(B, H, N, d)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        for causal in (False, True):
            row = {"B": B, "H": H, "N": N, "d": d, "causal": causal}
            for impl in ("fa2", "fa1"):
                if impl == "fa2":
                    a = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         B, H, N, d, d ** -0.5, causal, stream.cuda_stream)
                    call = fa2.fa2_fwd
                else:
                    a = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         ws.data_ptr(), ws_bytes, B, H, N, d, d ** -0.5, causal, stream.cuda_stream)
                    call = fa2.fa1_fwd

                def step():
                    if call(*a) != fa2.FA2_OK:
                        raise RuntimeError(f"{impl} failed")
                _, _, sec = time_calls(step, lambda: torch.cuda.synchronize(dev))
                flops = 4.0 * B * H * N * N * d / (2 if causal else 1)
                row[f"{impl}_ms"] = round(sec * 1e3, 5)
                row[f"{impl}_tflops"] = round(flops / sec / 1e12, 2)
            row["fa2_over_fa1"] = round(row["fa1_ms"] / row["fa2_ms"], 3)
            log(f"[sweep] {row}")
            points.append(row)
    return points


def bench_decode(args, w, torch, fa2):
    """A decoding workload through the split key/value path; prints one JSON line."""
    import numpy as np

    from exact_attention_fwd_amd.workloads import make_decode_inputs
    from oracle import attention_fp64

    log(f"[bench] decode workload {w.name} B={w.B} H={w.H} Nq={w.nq} Nk={w.N} d={w.d}")
    q, k, v = make_decode_inputs(w)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    out = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.nq), dtype=torch.float32, device=dev)
    n_splits = fa2.fa2_splitkv_splits(w.B, w.H, w.nq, w.N, w.d, 0)
    ws_bytes = fa2.fa2_splitkv_workspace_bytes(w.B, w.H, w.nq, w.N, w.d, 0)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    a = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), lse.data_ptr(), ws.data_ptr(),
         ws_bytes, w.B, w.H, w.nq, w.N, w.d, w.scale, 0, stream.cuda_stream)

    def step():
        if fa2.fa2_fwd_splitkv(*a) != fa2.FA2_OK:
            raise RuntimeError("fa2_fwd_splitkv failed")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    def timed():
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
    steps, warmup, sec = time_calls(step, lambda: torch.cuda.synchronize(dev), args.warmup, args.steps)
    args.steps, args.warmup = steps, warmup
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    timed()
    torch.cuda.synchronize(dev)
    wall = (time.perf_counter() - t0) / steps
    ev_ms = ev0.elapsed_time(ev1) / steps
    byt = w.hbm_bytes()
    value = byt / wall / 1e9
    achieved = byt / (ev_ms * 1e-3) / 1e9
    log(f"[bench] {steps} calls ({n_splits} key ranges): wall {wall * 1e3:.4f} ms/call, events "
        f"{ev_ms:.4f} ms, {value:.0f} GB/s ({100 * value / PEAK_HBM_GBS:.1f}% of HBM peak)")
    result = {
        "metric": METRIC_DECODE, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(wall * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} [B={w.B},H={w.H},Nq={w.nq},Nk={w.N},d={w.d}] non-causal "
                               f"fp16, N(0,{w.sigma:g}^2) inputs, {n_splits} key ranges",
                   "B": w.B, "H": w.H, "Nq": w.nq, "Nk": w.N, "d": w.d, "causal": False,
                   "n_splits": n_splits, "global_batch": w.B, "seq_len": w.N,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("decode", w.name),
                     "launch_ms": round(ev_ms, 5)},
    }
    if not args.no_parity:
        o_ref, l_ref = attention_fp64(q, k, v, w.scale)
        d_o = np.abs(out.cpu().numpy().astype(np.float64) - o_ref)
        d_l = np.abs(lse.cpu().numpy().astype(np.float64) - l_ref) / np.maximum(np.abs(l_ref), 1)
        result["parity"] = {"rows": int(w.B * w.H * w.nq), "max_abs_dO": float(d_o.max()),
                            "mean_abs_dO": float(d_o.mean()), "max_rel_dLSE": float(d_l.max()),
                            "pass": bool(d_o.max() <= 4e-3 and d_o.mean() <= 5e-4 and d_l.max() <= 1e-4)}
        log(f"[bench] parity {result['parity']}")
    if args.no_cpu_baseline:
        result["cpu_baseline"] = None
    else:
        from oracle.attention import oracle_threads
        t0 = time.perf_counter()
        attention_fp64(q, k, v, w.scale, threads=oracle_threads())
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": byt / dt / 1e9, "unit": "GB/s", "cores": oracle_threads(),
                                  "kind": "oracle", "sample": f"every row of {w.name}",
                                  "seconds": round(dt, 3)}
        log(f"[bench] cpu baseline {result['cpu_baseline']}")
    if not args.no_ceiling:
        ceil = measured_ceilings(torch, dev)
        best = max(ceil["read_gbs"], ceil["copy_gbs"])
        result["roofline"]["measured_ceiling"] = {
            "value": round(best, 1), "unit": "GB/s",
            "kind": "fastest library streaming kernel (copy_ read + write, torch.mv read)",
            "frac": round(result["roofline"]["achieved"] / best, 4),
            "copy_gbs": round(ceil["copy_gbs"], 1), "read_gbs": round(ceil["read_gbs"], 1),
            "how": ceil["how"]}
        log(f"[bench] measured ceilings {ceil}")
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: ~0.25 s worth)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default: ~0.4 s worth)")
    ap.add_argument("--workload", default="ref")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default) or the backward pass")
    ap.add_argument("--impl", choices=("fa2", "fa1"), default="fa2",
                    help="forward implementation: fa2_fwd (default) or the FA1-order comparator")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="instead: FA2 vs FA1 order at [B,32,2048,64], B = 1..16, one JSON line")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="instead: rebuild and time the forward's tile choices on the workload")
    ap.add_argument("--sweep-rounds", type=int, default=3, help="interleaved rounds of --tile-sweep")
    ap.add_argument("--split-sweep", action="store_true",
                    help="instead: time a decoding workload at each key-range count")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle wall time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the measured library ceilings (fp16 matmul, copy, read stream)")
    ap.add_argument("--ceiling", action="store_true",
                    help="instead: print only the measured library ceilings and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="instead: build profiles/traffic.json from rocprofv3 --pmc runs in DIR")
    ap.add_argument("--lds-probe", action="store_true",
                    help="instead: measure LDS read bandwidth per CU for ds_read_b128 and "
                         "ds_read_b64_tr_b16 at 4, 8 and 16 waves per CU, print one JSON line")
    ap.add_argument("--valu-probe", action="store_true",
                    help="instead: measure the VALU issue rate (add, fma, exp2 and mixes) at 1 to 4 "
                         "waves per SIMD, print one JSON line")
    ap.add_argument("--step-probe", action="store_true",
                    help="instead: time the register and LDS model of the d = 64 and d = 128 key step "
                         "(MFMAs alone, sequential, pipelined, + LDS operands, + barriers), print one "
                         "JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead: run a plain device copy of MIB MiB five times (the known-size "
                         "kernel that scales rocprofv3's FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()

    if args.summarize_counters:
        # entries from DIR replace those of the same path and workload;
        # the others (each with its own sha256 and factors) are kept
        res = summarize_counters(args.summarize_counters)
        try:
            with open(TRAFFIC_FILE) as f:
                old = json.load(f).get("workloads", {})
        except (OSError, ValueError):
            old = {}
        res["workloads"] = {**old, **res["workloads"]}
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(res, f, indent=1, sort_keys=True)
        for k, v in res["workloads"].items():
            log(f"[counters] {k}: {v['hbm_bytes_per_launch'] / 1e6:.2f} MB per call, "
                f"{v['ratio_to_algorithmic']}x algorithmic")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the attention forward of one "
              "(batch, head) shard needs no communication, so more GPUs would only shard B*H.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.ceiling:
        ceil = measured_ceilings(torch, torch.device("cuda:0"), seconds=1.0)
        ceil["fp16_matmul_frac_of_peak"] = ceil["fp16_matmul_tflops"] / PEAK_FP16_TFLOPS
        ceil["read_frac_of_peak"] = ceil["read_gbs"] / PEAK_HBM_GBS
        print(json.dumps(ceil), flush=True)
        return

    if args.lds_probe:
        print(json.dumps(lds_probe(torch)), flush=True)
        return

    if args.valu_probe:
        print(json.dumps(valu_probe(torch)), flush=True)
        return

    if args.step_probe:
        print(json.dumps(step_probe(torch)), flush=True)
        return

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 5}))
        return

    import exact_attention_fwd_amd as fa2
    from exact_attention_fwd_amd.workloads import WORKLOADS, make_qkv, sample_rows

    if args.batch_sweep:
        points = batch_sweep(torch, fa2)
        print(json.dumps({"metric": "FA2 vs FA1-order forward time, [B,32,2048,64] fp16",
                          "unit": "ms", "points": points}), flush=True)
        return

    w = WORKLOADS[args.workload]
    if args.tile_sweep:
        if w.Nq:
            ap.error("--tile-sweep times the square forward; pick a non-decoding workload")
        return tile_sweep(args, w, torch)
    if args.split_sweep:
        if not w.Nq:
            ap.error("--split-sweep needs a decoding workload (decode_64k, decode_b8_8k)")
        return split_sweep(args, w, torch, fa2)
    if w.Nq and (args.which != "fwd" or args.impl != "fa2"):
        ap.error(f"{w.name} is a decoding workload: it runs the split key/value forward only")
    if args.impl == "fa1" and (args.which != "fwd" or w.d != 64):
        ap.error("--impl fa1 is the forward comparator at head dim 64")
    if w.Nq:
        return bench_decode(args, w, torch, fa2)
    log(f"[bench] workload {w.name} B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.sigma, w.seed)
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    out = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # One validated call through the torch wrapper, then the timed steps call
    # the C entry point itself with the same (cached) pointers and stream.
    fa2.fwd(tq, tk, tv, scale=w.scale, causal=w.causal, out=out, lse=lse)
    if args.which == "fwd" and args.impl == "fa1":
        ws_bytes = fa2.fa1_workspace_bytes(w.B, w.H, w.N, w.d)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        entry = fa2.fa1_fwd
        args_c = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), lse.data_ptr(),
                  ws.data_ptr(), ws_bytes, w.B, w.H, w.N, w.d, w.scale, w.causal,
                  stream.cuda_stream)
    elif args.which == "fwd":
        entry = fa2.fa2_fwd
        args_c = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), lse.data_ptr(),
                  w.B, w.H, w.N, w.d, w.scale, w.causal, stream.cuda_stream)
    else:
        do = upstream_grad(w)
        tdo = torch.from_numpy(do).to(dev)
        gq, gk, gv, gdelta = fa2.bwd(tq, tk, tv, out, lse, tdo, scale=w.scale, causal=w.causal)
        entry = fa2.fa2_bwd
        args_c = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), lse.data_ptr(),
                  tdo.data_ptr(), gq.data_ptr(), gk.data_ptr(), gv.data_ptr(), gdelta.data_ptr(),
                  w.B, w.H, w.N, w.d, w.scale, w.causal, stream.cuda_stream)

    def step():
        status = entry(*args_c)
        if status != fa2.FA2_OK:
            raise RuntimeError(f"{args.which}: {fa2.fa2_status_string(status)}")

    # Size the default warm-up and timed loop from a few probe launches (they
    # count as warm-up).
    n_probe = 5
    torch.cuda.synchronize(dev)
    tp0 = time.perf_counter()
    for _ in range(n_probe):
        step()
    torch.cuda.synchronize(dev)
    t_one = max((time.perf_counter() - tp0) / n_probe, 1e-6)
    if args.warmup is None:
        args.warmup = max(20, math.ceil(0.4 / t_one))
    if args.steps is None:
        args.steps = max(10, math.ceil(0.25 / t_one))
    for _ in range(max(0, args.warmup - n_probe)):
        step()
    torch.cuda.synchronize(dev)

    # HIP events on the stream the kernel is launched on (torch's current one).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / args.steps

    flops = w.flops() if args.which == "fwd" else bwd_flops(w)
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (ev_ms * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps: wall {ms_per_step:.4f} ms/step, events {ev_ms:.4f} ms/launch, "
        f"{value:.1f} TFLOP/s ({100 * value / PEAK_FP16_TFLOPS:.1f}% of peak)")

    result = {
        "metric": (METRIC_BWD if args.which == "bwd" else
                   METRIC if args.impl == "fa2" else "FA1-order fwd TFLOP/s (comparator)"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} [B={w.B},H={w.H},N={w.N},d={w.d}] "
                               f"{'causal' if w.causal else 'non-causal'} fp16, N(0,{w.sigma:g}^2) inputs",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / PEAK_FP16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                     "traffic": measured_traffic(
                         "bwd" if args.which == "bwd" else args.impl.replace("fa2", "fwd"), w.name),
                     "launch_ms": round(ev_ms, 5)},
    }

    # The model of the key step, timed right after the timed region so that the
    # chip is in the same state (the clock under this load depends on it).
    step_model = None
    if (not args.no_ceiling and args.which == "fwd" and args.impl == "fa2" and not w.causal
            and w.d in (64, 128)):
        model = step_model_ceiling(torch, w.d)
        if model is not None:
            step_model = {
                "value": round(model, 1), "unit": "TFLOP/s", "frac": round(achieved / model, 4),
                "kind": f"the forward's key step at d = {w.d} alone (pipelined softmax, LDS operands, "
                        f"barriers, K/V staging; random fp16 operands; no prologue or epilogue)",
                "how": "bench.py --step-probe, last variant at two waves per SIMD, timed right after "
                       "the timed region"}
            log(f"[bench] step model {model:.1f} TFLOP/s")

    if args.which == "bwd":
        result["config"]["pass"] = "backward (dQ, dK, dV, delta)"
    if args.impl == "fa1":
        result["config"]["impl"] = "FA1 loop order (fa1_fwd)"
    if not args.no_parity and args.which == "bwd":
        # the first two heads of the timed output, every element: max error in
        # units of each gradient's worst-case rounding bound u (|G| + E + 2^-14)
        # (<= 2), rms error in units of the statistical one (u / sqrt 3) S (<= 1)
        from oracle import attention_bwd_fp64
        from oracle.attention_bwd import attention_bwd_error_scale, attention_bwd_error_std
        nh = min(2, w.B * w.H)
        sl = [x.reshape(1, w.B * w.H, w.N, w.d)[:, :nh] for x in (q, k, v, do)]
        ref = attention_bwd_fp64(*sl, w.scale, causal=w.causal)
        esc = attention_bwd_error_scale(*sl, w.scale, causal=w.causal)
        sdv = attention_bwd_error_std(*sl, w.scale, causal=w.causal)
        got = [t.reshape(1, w.B * w.H, *t.shape[2:])[:, :nh].cpu().numpy().astype(np.float64)
               for t in (gq, gk, gv, gdelta)]
        u = 2.0 ** -11
        ratios, rms = {}, {}
        for name, g, r, e, sd in zip(("dq", "dk", "dv", "delta"), got, ref, esc, sdv):
            ratios[name] = float((np.abs(g - r) / (u * (np.abs(r) + e + 2.0 ** -14))).max())
            den = float(np.sqrt(np.mean(np.square(sd)))) * u / math.sqrt(3.0)
            rms[name] = float(np.sqrt(np.mean(np.square(g - r)))) / den if den > 0 else 0.0
        result["parity"] = {"heads": nh, "max_ratio_to_rounding_bound": ratios,
                            "rms_ratio_to_statistical_bound": rms,
                            "pass": bool(max(ratios.values()) <= 2.0 and max(rms.values()) <= 1.0)}
        log(f"[bench] parity {result['parity']}")
    elif not args.no_parity:
        # sampled parity of the timed output, 64 seeded rows per (b, h)
        from oracle import attention_fp64
        rows = np.stack([np.stack([sample_rows(w.N, b, h, 64) for h in range(w.H)])
                         for b in range(w.B)])
        o_ref, l_ref = attention_fp64(q, k, v, w.scale, causal=w.causal, rows=rows)
        bi = np.arange(w.B)[:, None, None]
        hi = np.arange(w.H)[None, :, None]
        og = out.cpu().numpy()[bi, hi, rows].astype(np.float64)
        lg = lse.cpu().numpy()[bi, hi, rows].astype(np.float64)
        d_o = np.abs(og - o_ref)
        d_l = np.abs(lg - l_ref) / np.maximum(np.abs(l_ref), 1)
        result["parity"] = {"rows_per_head": 64, "max_abs_dO": float(d_o.max()),
                            "mean_abs_dO": float(d_o.mean()), "max_rel_dLSE": float(d_l.max()),
                            "pass": bool(d_o.max() <= 4e-3 and d_o.mean() <= 5e-4 and d_l.max() <= 1e-4)}
        log(f"[bench] parity {result['parity']}")

    if args.no_cpu_baseline:
        result["cpu_baseline"] = None
    else:
        log("[bench] timing the CPU oracle ...")
        result["cpu_baseline"] = (cpu_baseline(w, q, k, v, args.cpu_budget) if args.which == "fwd"
                                  else cpu_baseline_bwd(w, q, k, v, do, args.cpu_budget))
        log(f"[bench] cpu baseline {result['cpu_baseline']}")

    if not args.no_ceiling:
        ceil = measured_ceilings(torch, dev)
        result["roofline"]["measured_ceiling"] = {
            "value": round(ceil["fp16_matmul_tflops"], 1), "unit": "TFLOP/s",
            "kind": "dense fp16 matmul (hipBLASLt)",
            "frac": round(result["roofline"]["achieved"] / ceil["fp16_matmul_tflops"], 4),
            "copy_gbs": round(ceil["copy_gbs"], 1), "read_gbs": round(ceil["read_gbs"], 1),
            "how": ceil["how"]}
        log(f"[bench] measured ceilings {ceil}")
        if step_model is not None:
            result["roofline"]["measured_ceiling"]["step_model"] = step_model

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
