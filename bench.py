#!/usr/bin/env python3
"""Attention forward benchmark on one MI355X: TFLOP/s, fraction of the bf16
MFMA peak and L2 hit rate for each workgroup mapping mode.

One step = one attention forward pass (one kernel launch) over the workload's
synthetic inputs, which are resident in HBM before timing starts.  Default
workload: MHA, B=1, H_Q=H_KV=128, N=131072, d=128, non-causal, bf16 N(0,1)
inputs.  Every mapping mode is timed in turn; the headline value is Swizzled
Head-first.  Prints ONE JSON line on stdout (progress goes to stderr).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--modes 0,1,2,3] [--no-cpu-baseline]
  python bench.py --sweep OUT.md    every configuration x mapping mode, timed
  python bench.py --pass bwd [--workload NAME]   the backward pass (attn_bwd):
                  dQ, dK, dV from the forward's O and lse, one JSON line
  python bench.py --pass gemm [--workload NAME]  the CAC-scheduled GEMM
                  (cac_gemm) per tile map, with torch.mm as context
  python bench.py --pass decode [--workload NAME] split-KV decode (HBM-bound)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "fwd": ["chiplet_numa_aware_amd/csrc/attn_fwd_kernel.hpp",
            "chiplet_numa_aware_amd/csrc/wg_map.hpp",
            "chiplet_numa_aware_amd/csrc/fwd_launch.hpp",
            "chiplet_numa_aware_amd/csrc/attn_fwd_d64.hip",
            "chiplet_numa_aware_amd/csrc/attn_fwd_d128.hip",
            "chiplet_numa_aware_amd/csrc/attn_fwd.hip"],
    # the decode path of attn_fwd_split (units of at most 64 rows)
    "decode": ["chiplet_numa_aware_amd/csrc/decode_kernel.hpp",
               "chiplet_numa_aware_amd/csrc/attn_fwd_kernel.hpp",
               "chiplet_numa_aware_amd/csrc/wg_map.hpp",
               "chiplet_numa_aware_amd/csrc/attn_decode.hip",
               "chiplet_numa_aware_amd/csrc/merge_kernel.hpp"],
    "bwd": ["chiplet_numa_aware_amd/csrc/attn_bwd_kernel.hpp",
            "chiplet_numa_aware_amd/csrc/attn_fwd_kernel.hpp",
            "chiplet_numa_aware_amd/csrc/wg_map.hpp",
            "chiplet_numa_aware_amd/csrc/attn_bwd.hip"],
}
# Kernels whose counters a profile reports, per pass.
PASS_KERNELS = {"fwd": ["attn_fwd_kernel"],
                "bwd": ["attn_bwd_dkv_kernel", "attn_bwd_dq_kernel"],
                "gemm": ["cac_gemm_kernel"],
                "decode": ["attn_decode_kernel", "attn_merge_kernel"]}
DECODE_METRIC = "decode attention (attn_fwd_split + merge) GB/s against the HBM peak"
KERNEL_SOURCES["gemm"] = ["chiplet_numa_aware_amd/csrc/gemm_kernel.hpp",
                          "chiplet_numa_aware_amd/csrc/cac_map.hpp",
                          "chiplet_numa_aware_amd/csrc/attn_fwd_kernel.hpp",
                          "chiplet_numa_aware_amd/csrc/cac_gemm.hip"]
GEMM_METRIC = "CAC-scheduled bf16 GEMM TFLOP/s + % bf16 MFMA peak + L2 hit % per tile map"
GEMM_MODE_NAMES = ["naive_row_major", "naive_cluster", "swizzled_row_major", "swizzled_cluster"]
GEMM_WORKLOADS = {
    # name: (L, M, N, K); C = A B^T with A [L,M,K], B [L,N,K]
    # 8 tile columns: the dispatcher's round robin gives each XCD one column.
    "gemm_tall_64k_2k_8k": (1, 65536, 2048, 8192),
    "gemm_sq_16k": (1, 16384, 16384, 16384),
    # 4 tile columns, batched (per-batch B panels shared by the batch's tiles)
    "gemm_b8_16k_1k_4k": (8, 16384, 1024, 4096),
}
BWD_METRIC = "attn bwd TFLOP/s (dQ, dK, dV; 2.5x the forward's FLOPs) + % bf16 MFMA peak + L2 hit %"

METRIC = "attn fwd TFLOP/s + % bf16 MFMA peak + L2 hit %, MHA H=128 N=128K d=128"
# MI355X published dense bf16 MFMA peak (2.5 PFLOP/s).
PEAK_BF16_TFLOPS = 2500.0
_BASE_NAMES = ["naive_block_first", "naive_head_first",
               "swizzled_block_first", "swizzled_head_first"]
# Mode ids 0..15: the pages' four modes, each + 4 (longest first), and each
# of those + 8 (balanced split, which changes swizzled head-first only).
MODE_NAMES = _BASE_NAMES + [n + "_longest_first" for n in _BASE_NAMES]
MODE_NAMES = MODE_NAMES + [n + "_balanced_split" for n in MODE_NAMES]
SWEEP_MODES = (0, 1, 2, 3, 7, 15)
PROFILE_MODES = SWEEP_MODES  # one dispatch each, in this order, per profile pass

# Vector-ALU roofline of the online softmax.  Per (query, key) score the
# softmax needs one FMA (scale, minus the running max), one exp2, half a max3
# (the tile max, two scores per instruction), half a conversion to bf16 (two
# scores per instruction) and, where the head dim fills its padded width
# (d = 64 or 128), one add for the row sum; below it the P V MFMA sums the
# row through a 1 in V's padding.  A wave64 fp32 FMA, add, max3 or conversion
# issues in 4 SIMD cycles (16 lanes per cycle: 256 CUs x 4 SIMDs x 16 lanes x
# 2 FLOP x 2.4 GHz = 78.6 TFLOP/s, half the packed 157.3), v_exp_f32 in 8
# (measured: two issue slots).  So one wave's 64 scores take
# 4 + 8 + 2 + 2 (+ 4) = 16 (20) SIMD cycles.
SIMDS = 256 * 4
CLOCK_HZ = 2.4e9
SOFTMAX_SIMD_CYCLES_PER_WAVE = {"fma": 4, "exp2": 8, "max3_half": 2, "cvt_bf16_half": 2,
                                "add": 4}


def softmax_simd_cycles(d: int) -> int:
    """SIMD cycles of softmax vector work per wave64 of scores at head dim d."""
    c = dict(SOFTMAX_SIMD_CYCLES_PER_WAVE)
    if d not in (64, 128):
        del c["add"]
    return sum(c.values())


def alu_peak_tflops(d: int) -> float:
    """Credited TFLOP/s (4 d FLOP per score) at the softmax's vector-ALU
    bound."""
    return SIMDS * CLOCK_HZ * 64 / softmax_simd_cycles(d) * 4 * d / 1e12


def mfma_peak_tflops_credited(d: int) -> float:
    """Credited TFLOP/s at the MFMA peak: the kernel pads d to 64 or 128
    columns, and the padding is executed but not credited."""
    d_pad = 64 if d <= 64 else 128
    return PEAK_BF16_TFLOPS * d / d_pad


WORKLOADS = {
    # name: (B, H_Q, H_KV, N, d, causal)
    "mha_128k": (1, 128, 128, 131072, 128, False),
    "mha_128k_causal": (1, 128, 128, 131072, 128, True),
    "mha_32k": (1, 128, 128, 32768, 128, False),
    "mha_32k_causal": (1, 128, 128, 32768, 128, True),
    "mha_8k": (1, 128, 128, 8192, 128, False),
    "mha_8k_causal": (1, 128, 128, 8192, 128, True),
    "gqa64x8_128k_causal": (1, 64, 8, 131072, 128, True),
    "gqa64x8_32k_causal": (1, 64, 8, 32768, 128, True),
    "gqa64x8_8k_causal": (1, 64, 8, 8192, 128, True),
    "gqa32x4_b2_32k_causal": (2, 32, 4, 32768, 128, True),
    "mha12_b2_32k_causal": (2, 12, 12, 32768, 128, True),
    "mha12_b1_32k_causal": (1, 12, 12, 32768, 128, True),
    "dsv3_d56_128k_causal": (1, 128, 128, 131072, 56, True),
    "dsv3_d56_32k_causal": (1, 128, 128, 32768, 56, True),
    "mha_h8_1k": (1, 8, 8, 1024, 128, False),
    # K/V of one head (2 MiB) fits an XCD's L2: the kernel's compute-bound rate.
    "mha_b16_4k": (16, 128, 128, 4096, 128, False),
}


# The configurations measured per mapping mode (MHA at three lengths, causal
# and not; GQA 64/8 causal; the fallback shapes; d = 56).
SWEEP = ["mha_h8_1k", "mha_8k", "mha_8k_causal", "mha_32k", "mha_32k_causal",
         "mha_128k", "mha_128k_causal", "gqa64x8_8k_causal", "gqa64x8_32k_causal",
         "gqa64x8_128k_causal", "gqa32x4_b2_32k_causal", "mha12_b2_32k_causal",
         "mha12_b1_32k_causal", "dsv3_d56_32k_causal", "dsv3_d56_128k_causal"]


# Split-KV (decode) configurations: (B, H_Q, H_KV, N_q, N_kv, d, causal,
# splits).  Decode streams each KV head once, so HBM bandwidth bounds it.
SPLIT_WORKLOADS = {
    "decode_gqa64x8_b16_128k": (16, 64, 8, 1, 131072, 128, True, 16),
    "decode_gqa64x8_b64_32k": (64, 64, 8, 1, 32768, 128, True, 8),
    "decode_mha32_b8_32k": (8, 32, 32, 1, 32768, 128, True, 16),
}
HBM_PEAK_GBS = 8000.0


def split_bytes(B, H_Q, H_KV, N_q, N_kv, d, S) -> float:
    """Unique bytes of one call: Q, K, V, O (bf16), lse, and the fp32
    partials written and read back when S > 1."""
    rows = B * H_Q * N_q
    ws = 2 * S * rows * (d + 1) * 4 if S > 1 else 0
    return 2.0 * (2 * rows * d + 2 * B * H_KV * N_kv * d) + 4 * rows + ws


def device_info() -> dict:
    """GPU, partition and software versions the numbers were taken with."""
    import torch

    import chiplet_numa_aware_amd as attn
    props = torch.cuda.get_device_properties(0)
    xcd = attn.attn_num_xcd()
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "cus": props.multi_processor_count, "xcds": xcd,
            "partition": "SPX (one device spans all 8 XCDs)" if xcd == 8 else f"{xcd} XCDs",
            "rocm": rocm, "hip": torch.version.hip,
            "host_cores": len(os.sched_getaffinity(0))}


def emit(out: dict, args) -> None:
    """Prints the one JSON line (and writes it to --json-out when given)."""
    line = json.dumps(out)
    if getattr(args, "json_out", None):
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_flops(B, H_Q, N, d, causal) -> float:
    """Algorithmic FLOPs: QK^T and PV, 2*d each per (query, visible key)."""
    pairs = N * (N + 1) // 2 if causal else N * N
    return 4.0 * B * H_Q * d * pairs


def pass_flops(which, B, H_Q, N, d, causal) -> float:
    """Forward: attn_flops.  Backward: the five products of the gradient
    (S = Q K^T again, dV, dP, dQ, dK), 2*d each per (query, visible key),
    i.e. 2.5x the forward (the usual convention; the kernels recompute S and
    dP once more for dQ, which is not counted)."""
    f = attn_flops(B, H_Q, N, d, causal)
    return f if which == "fwd" else 2.5 * f


def describe(name) -> str:
    B, H_Q, H_KV, N, d, causal = WORKLOADS[name]
    kind = "MHA" if H_Q == H_KV else "GQA"
    return (f"{kind} fwd B={B} H_Q={H_Q} H_KV={H_KV} N={N} d={d} "
            f"{'causal' if causal else 'non-causal'}")


def kernel_hash(which: str = "fwd") -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[which]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_path(workload: str, which: str = "fwd") -> str:
    name = {"gemm": f"counters_gemm_{workload}.json",
            "decode": f"counters_decode_{workload}.json"}.get(
                which, f"counters_attn_{which}_{workload}.json")
    return os.path.join(PROFILES, name)


def stored_counters(workload: str, khash: str, which: str = "fwd"):
    """Counter-derived figures (L2 hit, HBM bytes) kept under profiles/ for
    this workload, or None when absent or taken on another kernel version."""
    path = counters_path(workload, which)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("kernel_hash") != khash:
        return None
    return data


def counters_source(workload: str, khash: str, which: str = "fwd", counters=None):
    """Where a line's l2_hit_pct / traffic come from: a committed rocprofv3
    counter summary of the same kernel sources (its file and hash), taken in
    a separate profiled run, not in this timed one."""
    if counters is None:
        return None
    return {"file": os.path.relpath(counters_path(workload, which), ROOT),
            "kernel_hash": khash,
            "note": "rocprofv3 counter passes recorded in that file (a separate "
                    "profiled process, possibly another box); not measured in "
                    "this timed run"}


def time_mode(attn, q, k, v, o, lse, causal, mode, steps, warmup, flops):
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        attn.attn_fwd(q, k, v, causal=causal, mapping=mode, o=o, lse=lse,
                      stream=stream)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        attn.attn_fwd(q, k, v, causal=causal, mapping=mode, o=o, lse=lse,
                      stream=stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_kernel_s = sum(kern_ms) / len(kern_ms) / 1e3
    med_ms = sorted(kern_ms)[len(kern_ms) // 2]
    return {
        "ms_per_step": wall / steps * 1e3,
        "tflops": flops / (wall / steps) / 1e12,
        "kernel_ms_avg": avg_kernel_s * 1e3,
        "kernel_ms_min": min(kern_ms),
        "kernel_ms_median": med_ms,
        "kernel_tflops": flops / avg_kernel_s / 1e12,
        "pct_peak": 100.0 * flops / avg_kernel_s / 1e12 / PEAK_BF16_TFLOPS,
    }


def time_calls(call, steps, warmup, flops):
    """`call(stream)` timed like time_mode: HIP events around each call on the
    stream the kernels run on, and the wall clock over all of them."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        call(stream)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        call(stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    avg_s = sum(kern_ms) / len(kern_ms) / 1e3
    return {
        "ms_per_step": wall / steps * 1e3,
        "tflops": flops / (wall / steps) / 1e12,
        "kernel_ms_avg": avg_s * 1e3,
        "kernel_ms_min": min(kern_ms),
        "kernel_ms_median": sorted(kern_ms)[len(kern_ms) // 2],
        "kernel_tflops": flops / avg_s / 1e12,
        "pct_peak": 100.0 * flops / avg_s / 1e12 / PEAK_BF16_TFLOPS,
    }


def cpu_baseline(q, k, v, causal, budget_s: float):
    """The fp64 oracle timed on this host on sampled rows of the workload."""
    import numpy as np
    import oracle  # the cpu_baseline leg is the one place bench.py uses it
    from chiplet_numa_aware_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    B, H_Q, N, d = q.shape
    H_KV = k.shape[1]
    # Up to 48 (b, h) pairs x 512 rows: about 10-20 s of fp64 work on a
    # 16-core host at the headline shape; the loop stops at the budget.
    rows_per_pair = 512
    samples = inputs.sample_rows(B, H_Q, H_KV, N, n_pairs=48,
                                 n_rows=rows_per_pair, seed=1234)
    done_flops, done_s, pairs = 0.0, 0.0, 0
    for b, h, rows in samples:
        g = oracle.kv_head(h, H_Q, H_KV)
        qh = q[b, h].float().cpu().numpy()[rows]
        kh = k[b, g].float().cpu().numpy()
        vh = v[b, g].float().cpu().numpy()
        t0 = time.perf_counter()
        oracle.attention_head_rows(qh, kh, vh, rows, causal)
        done_s += time.perf_counter() - t0
        allowed = (rows + 1) if causal else np.full(len(rows), N)
        done_flops += float(4.0 * d * allowed.sum())
        pairs += 1
        if done_s >= budget_s:
            break
    return {
        "value": done_flops / done_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{pairs} (batch, head) pairs x {rows_per_pair} query rows "
                   f"of the workload (seed 1234), fp64 numpy, "
                   f"{done_flops / 1e9:.1f} GFLOP in {done_s:.1f} s"),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


PROFILE_PASSES = {
    # pass name: counters (each pass is its own rocprofv3 run)
    "l2": ["TCC_HIT_sum", "TCC_MISS_sum"],
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "mfma": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
             "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
    # where the non-MFMA time goes: instruction mix and waits (wave-cycles
    # in units of 4 cycles)
    "issue": ["SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA"],
    "waits": ["SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY"],
}


def profile_commands(workload: str, out: str, which: str = "fwd"):
    """The rocprofv3 runs whose output --summarize-profile reads."""
    bench = "python3 /root/repo/bench.py"
    modes = "0,1,2,3" if which in ("gemm", "decode") else ",".join(map(str, PROFILE_MODES))
    sel = f"--workload {workload}" + ("" if which == "fwd" else f" --pass {which}")
    one = f"{bench} {sel} --steps 1 --warmup 0 --modes {modes} --no-cpu-baseline"
    # First the plain benchmark on the same box (its per-mode kernel times
    # are what the summary divides the algorithmic work by), then the traces.
    cmds = {"bench": (f"{bench} {sel} --steps 3 --warmup 1 --modes {modes} --no-cpu-baseline "
                      f"--json-out {out}/bench.json"),
            "trace": (f"rocprofv3 --kernel-trace --stats --output-format csv -d {out}/trace -o trace -- "
                      f"{bench} {sel} --steps 2 --warmup 1 --modes {modes} --no-cpu-baseline")}
    for name, ctrs in PROFILE_PASSES.items():
        cmds[name] = (f"rocprofv3 --pmc {' '.join(ctrs)} --output-format csv -d {out}/{name} -o {name} -- {one}")
    for name in ("fetch", "write"):
        cmds["copy_" + name] = (f"rocprofv3 --pmc {' '.join(PROFILE_PASSES[name])} --output-format csv "
                                f"-d {out}/copy_{name} -o copy_{name} -- {bench} --copy-calibration")
    return cmds


def _read_counters(path, kernel_substr):
    """{dispatch_id: {counter: value summed over dimensions}} and durations."""
    import csv
    vals, dur = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_substr not in r["Kernel_Name"]:
                continue
            dk = int(r["Dispatch_Id"])
            vals.setdefault(dk, {})
            vals[dk][r["Counter_Name"]] = vals[dk].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            dur[dk] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    return [vals[k] for k in sorted(vals)], [dur[k] for k in sorted(dur)]


def _recorded_commands(directory: str, workload: str, which: str = "fwd"):
    """The commands the profiling run executed: `commands.txt` written there
    by --print-profile-commands, else the commands for that directory."""
    path = os.path.join(directory, "commands.txt")
    if os.path.exists(path):
        import re
        with open(path) as f:
            # /root/repo is a link to wherever the run's copy of the
            # repository lived; name its paths through it
            cmds = [re.sub(r"/\S*?/repo/", "/root/repo/", line.strip())
                    for line in f if line.strip()]
        return dict(zip(profile_commands(workload, "X", which).keys(), cmds))
    return profile_commands(workload, os.path.abspath(directory), which)


def _headline_mode(modes, causal: bool) -> int:
    """The mapping a bench line reports as its value: the binding's default
    (swizzled head-first; with a causal mask also longest first and the
    balanced split) when it was timed, else the closest one timed."""
    for m in ((15, 7, 3) if causal else (3,)):
        if m in modes:
            return m
    return modes[-1]


def _same_box_bench(directory: str):
    """Per-mode results of the bench run recorded in DIR/bench.json (the
    profile's first command), or None."""
    path = os.path.join(directory, "bench.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        lines = [ln for ln in f.read().splitlines() if ln.strip()]
    return json.loads(lines[-1]).get("modes") if lines else None


def _issue_summary(c) -> dict:
    """Instructions per MFMA and the split of wave-cycles from one dispatch's
    issue (SQ_INSTS_*) and waits (SQ_WAIT_*, SQ_ACTIVE_INST_ANY) counters."""
    n_mfma = max(c["SQ_INSTS_MFMA"], 1.0)
    return {
        # SQ_INSTS_VALU counts the MFMAs too
        "valu_per_mfma": round((c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]) / n_mfma, 3),
        "salu_per_mfma": round(c["SQ_INSTS_SALU"] / n_mfma, 3),
        "lds_per_mfma": round(c["SQ_INSTS_LDS"] / n_mfma, 3),
        "active_inst_pct": round(100.0 * c["SQ_ACTIVE_INST_ANY"] / c["SQ_WAVE_CYCLES"], 2),
        "wait_any_pct": round(100.0 * c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"], 2),
        "wait_inst_any_pct": round(100.0 * c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"], 2),
    }


ISSUE_TABLE_HEAD = [
    "Instructions per MFMA (SQ_INSTS_*; VALU without the MFMAs) and the share of wave-cycles "
    "spent issuing (SQ_ACTIVE_INST_ANY), waiting on s_waitcnt or a barrier (SQ_WAIT_ANY) and "
    "waiting to issue (SQ_WAIT_INST_ANY), of SQ_WAVE_CYCLES.", "",
    "| mode | VALU / MFMA | SALU / MFMA | LDS / MFMA | issuing % | waitcnt+barrier % | issue-wait % |",
    "|---|---|---|---|---|---|---|"]


def _issue_row(name, i) -> str:
    return (f"| {name} | {i['valu_per_mfma']} | {i['salu_per_mfma']} | {i['lds_per_mfma']} | "
            f"{i['active_inst_pct']} | {i['wait_any_pct']} | {i['wait_inst_any_pct']} |")


def summarize_profile(directory: str, workload: str):
    """Turns the rocprofv3 CSVs of profile_commands() into profiles/ files."""
    import csv
    import glob
    B, H_Q, H_KV, N, d, causal = WORKLOADS[workload]
    flops = attn_flops(B, H_Q, N, d, causal)

    def one(pass_name, kernel="attn_fwd_kernel"):
        files = glob.glob(os.path.join(directory, pass_name, "*_counter_collection.csv"))
        if not files:
            raise SystemExit(f"missing {pass_name} counters under {directory}")
        return _read_counters(files[0], kernel)

    # Copy calibration: a plain 1 GiB device copy; its last dispatch is timed.
    cal = {}
    for name, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        v, _ = one("copy_" + name, kernel="copyBuffer")
        kib = v[-1][ctr]
        cal[ctr] = (1 << 30) / (kib * 1024.0)
    l2, durs = one("l2")
    fe, _ = one("fetch")
    wr, _ = one("write")
    mf, mdur = one("mfma")
    iss = None
    if (glob.glob(os.path.join(directory, "issue", "*_counter_collection.csv"))
            and glob.glob(os.path.join(directory, "waits", "*_counter_collection.csv"))):
        ia, _ = one("issue")
        ib, _ = one("waits")
        iss = [dict(a, **b) for a, b in zip(ia, ib)] if len(ia) == len(ib) else None
    same_box = _same_box_bench(directory)
    n_modes = len(l2)
    if not (len(fe) == len(wr) == len(mf) == n_modes == len(PROFILE_MODES)):
        raise SystemExit("expected one dispatch per mapping mode in every pass")
    # Kernel-trace statistics (average duration of the attention kernel).
    trace = glob.glob(os.path.join(directory, "trace", "*_kernel_stats.csv"))
    stats = []
    if trace:
        with open(trace[0]) as f:
            stats = [r for r in csv.DictReader(f)]
    unique = (2 * H_Q + 2 * H_KV) * B * N * d * 2 + 4 * B * H_Q * N
    modes = {}
    for m in range(n_modes):
        hit, miss = l2[m]["TCC_HIT_sum"], l2[m]["TCC_MISS_sum"]
        fetch_b = fe[m]["FETCH_SIZE"] * 1024.0 * cal["FETCH_SIZE"]
        write_b = wr[m]["WRITE_SIZE"] * 1024.0 * cal["WRITE_SIZE"]
        gui = mf[m]["GRBM_GUI_ACTIVE"]
        # GRBM_GUI_ACTIVE sums the busy cycles of every XCD.
        clock = gui / 8.0 / mdur[m] / 1e9
        simd_cycles = gui / 8.0 * 1024  # 256 CUs x 4 SIMDs
        modes[MODE_NAMES[PROFILE_MODES[m]]] = {
            "l2_hit_pct": round(100.0 * hit / (hit + miss), 2),
            "fetch_bytes": fetch_b, "write_bytes": write_b,
            "hbm_bytes": fetch_b + write_b,
            "fetch_over_unique": round(fetch_b / unique, 2),
            "mfma_busy_pct": round(100.0 * mf[m]["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles, 2),
            "mfma_flops_counted": mf[m]["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0,
            "clock_ghz": round(clock, 3),
            "kernel_ms_counter_run": round(durs[m] * 1e3, 2),
        }
        entry = modes[MODE_NAMES[PROFILE_MODES[m]]]
        if iss is not None and len(iss) == n_modes:
            entry["issue"] = _issue_summary(iss[m])
        if same_box and MODE_NAMES[PROFILE_MODES[m]] in same_box:
            sb = same_box[MODE_NAMES[PROFILE_MODES[m]]]
            entry["same_box_bench"] = {"kernel_ms_avg": sb["kernel_ms_avg"],
                                       "tflops": round(flops / (sb["kernel_ms_avg"] / 1e3) / 1e12, 1),
                                       "frac_of_peak": round(flops / (sb["kernel_ms_avg"] / 1e3) / 1e12
                                                             / PEAK_BF16_TFLOPS, 4)}
    data = {
        "kernel": "attn_numa::attn_fwd_kernel",
        "kernel_hash": kernel_hash(),
        "workload": workload, "description": describe(workload),
        "algorithmic_flops": flops, "unique_bytes": unique,
        "calibration": {"copy_bytes": 1 << 30, "scale": cal},
        "modes": modes,
        "commands": _recorded_commands(directory, workload),
    }
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"counters_attn_fwd_{workload}.json"), "w") as f:
        json.dump(data, f, indent=1)
    lines = [f"# attn_fwd_kernel, {describe(workload)}", "",
             f"Kernel source hash {data['kernel_hash']} (sha256 of the kernel sources, first 16 hex).",
             f"Algorithmic work {flops / 1e12:.1f} TFLOP per call; unique Q+K+V+O+lse footprint "
             f"{unique / 2**30:.2f} GiB.", "",
             "## rocprofv3 --kernel-trace --stats", "",
             "| kernel | calls | average ms | min ms | max ms |", "|---|---|---|---|---|"]
    for r in stats:
        if "attn_fwd_kernel" in r["Name"]:
            lines.append(f"| {r['Name'].split('(')[0]} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.2f} | "
                         f"{float(r['MinNs']) / 1e6:.2f} | {float(r['MaxNs']) / 1e6:.2f} |")
    lines += ["", f"(the trace mixes the {len(PROFILE_MODES)} mapping modes, 3 calls each: see the per-mode table)", "",
              "## Counters per mapping mode (one dispatch each)", "",
              "| mode | L2 hit % | HBM read GB | HBM write GB | read / unique | MFMA busy % | clock GHz | kernel ms | TFLOP/s |",
              "|---|---|---|---|---|---|---|---|---|"]
    for name, mm in modes.items():
        lines.append(f"| {name} | {mm['l2_hit_pct']} | {mm['fetch_bytes'] / 1e9:.1f} | {mm['write_bytes'] / 1e9:.2f} | "
                     f"{mm['fetch_over_unique']} | {mm['mfma_busy_pct']} | {mm['clock_ghz']} | "
                     f"{mm['kernel_ms_counter_run']} | {flops / (mm['kernel_ms_counter_run'] / 1e3) / 1e12:.0f} |")
    lines += ["", f"HBM bytes are FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what the same "
              f"counters read for a plain 1 GiB device copy: read x{cal['FETCH_SIZE']:.3f}, "
              f"write x{cal['WRITE_SIZE']:.3f}. They count L2-to-fabric traffic, so reads served by "
              f"the Infinity Cache are included.", "",
              "MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
              "clock = GRBM_GUI_ACTIVE / 8 / kernel duration.", ""]
    if any("same_box_bench" in mm for mm in modes.values()):
        lines += ["## Same-box benchmark (bench.py on the profiled box, before the profiler runs)", "",
                  f"HIP-event mean kernel time; TFLOP/s = {flops / 1e12:.1f} TFLOP / time; fraction of "
                  f"the {PEAK_BF16_TFLOPS:.0f} TFLOP/s bf16 peak.", "",
                  "| mode | kernel ms | TFLOP/s | frac of peak |", "|---|---|---|---|"]
        for name, mm in modes.items():
            if "same_box_bench" in mm:
                sb = mm["same_box_bench"]
                lines.append(f"| {name} | {sb['kernel_ms_avg']:.2f} | {sb['tflops']} | {sb['frac_of_peak']} |")
        lines.append("")
    if any("issue" in mm for mm in modes.values()):
        lines += ["## Where the non-MFMA time goes (SQ counters, one dispatch per mode)", ""] + ISSUE_TABLE_HEAD
        for name, mm in modes.items():
            if "issue" in mm:
                lines.append(_issue_row(name, mm["issue"]))
        lines.append("")
    lines += ["## Commands", ""]
    lines.append("Each pass is its own process, run as `cd /tmp && export TMPDIR=/tmp && <command>` "
                 "with the repository at /root/repo; then "
                 f"`python3 bench.py --workload {workload} --summarize-profile DIR` (DIR: the directory "
                 "the -d paths below share) "
                 "wrote this file.")
    lines.append("")
    for name, cmd in data["commands"].items():
        lines.append(f"- {name}: `{cmd}`")
    with open(os.path.join(PROFILES, f"attn_fwd_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({k: v for k, v in data.items() if k != "commands"}, indent=1))


def summarize_bwd_profile(directory: str, workload: str):
    """The backward pass's rocprofv3 CSVs (profile_commands(..., "bwd")) into
    profiles/attn_bwd_<workload>.md and counters_attn_bwd_<workload>.json:
    per mapping mode and per gradient kernel, L2 hit rate, HBM bytes, MFMA
    busy share, clock and duration."""
    import csv
    import glob
    B, H_Q, H_KV, N, d, causal = WORKLOADS[workload]
    flops = pass_flops("bwd", B, H_Q, N, d, causal)

    def one(pass_name, kernel):
        files = glob.glob(os.path.join(directory, pass_name, "*_counter_collection.csv"))
        if not files:
            raise SystemExit(f"missing {pass_name} counters under {directory}")
        return _read_counters(files[0], kernel)

    cal = {}
    for name, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        v, _ = one("copy_" + name, "copyBuffer")
        cal[ctr] = (1 << 30) / (v[-1][ctr] * 1024.0)
    _, pre_durs = one("l2", "attn_bwd_pre_kernel")
    q_bytes, kv_bytes = B * H_Q * N * d * 2, B * H_KV * N * d * 2
    unique = {"attn_bwd_dkv_kernel": 2 * q_bytes + 4 * kv_bytes + 8 * B * H_Q * N,
              "attn_bwd_dq_kernel": 3 * q_bytes + 2 * kv_bytes + 8 * B * H_Q * N}
    per_kernel = {}
    for kern in PASS_KERNELS["bwd"]:
        l2, durs = one("l2", kern)
        fe, _ = one("fetch", kern)
        wr, _ = one("write", kern)
        mf, mdur = one("mfma", kern)
        if not (len(l2) == len(fe) == len(wr) == len(mf) == len(PROFILE_MODES)):
            raise SystemExit(f"expected one {kern} dispatch per mapping mode in every pass")
        iss = None
        if (glob.glob(os.path.join(directory, "issue", "*_counter_collection.csv"))
                and glob.glob(os.path.join(directory, "waits", "*_counter_collection.csv"))):
            ia, _ = one("issue", kern)
            ib, _ = one("waits", kern)
            if len(ia) == len(ib) == len(PROFILE_MODES):
                iss = [dict(a, **b) for a, b in zip(ia, ib)]
        rows = {}
        for m in range(len(PROFILE_MODES)):
            hit, miss = l2[m]["TCC_HIT_sum"], l2[m]["TCC_MISS_sum"]
            fetch_b = fe[m]["FETCH_SIZE"] * 1024.0 * cal["FETCH_SIZE"]
            write_b = wr[m]["WRITE_SIZE"] * 1024.0 * cal["WRITE_SIZE"]
            gui = mf[m]["GRBM_GUI_ACTIVE"]
            rows[MODE_NAMES[PROFILE_MODES[m]]] = {
                "l2_hit_pct": round(100.0 * hit / (hit + miss), 2),
                "fetch_bytes": fetch_b, "write_bytes": write_b,
                "fetch_over_unique": round(fetch_b / unique[kern], 2),
                "mfma_busy_pct": round(100.0 * mf[m]["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui / 8.0 * 1024), 2),
                "clock_ghz": round(gui / 8.0 / mdur[m] / 1e9, 3),
                "kernel_ms_counter_run": round(durs[m] * 1e3, 3),
            }
            if iss is not None:
                rows[MODE_NAMES[PROFILE_MODES[m]]]["issue"] = _issue_summary(iss[m])
        per_kernel[kern] = rows
    modes = {}
    for m, mode in enumerate(PROFILE_MODES):
        name = MODE_NAMES[mode]
        total = pre_durs[m] * 1e3 + sum(per_kernel[k][name]["kernel_ms_counter_run"] for k in per_kernel)
        modes[name] = {"ms": round(total, 3), "tflops": round(flops / (total / 1e3) / 1e12, 1),
                       "pre_ms": round(pre_durs[m] * 1e3, 3)}
    same_box = _same_box_bench(directory)
    if same_box:
        for name in modes:
            if name in same_box:
                sb = same_box[name]
                modes[name]["same_box_bench"] = {
                    "kernel_ms_avg": sb["kernel_ms_avg"],
                    "tflops": round(flops / (sb["kernel_ms_avg"] / 1e3) / 1e12, 1),
                    "frac_of_peak": round(flops / (sb["kernel_ms_avg"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    trace = glob.glob(os.path.join(directory, "trace", "*_kernel_stats.csv"))
    stats = []
    if trace:
        with open(trace[0]) as f:
            stats = [r for r in csv.DictReader(f) if "attn_bwd" in r["Name"]]
    data = {
        "kernels": ["attn_numa::attn_bwd_pre_kernel"] + [f"attn_numa::{k}" for k in PASS_KERNELS["bwd"]],
        "kernel_hash": kernel_hash("bwd"),
        "workload": workload, "description": describe(workload).replace(" fwd ", " bwd "),
        "algorithmic_flops": flops, "unique_bytes": unique,
        "calibration": {"copy_bytes": 1 << 30, "scale": cal},
        "modes": modes, "per_kernel": per_kernel,
        "commands": _recorded_commands(directory, workload, "bwd"),
    }
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"counters_attn_bwd_{workload}.json"), "w") as f:
        json.dump(data, f, indent=1)
    lines = [f"# attn_bwd (attn_bwd_pre, attn_bwd_dkv, attn_bwd_dq), {data['description']}", "",
             f"Kernel source hash {data['kernel_hash']} (sha256 of the backward's sources, first 16 hex).",
             f"Algorithmic work {flops / 1e12:.1f} TFLOP per call (2.5x the forward's).", "",
             "## rocprofv3 --kernel-trace --stats", "",
             "| kernel | calls | average ms | min ms | max ms |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name'].split('(')[0]} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                     f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} |")
    lines += ["", f"(the trace mixes the {len(PROFILE_MODES)} mapping modes, 3 calls each: see the per-mode tables)",
              "", "## Whole backward per mapping mode (counter runs: pre + dK/dV + dQ durations)", "",
              "| mode | ms | TFLOP/s | % of bf16 peak |", "|---|---|---|---|"]
    for name, mm in modes.items():
        lines.append(f"| {name} | {mm['ms']} | {mm['tflops']} | {100 * mm['tflops'] / PEAK_BF16_TFLOPS:.1f} |")
    if any("same_box_bench" in mm for mm in modes.values()):
        lines += ["", "## Same-box benchmark (bench.py on the profiled box, before the profiler runs)", "",
                  f"HIP-event mean time of one attn_bwd call (its three kernels); TFLOP/s = "
                  f"{flops / 1e12:.1f} TFLOP / time; fraction of the {PEAK_BF16_TFLOPS:.0f} TFLOP/s bf16 peak.", "",
                  "| mode | ms | TFLOP/s | frac of peak |", "|---|---|---|---|"]
        for name, mm in modes.items():
            if "same_box_bench" in mm:
                sb = mm["same_box_bench"]
                lines.append(f"| {name} | {sb['kernel_ms_avg']:.2f} | {sb['tflops']} | {sb['frac_of_peak']} |")
    for kern, rows in per_kernel.items():
        if any("issue" in mm for mm in rows.values()):
            lines += ["", f"## {kern}, where the non-MFMA time goes (SQ counters, one dispatch per mode)", ""]
            lines += ISSUE_TABLE_HEAD
            for name, mm in rows.items():
                if "issue" in mm:
                    lines.append(_issue_row(name, mm["issue"]))
    for kern, rows in per_kernel.items():
        lines += ["", f"## {kern}, counters per mapping mode (one dispatch each)", "",
                  "| mode | L2 hit % | HBM read GB | HBM write GB | read / unique | MFMA busy % | clock GHz | ms |",
                  "|---|---|---|---|---|---|---|---|"]
        for name, mm in rows.items():
            lines.append(f"| {name} | {mm['l2_hit_pct']} | {mm['fetch_bytes'] / 1e9:.1f} | "
                         f"{mm['write_bytes'] / 1e9:.2f} | {mm['fetch_over_unique']} | {mm['mfma_busy_pct']} | "
                         f"{mm['clock_ghz']} | {mm['kernel_ms_counter_run']} |")
    lines += ["", f"HBM bytes: FETCH_SIZE and WRITE_SIZE scaled by a plain 1 GiB copy's counts "
              f"(read x{cal['FETCH_SIZE']:.3f}, write x{cal['WRITE_SIZE']:.3f}). Unique bytes: dK/dV "
              "kernel Q, dO, K, V, dK, dV and the two fp32 row statistics; dQ kernel Q, dO, K, V, dQ and "
              "the statistics.", "", "## Commands", "",
              "Each pass is its own process, run as `cd /tmp && export TMPDIR=/tmp && <command>` "
              "with the repository at /root/repo; then "
              f"`python3 bench.py --workload {workload} --pass bwd --summarize-profile DIR` wrote this file.", ""]
    for name, cmd in data["commands"].items():
        lines.append(f"- {name}: `{cmd}`")
    with open(os.path.join(PROFILES, f"attn_bwd_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({k: v for k, v in data.items() if k != "commands"}, indent=1))


def run_bwd(args, attn, inputs):
    """--pass bwd: times attn_bwd per mapping mode; prints one JSON line."""
    import torch
    B, H_Q, H_KV, N, d, causal = WORKLOADS[args.workload]
    modes = [int(m) for m in args.modes.split(",") if m.strip() != ""]
    headline = _headline_mode(modes, causal)
    flops = pass_flops("bwd", B, H_Q, N, d, causal)
    log(f"workload {describe(args.workload)} backward: {flops / 1e12:.1f} TFLOP per call")
    q, k, v = inputs.make_qkv(B, H_Q, H_KV, N, d, seed=1000, device="cuda")
    dout = inputs.normal_bf16((B, H_Q, N, d), 1003, "cuda")
    o, lse = attn.attn_fwd(q, k, v, causal=causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((B, H_Q, 2, N), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    results = {}
    for mode in modes:
        def call(stream, mode=mode):
            attn.attn_bwd(q, k, v, o, dout, lse, causal=causal, mapping=mode, dq=dq, dk=dk,
                          dv=dv, ws=ws, stream=stream)
        r = time_calls(call, args.steps, args.warmup, flops)
        results[mode] = r
        log(f"  {MODE_NAMES[mode]:34s} {r['kernel_tflops']:8.1f} TFLOP/s "
            f"({r['pct_peak']:.1f}% of peak, {r['kernel_ms_avg']:.2f} ms)")
    counters = stored_counters(args.workload, kernel_hash("bwd"), "bwd")
    head = results[headline]
    modes_out = {}
    for mode, r in results.items():
        entry = {k2: round(v2, 4) for k2, v2 in r.items()}
        if counters:
            for kern, rows in counters["per_kernel"].items():
                if MODE_NAMES[mode] in rows:
                    entry[kern.replace("attn_bwd_", "").replace("_kernel", "") + "_l2_hit_pct"] = \
                        rows[MODE_NAMES[mode]]["l2_hit_pct"]
        modes_out[MODE_NAMES[mode]] = entry
    traffic = None
    if counters:
        traffic = sum(rows[MODE_NAMES[headline]]["fetch_bytes"] + rows[MODE_NAMES[headline]]["write_bytes"]
                      for rows in counters["per_kernel"].values() if MODE_NAMES[headline] in rows)
    out = {
        "metric": BWD_METRIC,
        "value": round(head["kernel_tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: bf16 N(0,1) Q/K/V/dO from fixed seeds",
        "config": {"workload": describe(args.workload).replace(" fwd ", " bwd "),
                   "B": B, "H_Q": H_Q, "H_KV": H_KV, "N": N, "d": d, "causal": causal,
                   "mapping": MODE_NAMES[headline], "parallelism": "single GPU"},
        "pct_peak": round(head["pct_peak"], 2),
        "modes": modes_out,
        "roofline": {"bound": "mfma", "achieved": round(head["kernel_tflops"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(head["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "scope": "one attn_bwd call (its three kernels, one stream)",
                     "executed": _bwd_executed(head["kernel_tflops"], d)},
        "kernel_hash": kernel_hash("bwd"),
        "counters_source": counters_source(args.workload, kernel_hash("bwd"), "bwd", counters),
    }
    if 0 in results and headline != 0:
        out["speedup_vs_naive_block_first"] = round(
            results[0]["kernel_ms_avg"] / head["kernel_ms_avg"], 4)
    emit(out, args)


def _bwd_executed(credited_tflops: float, d: int) -> dict:
    """The MFMA work attn_bwd executes: per (query, visible key) 8 D_PAD FLOP
    in the dK/dV kernel (S, dP, dV, dK) and 6 D_PAD in the dQ kernel (S and
    dP again, dQ), against the 10 d credited (2.5x the forward's 4 d)."""
    d_pad = 64 if d <= 64 else 128
    ex = credited_tflops * 14.0 * d_pad / (10.0 * d)
    return {"tflops": round(ex, 2), "frac": round(ex / PEAK_BF16_TFLOPS, 4),
            "flop_per_pair": f"14 x {d_pad} executed against 10 x {d} credited"}


def gemm_describe(name) -> str:
    L, M, N, K = GEMM_WORKLOADS[name]
    return f"GEMM C = A B^T, L={L} M={M} N={N} K={K} bf16"


def run_gemm(args, attn, inputs):
    """--pass gemm: times cac_gemm per tile map (and torch.mm on the same
    operands as context); prints one JSON line."""
    import torch
    L, M, N, K = GEMM_WORKLOADS[args.workload]
    modes = [int(m) for m in args.modes.split(",") if m.strip() != ""]
    flops = 2.0 * L * M * N * K
    log(f"workload {gemm_describe(args.workload)}: {flops / 1e12:.2f} TFLOP per call")
    a = inputs.normal_bf16((L, M, K), 1000, "cuda")
    b = inputs.normal_bf16((L, N, K), 1001, "cuda")
    c = torch.empty((L, M, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    results = {}
    for mode in modes:
        log(f"  timing cac_gemm mapping {mode} ({GEMM_MODE_NAMES[mode]})")

        def call(stream, mode=mode):
            attn.cac_gemm(a, b, mapping=mode, c=c, stream=stream)
        r = time_calls(call, args.steps, args.warmup, flops)
        results[mode] = r
        log(f"  {GEMM_MODE_NAMES[mode]:20s} {r['kernel_tflops']:8.1f} TFLOP/s "
            f"({r['pct_peak']:.1f}% of peak, {r['kernel_ms_avg']:.3f} ms)")
    # Context: the vendor library on the same operands, one plain 2-D GEMM per
    # batch (torch.mm of A[l] and the transposed view of B[l]); batched bf16
    # products with a transposed right operand are avoided on purpose.
    log("  timing torch.mm per batch (hipBLASLt)")

    def library(stream):
        for l in range(L):
            torch.mm(a[l], b[l].t(), out=c[l])
    ref = time_calls(library, args.steps, args.warmup, flops)
    log(f"  torch.mm (hipBLASLt)      {ref['kernel_tflops']:8.1f} TFLOP/s")
    headline = 3 if 3 in modes else modes[-1]
    counters = stored_counters(args.workload, kernel_hash("gemm"), "gemm")
    head = results[headline]
    modes_out = {}
    for mode, r in results.items():
        entry = {k2: round(v2, 4) for k2, v2 in r.items()}
        if counters and GEMM_MODE_NAMES[mode] in counters["modes"]:
            entry["l2_hit_pct"] = counters["modes"][GEMM_MODE_NAMES[mode]]["l2_hit_pct"]
        modes_out[GEMM_MODE_NAMES[mode]] = entry
    traffic = None
    if counters and GEMM_MODE_NAMES[headline] in counters["modes"]:
        cm = counters["modes"][GEMM_MODE_NAMES[headline]]
        traffic = cm["fetch_bytes"] + cm["write_bytes"]
    out = {
        "metric": GEMM_METRIC,
        "value": round(head["kernel_tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: bf16 N(0,1) A/B from fixed seeds",
        "config": {"workload": gemm_describe(args.workload), "L": L, "M": M, "N": N, "K": K,
                   "mapping": GEMM_MODE_NAMES[headline], "cluster": "4 x 8 tiles of 256 x 256",
                   "parallelism": "single GPU"},
        "pct_peak": round(head["pct_peak"], 2),
        "modes": modes_out,
        "torch_mm_tflops": round(ref["kernel_tflops"], 2),
        "roofline": {"bound": "mfma", "achieved": round(head["kernel_tflops"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(head["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "kernel_hash": kernel_hash("gemm"),
        "counters_source": counters_source(args.workload, kernel_hash("gemm"), "gemm", counters),
    }
    if 0 in results and headline != 0:
        out["speedup_vs_naive_row_major"] = round(results[0]["kernel_ms_avg"] / head["kernel_ms_avg"], 4)
    emit(out, args)


def summarize_gemm_profile(directory: str, workload: str):
    """rocprofv3 CSVs of profile_commands(..., "gemm") into
    profiles/cac_gemm_<workload>.md and counters_gemm_<workload>.json."""
    import csv
    import glob
    L, M, N, K = GEMM_WORKLOADS[workload]
    flops = 2.0 * L * M * N * K

    def one(pass_name, kernel):
        files = glob.glob(os.path.join(directory, pass_name, "*_counter_collection.csv"))
        if not files:
            raise SystemExit(f"missing {pass_name} counters under {directory}")
        return _read_counters(files[0], kernel)

    cal = {}
    for name, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        v, _ = one("copy_" + name, "copyBuffer")
        cal[ctr] = (1 << 30) / (v[-1][ctr] * 1024.0)
    l2, durs = one("l2", "cac_gemm_kernel")
    fe, _ = one("fetch", "cac_gemm_kernel")
    wr, _ = one("write", "cac_gemm_kernel")
    mf, mdur = one("mfma", "cac_gemm_kernel")
    if not (len(l2) == len(fe) == len(wr) == len(mf) == 4):
        raise SystemExit("expected one cac_gemm dispatch per tile map in every pass")
    iss = None
    if (glob.glob(os.path.join(directory, "issue", "*_counter_collection.csv"))
            and glob.glob(os.path.join(directory, "waits", "*_counter_collection.csv"))):
        ia, _ = one("issue", "cac_gemm_kernel")
        ib, _ = one("waits", "cac_gemm_kernel")
        if len(ia) == len(ib) == 4:
            iss = [dict(x, **y) for x, y in zip(ia, ib)]
    unique = 2 * L * (M * K + N * K + M * N)
    modes = {}
    for m in range(4):
        hit, miss = l2[m]["TCC_HIT_sum"], l2[m]["TCC_MISS_sum"]
        fetch_b = fe[m]["FETCH_SIZE"] * 1024.0 * cal["FETCH_SIZE"]
        write_b = wr[m]["WRITE_SIZE"] * 1024.0 * cal["WRITE_SIZE"]
        gui = mf[m]["GRBM_GUI_ACTIVE"]
        modes[GEMM_MODE_NAMES[m]] = {
            "l2_hit_pct": round(100.0 * hit / (hit + miss), 2),
            "fetch_bytes": fetch_b, "write_bytes": write_b,
            "fetch_over_unique": round(fetch_b / unique, 2),
            "mfma_busy_pct": round(100.0 * mf[m]["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui / 8.0 * 1024), 2),
            "clock_ghz": round(gui / 8.0 / mdur[m] / 1e9, 3),
            "kernel_ms_counter_run": round(durs[m] * 1e3, 3),
            "tflops_counter_run": round(flops / durs[m] / 1e12, 1),
            # per GHz of the clock the dispatch ran at: tile maps compared
            # without the power-limit clock of each run
            "tflops_per_ghz": round(flops / durs[m] / 1e12 / (gui / 8.0 / mdur[m] / 1e9), 1),
        }
        if iss is not None:
            modes[GEMM_MODE_NAMES[m]]["issue"] = _issue_summary(iss[m])
    same_box = _same_box_bench(directory)
    if same_box:
        for name, mm in modes.items():
            if name in same_box:
                mm["same_box_bench_tflops"] = round(same_box[name]["kernel_tflops"], 1)
    trace = glob.glob(os.path.join(directory, "trace", "*_kernel_stats.csv"))
    stats = []
    if trace:
        with open(trace[0]) as f:
            stats = [r for r in csv.DictReader(f)]
    data = {"kernel": "attn_numa::cac_gemm_kernel", "kernel_hash": kernel_hash("gemm"),
            "workload": workload, "description": gemm_describe(workload),
            "algorithmic_flops": flops, "unique_bytes": unique,
            "calibration": {"copy_bytes": 1 << 30, "scale": cal}, "modes": modes,
            "commands": _recorded_commands(directory, workload, "gemm")}
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"counters_gemm_{workload}.json"), "w") as f:
        json.dump(data, f, indent=1)
    lines = [f"# cac_gemm_kernel, {gemm_describe(workload)}", "",
             f"Kernel source hash {data['kernel_hash']} (sha256 of the GEMM's sources, first 16 hex).",
             f"Algorithmic work {flops / 1e12:.2f} TFLOP per call; unique A+B+C "
             f"{unique / 2**30:.2f} GiB.", "", "## rocprofv3 --kernel-trace --stats", "",
             "| kernel | calls | average ms | min ms | max ms |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name'].split('(')[0]} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                     f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} |")
    lines += ["", "(the trace mixes the 4 tile maps, 3 calls each, and torch.mm's kernels)", "",
              "## Counters per tile map (one dispatch each)", "",
              "| tile map | L2 hit % | HBM read GB | HBM write GB | read / unique | MFMA busy % | clock GHz | ms | TFLOP/s | TFLOP/s per GHz | same-box bench TFLOP/s |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, mm in modes.items():
        lines.append(f"| {name} | {mm['l2_hit_pct']} | {mm['fetch_bytes'] / 1e9:.2f} | "
                     f"{mm['write_bytes'] / 1e9:.2f} | {mm['fetch_over_unique']} | {mm['mfma_busy_pct']} | "
                     f"{mm['clock_ghz']} | {mm['kernel_ms_counter_run']} | {mm['tflops_counter_run']} | "
                     f"{mm['tflops_per_ghz']} | {mm.get('same_box_bench_tflops', '')} |")
    lines += ["", f"HBM bytes: FETCH_SIZE and WRITE_SIZE scaled by a plain 1 GiB copy's counts "
              f"(read x{cal['FETCH_SIZE']:.3f}, write x{cal['WRITE_SIZE']:.3f}).", ""]
    if any("issue" in mm for mm in modes.values()):
        lines += ["## Where the non-MFMA time goes (SQ counters, one dispatch per tile map)", ""] + ISSUE_TABLE_HEAD
        for name, mm in modes.items():
            if "issue" in mm:
                lines.append(_issue_row(name, mm["issue"]))
        lines.append("")
    lines += ["## Commands", "",
              "Each pass is its own process, run as `cd /tmp && export TMPDIR=/tmp && <command>` "
              "with the repository at /root/repo; then "
              f"`python3 bench.py --workload {workload} --pass gemm --summarize-profile DIR` wrote this file.", ""]
    for name, cmd in data["commands"].items():
        lines.append(f"- {name}: `{cmd}`")
    with open(os.path.join(PROFILES, f"cac_gemm_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({k: v for k, v in data.items() if k != "commands"}, indent=1))


def decode_describe(name) -> str:
    B, H_Q, H_KV, N_q, N_kv, d, causal, S = SPLIT_WORKLOADS[name]
    return (f"decode B={B} H_Q={H_Q} H_KV={H_KV} N_q={N_q} N_kv={N_kv} d={d} "
            f"{'causal' if causal else 'non-causal'}, {S} splits")


def run_decode(args, attn, inputs):
    """--pass decode: attn_fwd_split (split-KV + merge) per mapping on a
    decode workload; HBM-bound, so GB/s against the HBM peak.  One JSON line."""
    import torch
    B, H_Q, H_KV, N_q, N_kv, d, causal, S = SPLIT_WORKLOADS[args.workload]
    modes = [int(m) for m in args.modes.split(",") if m.strip() != ""]
    nbytes = split_bytes(B, H_Q, H_KV, N_q, N_kv, d, S)
    log(f"workload {decode_describe(args.workload)}: {nbytes / 1e9:.2f} GB per call")
    q = inputs.normal_bf16((B, H_Q, N_q, d), 1000, "cuda")
    k = inputs.normal_bf16((B, H_KV, N_kv, d), 1001, "cuda")
    v = inputs.normal_bf16((B, H_KV, N_kv, d), 1002, "cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H_Q, N_q), dtype=torch.float32, device="cuda")
    o_ws = torch.empty((S, B, H_Q, N_q, d), dtype=torch.float32, device="cuda")
    lse_ws = torch.empty((S, B, H_Q, N_q), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    results = {}
    for mode in modes:
        def call(stream, mode=mode):
            attn.attn_fwd_split(q, k, v, causal=causal, num_splits=S, mapping=mode, o=o, lse=lse,
                                o_ws=o_ws, lse_ws=lse_ws, stream=stream)
        r = time_calls(call, max(args.steps, 10), args.warmup, 1.0)
        r["gbs"] = nbytes / (r["kernel_ms_avg"] / 1e3) / 1e9
        results[mode] = r
        log(f"  {MODE_NAMES[mode]:22s} {r['gbs']:8.0f} GB/s ({100 * r['gbs'] / HBM_PEAK_GBS:.1f}% of "
            f"the HBM peak, {r['kernel_ms_avg']:.3f} ms)")
    headline = 3 if 3 in modes else modes[-1]
    counters = stored_counters(args.workload, kernel_hash("decode"), "decode")
    head = results[headline]
    modes_out = {}
    for mode, r in results.items():
        entry = {"gbs": round(r["gbs"], 1), "kernel_ms_avg": round(r["kernel_ms_avg"], 4),
                 "ms_per_step": round(r["ms_per_step"], 4)}
        if counters and MODE_NAMES[mode] in counters["modes"]:
            entry["l2_hit_pct"] = counters["modes"][MODE_NAMES[mode]]["l2_hit_pct"]
        modes_out[MODE_NAMES[mode]] = entry
    traffic = None
    if counters and MODE_NAMES[headline] in counters["modes"]:
        cm = counters["modes"][MODE_NAMES[headline]]
        traffic = cm["fetch_bytes"] + cm["write_bytes"]
    out = {
        "metric": DECODE_METRIC,
        "value": round(head["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": max(args.steps, 10), "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: bf16 N(0,1) Q/K/V from fixed seeds",
        "config": {"workload": decode_describe(args.workload), "B": B, "H_Q": H_Q, "H_KV": H_KV,
                   "N_q": N_q, "N_kv": N_kv, "d": d, "causal": causal, "splits": S,
                   "mapping": MODE_NAMES[headline], "parallelism": "single GPU"},
        "modes": modes_out,
        "roofline": {"bound": "hbm", "achieved": round(head["gbs"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(head["gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "scope": "one attn_fwd_split call (decode kernel + merge kernel, one stream)"},
        "algorithmic_bytes": nbytes,
        "kernel_hash": kernel_hash("decode"),
        "counters_source": counters_source(args.workload, kernel_hash("decode"), "decode", counters),
    }
    emit(out, args)


def summarize_decode_profile(directory: str, workload: str):
    """rocprofv3 CSVs of profile_commands(..., "decode") into
    profiles/attn_decode_<workload>.md and counters_decode_<workload>.json:
    per mapping, the decode and merge kernels' L2 hit, HBM bytes, durations."""
    import csv
    import glob
    B, H_Q, H_KV, N_q, N_kv, d, causal, S = SPLIT_WORKLOADS[workload]
    nbytes = split_bytes(B, H_Q, H_KV, N_q, N_kv, d, S)

    def one(pass_name, kernel):
        files = glob.glob(os.path.join(directory, pass_name, "*_counter_collection.csv"))
        if not files:
            raise SystemExit(f"missing {pass_name} counters under {directory}")
        return _read_counters(files[0], kernel)

    cal = {}
    for name, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        v, _ = one("copy_" + name, "copyBuffer")
        cal[ctr] = (1 << 30) / (v[-1][ctr] * 1024.0)
    per = {}
    for kern in PASS_KERNELS["decode"]:
        l2, durs = one("l2", kern)
        fe, _ = one("fetch", kern)
        wr, _ = one("write", kern)
        # the decode pass times at least 10 calls per mapping, in mapping
        # order: keep the last dispatch of each
        if not (len(l2) == len(fe) == len(wr) and len(l2) % 4 == 0 and l2):
            raise SystemExit(f"expected the same number of {kern} dispatches per mapping in every pass")
        k = len(l2) // 4
        pick = [(m + 1) * k - 1 for m in range(4)]
        per[kern] = ([l2[i] for i in pick], [durs[i] for i in pick],
                     [fe[i] for i in pick], [wr[i] for i in pick])
    modes = {}
    for m in range(4):
        hit = sum(per[k][0][m]["TCC_HIT_sum"] for k in per)
        miss = sum(per[k][0][m]["TCC_MISS_sum"] for k in per)
        fetch_b = sum(per[k][2][m]["FETCH_SIZE"] for k in per) * 1024.0 * cal["FETCH_SIZE"]
        write_b = sum(per[k][3][m]["WRITE_SIZE"] for k in per) * 1024.0 * cal["WRITE_SIZE"]
        ms = sum(per[k][1][m] for k in per) * 1e3
        modes[MODE_NAMES[m]] = {
            "l2_hit_pct": round(100.0 * hit / (hit + miss), 2),
            "fetch_bytes": fetch_b, "write_bytes": write_b,
            "hbm_over_algorithmic": round((fetch_b + write_b) / nbytes, 3),
            "decode_ms": round(per["attn_decode_kernel"][1][m] * 1e3, 4),
            "merge_ms": round(per["attn_merge_kernel"][1][m] * 1e3, 4),
            "gbs_counter_run": round(nbytes / (ms / 1e3) / 1e9, 1),
        }
    data = {"kernels": ["attn_numa::attn_decode_kernel", "attn_numa::attn_merge_kernel"],
            "kernel_hash": kernel_hash("decode"), "workload": workload,
            "description": decode_describe(workload), "algorithmic_bytes": nbytes,
            "calibration": {"copy_bytes": 1 << 30, "scale": cal}, "modes": modes,
            "commands": _recorded_commands(directory, workload, "decode")}
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"counters_decode_{workload}.json"), "w") as f:
        json.dump(data, f, indent=1)
    trace = glob.glob(os.path.join(directory, "trace", "*_kernel_stats.csv"))
    stats = []
    if trace:
        with open(trace[0]) as f:
            stats = [r for r in csv.DictReader(f) if "attn_" in r["Name"]]
    lines = [f"# attn_decode_kernel + attn_merge_kernel, {decode_describe(workload)}", "",
             f"Kernel source hash {data['kernel_hash']} (sha256 of the decode path's sources, first 16 hex).",
             f"Algorithmic bytes {nbytes / 1e9:.2f} GB per call (Q, K, V, O, lse and the fp32 partials "
             "written and read back).", "", "## rocprofv3 --kernel-trace --stats", "",
             "| kernel | calls | average ms | min ms | max ms |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name'].split('(')[0]} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                     f"{float(r['MinNs']) / 1e6:.4f} | {float(r['MaxNs']) / 1e6:.4f} |")
    lines += ["", "(the trace mixes the 4 mappings: warmup and timed calls of each, in order)", "",
              "## Counters per mapping (decode + merge kernels, one call each)", "",
              "| mapping | L2 hit % | HBM read GB | HBM write GB | HBM / algorithmic | decode ms | merge ms | GB/s |",
              "|---|---|---|---|---|---|---|---|"]
    for name, mm in modes.items():
        lines.append(f"| {name} | {mm['l2_hit_pct']} | {mm['fetch_bytes'] / 1e9:.2f} | "
                     f"{mm['write_bytes'] / 1e9:.3f} | {mm['hbm_over_algorithmic']} | {mm['decode_ms']} | "
                     f"{mm['merge_ms']} | {mm['gbs_counter_run']} |")
    lines += ["", f"HBM bytes: FETCH_SIZE and WRITE_SIZE scaled by a plain 1 GiB copy's counts "
              f"(read x{cal['FETCH_SIZE']:.3f}, write x{cal['WRITE_SIZE']:.3f}).", "", "## Commands", "",
              "Each pass is its own process, run as `cd /tmp && export TMPDIR=/tmp && <command>` "
              "with the repository at /root/repo; then "
              f"`python3 bench.py --workload {workload} --pass decode --summarize-profile DIR` wrote this file.", ""]
    for name, cmd in data["commands"].items():
        lines.append(f"- {name}: `{cmd}`")
    with open(os.path.join(PROFILES, f"attn_decode_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({k: v for k, v in data.items() if k != "commands"}, indent=1))


def run_sweep(out_path: str):
    """Times every SWEEP configuration under the four mapping modes (2 warmup
    calls, then the median of 5 calls, 10 when N <= 32K) and writes a table."""
    import torch
    import chiplet_numa_aware_amd as attn
    from chiplet_numa_aware_amd import inputs
    rows = []
    for name in SWEEP:
        B, H_Q, H_KV, N, d, causal = WORKLOADS[name]
        flops = attn_flops(B, H_Q, N, d, causal)
        q, k, v = inputs.make_qkv(B, H_Q, H_KV, N, d, seed=1000, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty(B, H_Q, N, device="cuda", dtype=torch.float32)
        steps = 10 if N <= 32768 else 5
        res = {}
        for mode in SWEEP_MODES:
            r = time_mode(attn, q, k, v, o, lse, causal, mode, steps, 2, flops)
            res[MODE_NAMES[mode]] = flops / (r["kernel_ms_median"] / 1e3) / 1e12
            log(f"  {name:24s} {MODE_NAMES[mode]:22s} {r['kernel_ms_median']:9.3f} ms "
                f"{res[MODE_NAMES[mode]]:7.1f} TFLOP/s")
        rows.append((name, flops, res))
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    lines = ["# attn_fwd_kernel: TFLOP/s per configuration and mapping mode", "",
             f"Kernel source hash {kernel_hash()}. Median of the HIP-event kernel times of 5 "
             "calls (10 when N <= 32K) after 2 warmup calls, seed 1000; "
             f"TFLOP/s = algorithmic FLOP / median; % of the {PEAK_BF16_TFLOPS:.0f} TFLOP/s "
             "bf16 peak in parentheses for swizzled head-first.", "",
             "SHF+LF is swizzled head-first with the longest-first row-block order (mode 7); "
             "SHF+LF+BS adds the balanced split (mode 15, the binding's default under a causal "
             "mask; it differs from mode 7 only where the XCD count does not divide the ACC count).", "",
             "| configuration | TFLOP | NBF | NHF | SBF | SHF | SHF / NBF | SHF+LF | SHF+LF+BS |",
             "|---|---|---|---|---|---|---|---|---|"]
    for name, flops, res in rows:
        t = [res[MODE_NAMES[m]] for m in SWEEP_MODES]
        lines.append(f"| {describe(name)} | {flops / 1e12:.2f} | {t[0]:.0f} | {t[1]:.0f} | {t[2]:.0f} | "
                     f"{t[3]:.0f} ({100 * t[3] / PEAK_BF16_TFLOPS:.1f}%) | {t[3] / t[0]:.2f} | "
                     f"{t[4]:.0f} ({100 * t[4] / PEAK_BF16_TFLOPS:.1f}%) | "
                     f"{t[5]:.0f} ({100 * t[5] / PEAK_BF16_TFLOPS:.1f}%) |")
    split_rows = []
    for name, (B, H_Q, H_KV, N_q, N_kv, d, causal, S) in SPLIT_WORKLOADS.items():
        q = inputs.normal_bf16((B, H_Q, N_q, d), 1000, "cuda")
        k = inputs.normal_bf16((B, H_KV, N_kv, d), 1001, "cuda")
        v = inputs.normal_bf16((B, H_KV, N_kv, d), 1002, "cuda")
        o = torch.empty_like(q)
        lse = torch.empty(B, H_Q, N_q, device="cuda", dtype=torch.float32)
        o_ws = torch.empty(S, B, H_Q, N_q, d, device="cuda", dtype=torch.float32)
        lse_ws = torch.empty(S, B, H_Q, N_q, device="cuda", dtype=torch.float32)
        flops = 4.0 * B * H_Q * d * N_q * N_kv
        nbytes = split_bytes(B, H_Q, H_KV, N_q, N_kv, d, S)
        stream = torch.cuda.current_stream()
        res = {}
        for mode in (0, 3):
            for _ in range(2):
                attn.attn_fwd_split(q, k, v, causal=causal, num_splits=S, mapping=mode, o=o,
                                    lse=lse, o_ws=o_ws, lse_ws=lse_ws, stream=stream)
            ts = []
            for _ in range(10):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                attn.attn_fwd_split(q, k, v, causal=causal, num_splits=S, mapping=mode, o=o,
                                    lse=lse, o_ws=o_ws, lse_ws=lse_ws, stream=stream)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ms = sorted(ts)[len(ts) // 2]
            res[MODE_NAMES[mode]] = {"ms": ms, "gbs": nbytes / (ms / 1e3) / 1e9,
                                     "tflops": flops / (ms / 1e3) / 1e12}
            log(f"  {name:24s} {MODE_NAMES[mode]:22s} {ms:9.3f} ms "
                f"{res[MODE_NAMES[mode]]['gbs']:8.0f} GB/s")
        split_rows.append((name, (B, H_Q, H_KV, N_q, N_kv, d, causal, S), nbytes, res))
        del q, k, v, o, lse, o_ws, lse_ws
        torch.cuda.empty_cache()
    # Practical reference for a streaming kernel: a plain 4 GiB device copy
    # (bytes read + written over its median time).
    src = torch.empty(1 << 30, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    cts = []
    for i in range(7):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            cts.append(e0.elapsed_time(e1))
    copy_gbs = 2.0 * src.numel() * 4 / (sorted(cts)[len(cts) // 2] / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    lines += ["", "## Split-KV decode (attn_fwd_split + merge, one call)", "",
              f"Decode path source hash {kernel_hash('decode')} (the decode kernel, the merge "
              "kernel, the remap and their launch code).", "",
              "HBM-bound: bytes = Q + K + V + O + lse + the fp32 partials written and read back; "
              f"GB/s against the {HBM_PEAK_GBS:.0f} GB/s HBM peak. Median of 10 calls. A plain 4 GiB "
              f"device copy (torch, read + write) runs at {copy_gbs:.0f} GB/s "
              f"({100 * copy_gbs / HBM_PEAK_GBS:.1f}% of the peak) on the same GPU.", "",
              "| configuration | splits | MB | NBF ms | SHF ms | SHF GB/s (% of peak) |",
              "|---|---|---|---|---|---|"]
    for name, (B, H_Q, H_KV, N_q, N_kv, d, causal, S), nbytes, res in split_rows:
        sh = res["swizzled_head_first"]
        lines.append(f"| decode B={B} H_Q={H_Q} H_KV={H_KV} N_q={N_q} N_kv={N_kv} d={d} "
                     f"{'causal' if causal else ''} | {S} | {nbytes / 1e6:.0f} | "
                     f"{res['naive_block_first']['ms']:.3f} | {sh['ms']:.3f} | "
                     f"{sh['gbs']:.0f} ({100 * sh['gbs'] / HBM_PEAK_GBS:.1f}%) |")
    lines += ["", "Command: `python3 bench.py --sweep OUT.md` (this file is OUT.md)."]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"sweep": {name: res for name, _, res in rows},
                      "split": {name: res for name, _, _, res in split_rows}}))


def _fwd_roofline(d: int, achieved: float, traffic):
    """The forward kernel's binding roofline: the MFMA peak (dense bf16,
    2.5 PFLOP/s) unless the softmax's vector-ALU bound is lower, as at
    d = 64 (2013 credited TFLOP/s against 2500).  At d = 56 the two nearly
    meet (2202 against 2187 for the padded MFMAs).  The other bound is
    reported beside it."""
    mfma = {"bound": "mfma", "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "achieved": round(achieved, 2), "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "peak_credited_at_padded_d": round(mfma_peak_tflops_credited(d), 1)}
    alu_peak = alu_peak_tflops(d)
    alu = {"bound": "alu", "peak": round(alu_peak, 1), "unit": "TFLOP/s (credited)",
           "achieved": round(achieved, 2), "frac": round(achieved / alu_peak, 4),
           "derivation": f"softmax vector work per wave64 of scores: fma 4 + exp2 8 + half a "
                         f"max3 2 + half a bf16 conversion 2"
                         f"{' + row-sum add 4' if d in (64, 128) else ' (the row sum rides the P V MFMA)'}"
                         f" = {softmax_simd_cycles(d)} SIMD cycles; 1024 SIMDs at 2.4 GHz"}
    if alu_peak < mfma_peak_tflops_credited(d):
        primary, other = alu, mfma
    else:
        primary, other = mfma, alu
    primary = dict(primary, traffic=traffic)
    primary["secondary"] = other
    return primary


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None,
                    choices=sorted(WORKLOADS) + sorted(GEMM_WORKLOADS) + sorted(SPLIT_WORKLOADS),
                    help="default: mha_128k (gemm_tall_64k_2k_8k for --pass gemm, "
                         "decode_gqa64x8_b16_128k for --pass decode)")
    ap.add_argument("--modes", default="0,1,2,3",
                    help="mapping modes to time; the headline is the binding's "
                         "default (3, or 15 with a causal mask; else 7 or 3) when "
                         "listed, else the last one")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd", "gemm", "decode"), default="fwd",
                    help="fwd: attn_fwd (default); bwd: attn_bwd on the forward's O, lse; "
                         "gemm: cac_gemm (workloads gemm_*); decode: attn_fwd_split "
                         "(workloads decode_*)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--json-out", metavar="PATH",
                    help="also write the JSON line to PATH")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--sweep", metavar="OUT_MD",
                    help="time every configuration x mapping mode, write a table")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (twice), the "
                         "reference for scaling HBM byte counters")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="summarize rocprofv3 CSV output under DIR (made by the "
                         "commands --print-profile-commands lists) into profiles/")
    ap.add_argument("--print-profile-commands", metavar="OUT",
                    help="print the rocprofv3 commands for --workload, output under OUT")
    args = ap.parse_args()
    if args.workload is None:
        args.workload = {"gemm": "gemm_tall_64k_2k_8k",
                         "decode": "decode_gqa64x8_b16_128k"}.get(args.which, "mha_128k")
    if (args.which == "gemm") != (args.workload in GEMM_WORKLOADS):
        ap.error("--pass gemm takes a gemm_* workload; the attention passes take the others")
    if (args.which == "decode") != (args.workload in SPLIT_WORKLOADS):
        ap.error("--pass decode takes a decode_* workload; the other passes take the others")
    if args.summarize_profile:
        if args.which == "decode":
            summarize_decode_profile(args.summarize_profile, args.workload)
        elif args.which == "gemm":
            summarize_gemm_profile(args.summarize_profile, args.workload)
        elif args.which == "bwd":
            summarize_bwd_profile(args.summarize_profile, args.workload)
        else:
            summarize_profile(args.summarize_profile, args.workload)
        return
    if args.print_profile_commands:
        for cmd in profile_commands(args.workload, args.print_profile_commands, args.which).values():
            print(cmd)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the attention forward pass here runs "
              "on a single MI355X; multi-GPU runs are not part of this build.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import chiplet_numa_aware_amd as attn
    from chiplet_numa_aware_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}))
        return
    attn.load_library()
    if args.sweep:
        run_sweep(args.sweep)
        return
    if args.which == "bwd":
        run_bwd(args, attn, inputs)
        return
    if args.which == "gemm":
        run_gemm(args, attn, inputs)
        return
    if args.which == "decode":
        run_decode(args, attn, inputs)
        return
    B, H_Q, H_KV, N, d, causal = WORKLOADS[args.workload]
    modes = [int(m) for m in args.modes.split(",") if m.strip() != ""]
    headline = _headline_mode(modes, causal)
    flops = attn_flops(B, H_Q, N, d, causal)
    log(f"workload {describe(args.workload)}: {flops / 1e12:.1f} TFLOP per call")

    q, k, v = inputs.make_qkv(B, H_Q, H_KV, N, d, seed=1000, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H_Q, N), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    results = {}
    for mode in modes:
        r = time_mode(attn, q, k, v, o, lse, causal, mode, args.steps,
                      args.warmup, flops)
        results[mode] = r
        log(f"  {MODE_NAMES[mode]:22s} {r['tflops']:8.1f} TFLOP/s "
            f"({r['pct_peak']:.1f}% of peak, kernel {r['kernel_ms_avg']:.2f} ms)")

    khash = kernel_hash()
    counters = stored_counters(args.workload, khash)
    head = results[headline]
    modes_out = {}
    for mode, r in results.items():
        entry = {k2: round(v2, 4) for k2, v2 in r.items()}
        if counters and MODE_NAMES[mode] in counters.get("modes", {}):
            c = counters["modes"][MODE_NAMES[mode]]
            entry["l2_hit_pct"] = c.get("l2_hit_pct")
            entry["hbm_bytes_per_launch"] = c.get("hbm_bytes")
        modes_out[MODE_NAMES[mode]] = entry

    traffic = None
    l2_hit = None
    if counters and MODE_NAMES[headline] in counters.get("modes", {}):
        c = counters["modes"][MODE_NAMES[headline]]
        traffic = c.get("hbm_bytes")
        l2_hit = c.get("l2_hit_pct")

    out = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: bf16 N(0,1) Q/K/V from fixed seeds",
        "config": {
            "workload": describe(args.workload),
            "B": B, "H_Q": H_Q, "H_KV": H_KV, "N": N, "d": d,
            "causal": causal, "mapping": MODE_NAMES[headline],
            "block_m": attn.BLOCK_M, "parallelism": "single GPU",
        },
        "pct_peak": round(head["pct_peak"], 2),
        "l2_hit_pct": l2_hit,
        "modes": modes_out,
        "roofline": _fwd_roofline(d, head["kernel_tflops"], traffic),
        "kernel_hash": khash,
        "counters_source": counters_source(args.workload, khash, "fwd", counters),
        "device": device_info(),
    }
    if 0 in results and headline in results and headline != 0:
        out["speedup_vs_naive_block_first"] = round(
            results[0]["kernel_ms_avg"] / results[headline]["kernel_ms_avg"], 4)
    if args.workload == "mha_128k":
        # The digest page's own figures for this workload (MI300X, Triton
        # FA2, relative numbers only): context, not a target.
        out["context_mi300x"] = {
            "speedup_vs_naive_block_first": [1.43, 1.56],
            "l2_hit_pct_swizzled_head_first": [90, 97],
            "l2_hit_pct_naive_block_first": 1,
        }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host (cpu_baseline)")
        out["cpu_baseline"] = cpu_baseline(q, k, v, causal, args.cpu_seconds)
    emit(out, args)


if __name__ == "__main__":
    main()
