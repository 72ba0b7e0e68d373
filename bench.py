#!/usr/bin/env python3
"""Benchmark of exact tiled attention on one MI355X; prints ONE JSON line.

A step is one pass of the whole hot path over one batch of synthetic input:
  * forward, one head, N = 8192, d = 128, BF16, non-causal (the headline case),
  * forward on the same inputs, causal,
  * split-KV GQA decode: B = 16, Hq = 32, Hkv = 8, L = 8192, d = 128, 16 chunks.
Inputs are seeded N(0,1) draws rounded to BF16 and resident in HBM before the
timed region, which runs K whole steps back to back (ms_per_step is its wall
time per step). Before the W warm-up steps the step runs untimed for 0.5 s so
the clock and address translation reach steady state. `value` is the non-causal forward's algorithmic TFLOP/s: 4 N^2 d
per call over the call's average duration, measured with HIP events on the
stream the kernels run on around K back-to-back calls (a call is the forward
kernel, plus the combine kernel when the keys are split). The decode rate is
reported as algorithmic HBM GB/s (K and V read once per KV head). The "also"
section adds other workloads and, for the step's three calls, cold-cache
timings (median and minimum of 50 single calls, each after reading 1 GiB).
"cpu_baseline" also carries "seconds_by_config": the oracle's time per
workload config over the rows its parity checks use (one head or sequence
timed, scaled by their count; all-rows times of sampled configs extrapolated).
"rocprof_counters" repeats, per workload, the committed rocprofv3 counter
figures (HBM-side bytes over the Q+K+V+O floor, L2 hit rate, MFMA busy, clock)
while the library's sources are the ones they were taken from, else null.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --calibrate-copy   (plain copy kernel of known size, for
                                           normalising hardware byte counters)
       python bench.py --only WORKLOAD [--reps R]
                                          (one workload alone after a 0.5 s
                                           untimed settle, for profilers:
                                           fwd-1x1x8192, fwd-1x1x8192-causal,
                                           fwd-1x32x4096, fwd-1x32x4096-causal,
                                           fwd-1x8x131072-causal, decode, decode-varlen,
                                           bwd-1x32x4096, bwd-1x32x4096-causal,
                                           fwd-fp8-1x32x4096, fwd-fp8-1x32x4096-causal)
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

METRIC = "attention fwd TFLOP/s & % BF16 MFMA peak (N=8K,d=128); decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 MFMA
# The analytic H100 figures of "FlashAttention HBM bytes, one head, 8K" ("A strong
# answer"): a model of one 8K head at d = 128 on an H100 SXM, printed there for context.
# They are the page's model: not measurements, and not a target.
PAGES_H100_MODEL = {
    "source": "FlashAttention HBM bytes, one head, 8K (A strong answer): analytic model, not measured",
    "h100_bf16_dense_tflops": 989.0,
    "h100_hbm_tbs": 3.35,
    "fwd_1x1x8192_d128_compute_floor_us": 34.7,
    "fwd_1x1x8192_d128_naive_us": 163.0,
    "fwd_1x1x8192_d128_hbm_floor_us": 2.5,
}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "fa_fwd_1x1x8192_d128_counters.txt")
KERNEL_SOURCES = ["fa_fwd.hip", "fa_device.h", "fa_launch.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_tiled_attention_fa_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per forward launch from the committed counter summary, if current."""
    if not os.path.exists(COUNTERS_FILE):
        return None, None
    fields = {}
    for line in open(COUNTERS_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, None
    try:
        return float(fields["hbm_bytes_per_launch"]), float(fields["call_hbm_bytes"])
    except (KeyError, ValueError):
        return None, None


ALL_COUNTERS_FILE = os.path.join(ROOT, "profiles", "fa_fwd_decode_counters_by_workload.md")


def all_sources_hash() -> str:
    """Digest of every kernel and host source of the library (csrc/*.hip, *.h, sorted by name)."""
    d = os.path.join(ROOT, "exact_tiled_attention_fa_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(d, name), "rb").read())
    return h.hexdigest()[:16]


def measured_counters():
    """Per-workload rocprofv3 figures (HBM-side bytes over the floor, L2 hit rate, MFMA busy, clock) from the
    committed counter summary, or None when it is missing or was taken from other sources."""
    if not os.path.exists(ALL_COUNTERS_FILE):
        return None
    recs, digest = {}, None
    for line in open(ALL_COUNTERS_FILE):
        t = line.strip()
        if t.startswith("sources_sha256_16:"):
            digest = t.split(":", 1)[1].strip()
        elif t.startswith("{") and '"workload"' in t:
            r = json.loads(t)
            out = {"bytes_over_floor": r["bytes_over_floor"], "call_bytes": r["call_bytes"],
                   "floor_bytes": r["floor_bytes"]}
            k0 = next(iter(r["kernels"].values()))  # the call's main kernel
            for f in ("l2_hit", "mfma_util_counted", "mfma_busy_est", "clock_ghz_est"):
                if f in k0:
                    out[f] = k0[f]
            recs[r["workload"]] = out
    if digest != all_sources_hash() or not recs:
        return None
    return recs


SETTLE_S = 0.5


def settle(fn, seconds: float = SETTLE_S) -> None:
    """Run `fn` untimed, synchronising every 16 calls, until `seconds` have passed."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            fn()
        torch.cuda.synchronize()


def calibrate_copy() -> None:
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def run_only(name: str, reps: int) -> None:
    """Launch one workload `reps` times (after two warm-ups) and print its mean time."""
    import numpy as np
    import torch

    import exact_tiled_attention_fa_amd as fa
    import seeded_inputs as si

    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    fwd_cases = {"fwd-1x1x8192": si.ONE_HEAD_8K, "fwd-1x1x8192-causal": si.ONE_HEAD_8K_CAUSAL,
                 "fwd-1x32x4096": si.HEADS32_4K, "fwd-1x32x4096-causal": si.HEADS32_4K_CAUSAL,
                 "fwd-1x8x131072-causal": si.LONG_128K}
    if name in fwd_cases:
        case = fwd_cases[name]
        q, k, v = (up(x) for x in si.fwd_inputs(case))
        o = torch.empty_like(q)
        lse = torch.empty((case.B, case.Hq, case.N), dtype=torch.float32, device=dev)
        fn = fa.prepare_fwd(q, k, v, o, lse, causal=case.causal, scale=case.scale)
        work = 4.0 * case.N ** 2 * case.d * case.B * case.Hq / (2 if case.causal else 1)
        unit = "TFLOP/s"
    elif name in ("fwd-fp8-1x32x4096", "fwd-fp8-1x32x4096-causal"):
        case = si.HEADS32_4K_CAUSAL if name.endswith("causal") else si.HEADS32_4K
        q8, k8, v8, qs, ks, vs = si.fwd_fp8_inputs(case)
        q, k, v = (torch.from_numpy(x).to(dev).view(torch.float8_e4m3fn) for x in (q8, k8, v8))
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty((case.B, case.Hq, case.N), dtype=torch.float32, device=dev)
        fn = fa.prepare_fwd_fp8(q, k, v, qs, ks, vs, o, lse, causal=case.causal, scale=case.scale)
        work = 4.0 * case.N ** 2 * case.d * case.B * case.Hq / (2 if case.causal else 1)
        unit = "TFLOP/s"
    elif name in ("bwd-1x32x4096", "bwd-1x32x4096-causal"):
        case = si.HEADS32_4K_CAUSAL if name.endswith("causal") else si.HEADS32_4K
        q, k, v = (up(x) for x in si.fwd_inputs(case))
        g = up(si.normal_bf16(np.random.default_rng(case.seed + 10_000), (case.B, case.Hq, case.N, case.d)))
        o, lse = fa.fwd(q, k, v, causal=case.causal, scale=case.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.bwd_workspace_bytes(case.B, case.Hq, case.N, case.d), dtype=torch.uint8, device=dev)
        fn = fa.prepare_bwd(q, k, v, o, lse, g, dq, dk, dv, ws, causal=case.causal, scale=case.scale)
        work = 10.0 * case.N ** 2 * case.d * case.B * case.Hq / (2 if case.causal else 1)
        unit = "TFLOP/s"
    elif name in ("decode", "decode-varlen"):
        case = si.DECODE_GQA
        q, k, v = (up(x) for x in si.decode_inputs(case))
        ws = torch.empty(fa.decode_workspace_bytes(case.B, case.Hq, case.L, case.d, case.num_splits),
                         dtype=torch.uint8, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((case.B, case.Hq), dtype=torch.float32, device=dev)
        if name == "decode":
            fn = fa.prepare_decode(q, k, v, o, lse, ws, num_splits=case.num_splits, scale=case.scale)
            work = 2.0 * case.B * case.Hkv * case.L * case.d * 2
        else:  # the main run's lengths: uniform in 1..L, seeded
            lens = np.random.default_rng(case.seed).integers(1, case.L + 1, size=case.B).astype(np.int32)
            fn = fa.prepare_decode(q, k, v, o, lse, ws, num_splits=case.num_splits, scale=case.scale,
                                   seq_lens=torch.from_numpy(lens).to(dev))
            work = 2.0 * int(lens.astype(np.int64).sum()) * case.Hkv * case.d * 2
        unit = "GB/s"
    else:
        raise SystemExit(f"unknown workload {name}")
    settle(fn)
    stream = torch.cuda.current_stream(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / reps
    rate = work / t / (1e12 if unit == "TFLOP/s" else 1e9)
    print(json.dumps({"workload": name, "reps": reps, "us": round(t * 1e6, 2), "rate": round(rate, 2),
                      "unit": unit}), flush=True)


def cpu_baseline(case, seconds: float, gpu_outputs=None) -> dict:
    """The FP64 oracle as it stands, timed on this host's cores over whole passes of the workload;
    with gpu_outputs, also the GPU results' errors against it per workload config."""
    import numpy as np
    import seeded_inputs as si
    from oracle import fa_oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # threadpoolctl missing: report the affinity set
        cores = len(os.sched_getaffinity(0))
    qb, kb, vb = si.fwd_inputs(case)
    q, k, v = (si.bf16_bits_to_f32(x) for x in (qb, kb, vb))
    rows_total = 0
    t0 = time.perf_counter()
    passes = 0
    while True:
        fa_oracle.attention_ref(q, k, v, case.causal, case.scale)
        passes += 1
        rows_total += case.N
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    flops = passes * 4.0 * case.N * case.N * case.d
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{passes} full pass(es) of the 1x1x8192 d128 non-causal forward ({rows_total} rows) "
                      f"in {dt:.1f} s, FP64 NumPy three-pass attention",
            "seconds_by_config": oracle_seconds_by_config(),
            "parity_by_config": parity_by_config(gpu_outputs) if gpu_outputs else None}


def parity_by_config(gpu_outputs: dict) -> dict:
    """Errors of this run's GPU results against the FP64 oracle, per workload config, on the rows
    the parity tests check (every row of the tiny, 8K and decode configs; the seeded 1,024 rows
    per head of the 32-head 4K and 128K ones). gpu_outputs[name] = (case, o, lse, rows) with o and
    lse numpy arrays of exactly those rows (rows None = all). Tolerances: O max abs <= 1e-2 and
    |dlse| / max(|lse|, 1) <= 1e-3."""
    import numpy as np
    import seeded_inputs as si
    from oracle import fa_oracle
    out = {}
    for name, (case, o_gpu, lse_gpu, rows, inputs) in gpu_outputs.items():
        t0 = time.perf_counter()
        q, k, v = (si.bf16_bits_to_f32(x) for x in inputs)
        if isinstance(case, si.DecodeCase):
            o_ref, lse_ref = fa_oracle.decode_ref(q, k, v, case.scale)
        else:
            o_ref, lse_ref = fa_oracle.attention_ref(q, k, v, case.causal, case.scale, rows=rows)
        err = np.abs(o_gpu.astype(np.float64) - o_ref)
        lrel = np.abs(lse_gpu.astype(np.float64) - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
        o_max, l_max = float(err.max()), float(lrel.max())
        out[name] = {"rows_checked": int(o_ref.shape[-2] * o_ref.shape[1] * o_ref.shape[0])
                     if not isinstance(case, si.DecodeCase) else int(o_ref.shape[0] * o_ref.shape[1]),
                     "o_max_abs": float(f"{o_max:.3e}"),
                     "o_rel_rms": float(f"{float(np.sqrt((err ** 2).sum() / (o_ref ** 2).sum())):.3e}"),
                     "lse_max_rel": float(f"{l_max:.3e}"),
                     "pass": bool(o_max <= 1e-2 and l_max <= 1e-3),
                     "oracle_s": round(time.perf_counter() - t0, 2)}
    return out


def oracle_seconds_by_config(cases=None, decode_cases=None) -> dict:
    """Seconds the FP64 oracle takes per workload config, over the rows its parity checks use.

    The oracle treats heads (and decode sequences) independently, so each config is timed on one
    head (one sequence) of seeded N(0,1) inputs of its shape and scaled by the head (sequence) count;
    large configs use the parity tests' seeded sample of rows per head, with the time for every
    row extrapolated linearly (the oracle scores every key of a row, masked or not)."""
    import dataclasses
    import numpy as np
    import seeded_inputs as si
    from oracle import fa_oracle
    if cases is None:
        cases = (si.TINY, si.ONE_HEAD_8K, si.ONE_HEAD_8K_CAUSAL, si.HEADS32_4K, si.HEADS32_4K_CAUSAL, si.LONG_128K)
    if decode_cases is None:
        decode_cases = (si.DECODE_GQA,)
    out = {}
    for case in cases:
        one = dataclasses.replace(case, B=1, Hq=1, Hkv=1)
        q, k, v = (si.bf16_bits_to_f32(x) for x in si.fwd_inputs(one))
        rows = None
        if case.sampled_rows and case.sampled_rows < case.N:
            rows = si.sample_rows(case.seed, 0, case.N, case.sampled_rows)
        t0 = time.perf_counter()
        fa_oracle.attention_ref(q, k, v, case.causal, case.scale, rows=rows)
        dt = time.perf_counter() - t0
        heads = case.B * case.Hq
        rec = {"seconds_one_head": round(dt, 3), "rows_per_head": case.N if rows is None else len(rows),
               "heads": heads, "seconds": round(dt * heads, 3)}
        if rows is not None:
            rec["seconds_all_rows_extrapolated"] = round(dt * heads * case.N / len(rows), 1)
        out[case.name] = rec
        del q, k, v
    for case in decode_cases:
        one = dataclasses.replace(case, B=1)
        q, k, v = (si.bf16_bits_to_f32(x) for x in si.decode_inputs(one))
        t0 = time.perf_counter()
        fa_oracle.decode_ref(q, k, v, case.scale)
        dt = time.perf_counter() - t0
        out[case.name] = {"seconds_one_sequence": round(dt, 3), "sequences": case.B, "rows": case.B * case.Hq,
                          "seconds": round(dt * case.B, 3)}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="bounded CPU oracle sample length")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary (non-step) measurements")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--only", default=None, help="run one workload alone (for profilers)")
    ap.add_argument("--reps", type=int, default=5)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the forward would shard by head "
              "with no exchange between GPUs). Run with --gpus 1.", file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch

    import exact_tiled_attention_fa_amd as fa
    import seeded_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy()
        return 0
    if args.only:
        run_only(args.only, args.reps)
        return 0

    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    fcase = si.ONE_HEAD_8K
    q, k, v = (up(x) for x in si.fwd_inputs(fcase))
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, fcase.N), dtype=torch.float32, device=dev)
    o_c = torch.empty_like(q)
    lse_c = torch.empty_like(lse)
    dcase = si.DECODE_GQA
    dq, dk, dv = (up(x) for x in si.decode_inputs(dcase))
    do = torch.empty_like(dq)
    dlse = torch.empty((dcase.B, dcase.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(dcase.B, dcase.Hq, dcase.L, dcase.d, dcase.num_splits),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    # Argument checks happen once here; each launch then costs one C call.
    run_fwd = fa.prepare_fwd(q, k, v, o, lse, causal=False, scale=fcase.scale)
    run_fwd_c = fa.prepare_fwd(q, k, v, o_c, lse_c, causal=True, scale=fcase.scale)
    run_dec = fa.prepare_decode(dq, dk, dv, do, dlse, ws, num_splits=dcase.num_splits, scale=dcase.scale)

    def step():
        run_fwd()
        run_fwd_c()
        run_dec()

    # Settle: run the step untimed for at least SETTLE_S seconds (the shader
    # clock and address translation take milliseconds to reach steady state;
    # a cold GPU runs the first millisecond of work up to 20% slower), then
    # the W warm-up steps.
    settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / max(args.steps, 1)

    # Per-operation call durations: HIP events on the launch stream around
    # `steps` back-to-back calls of one operation (an event between every two
    # launches would add its own gap to each interval).
    def per_call_s(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    reps = max(args.steps, 1)
    t_fwd, t_fwd_c, t_dec = per_call_s(run_fwd, reps), per_call_s(run_fwd_c, reps), per_call_s(run_dec, reps)
    flops = 4.0 * fcase.N * fcase.N * fcase.d
    tflops = flops / t_fwd / 1e12

    # The dominant kernel alone (the headline call's attention kernel, without
    # its key-split merge): an event recorded before each call and one that the
    # library records right after the kernel (fa_fwd_ws_timed), over `reps`
    # back-to-back calls. Each interval also holds the kernel's dispatch after
    # the previous call's merge, so it slightly overstates the kernel's time.
    def kernel_s(fn, reps):
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        mids = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        for e in starts + mids:  # torch creates each HIP event at its first record
            e.record(stream)
        torch.cuda.synchronize()
        for a, m in zip(starts, mids):
            a.record(stream)
            fn(after_attention=m)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(m) for a, m in zip(starts, mids)) * 1e-3 / reps

    t_kernel = kernel_s(run_fwd, reps)
    tflops_kernel = flops / t_kernel / 1e12
    tflops_c = flops / 2 / t_fwd_c / 1e12
    kv_bytes = 2 * dcase.B * dcase.Hkv * dcase.L * dcase.d * 2
    dec_gbs = kv_bytes / t_dec / 1e9

    extra = {}
    gpu_outputs = {}  # per workload config: GPU results on the rows the oracle checks

    def sampled(case, o_t, l_t):
        rows = (np.stack([si.sample_rows(case.seed, h, case.N, case.sampled_rows) for h in range(case.Hq)])
                if case.sampled_rows else None)
        o_np = o_t.float().cpu().numpy()
        l_np = l_t.float().cpu().numpy()
        if rows is not None:
            o_np = np.stack([o_np[:, h, rows[h]] for h in range(case.Hq)], axis=1)
            l_np = np.stack([l_np[:, h, rows[h]] for h in range(case.Hq)], axis=1)
        return o_np, l_np, rows

    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        fin = si.fwd_inputs(fcase)
        gpu_outputs[fcase.name] = (fcase, *sampled(fcase, o, lse)[:2], None, fin)
        gpu_outputs[si.ONE_HEAD_8K_CAUSAL.name] = (si.ONE_HEAD_8K_CAUSAL, *sampled(si.ONE_HEAD_8K_CAUSAL, o_c,
                                                                                    lse_c)[:2], None, fin)
        gpu_outputs[dcase.name] = (dcase, do.float().cpu().numpy()[:, :, 0], dlse.float().cpu().numpy(), None,
                                   si.decode_inputs(dcase))
        tin = si.fwd_inputs(si.TINY)
        qt, kt, vt = (up(x) for x in tin)
        ot, lt = fa.fwd(qt, kt, vt, causal=False, scale=si.TINY.scale)
        torch.cuda.synchronize()
        gpu_outputs[si.TINY.name] = (si.TINY, *sampled(si.TINY, ot, lt)[:2], None, tin)
        del qt, kt, vt, ot, lt

    if not args.no_extra:
        # The named fa_fwd entry point at the headline shape: on its key-split path it takes a
        # stream-ordered temporary buffer per call (hipMallocAsync / hipFreeAsync) where fa_fwd_ws,
        # timed above, uses a caller workspace.
        lib = fa._lib.lib()
        st_h = stream.cuda_stream
        o_x = torch.empty_like(q)
        l_x = torch.empty_like(lse)

        def run_fa_fwd():
            fa._lib.check(lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_x.data_ptr(), l_x.data_ptr(),
                                     1, 1, 1, fcase.N, fcase.d, 0, fcase.scale, st_h), "fa_fwd")

        def run_noalloc():
            fa._lib.check(lib.fa_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_x.data_ptr(),
                                             l_x.data_ptr(), 1, 1, 1, fcase.N, fcase.d, 0, fcase.scale, st_h),
                          "fa_fwd_noalloc")
        for key, fn in (("fwd_1x1x8192_d128_fa_fwd", run_fa_fwd), ("fwd_1x1x8192_d128_fa_fwd_noalloc", run_noalloc)):
            settle(fn, 0.2)
            t = per_call_s(fn, reps)
            extra[key] = {"us": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 2),
                          "frac_peak": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del o_x, l_x
        # Cold caches: before each of 50 single calls a 1 GiB buffer is read
        # (more than the 256 MiB last-level cache; reading leaves clean lines,
        # where a write would leave write-backs to compete with the call), then
        # the call is timed alone with events on the kernels' stream; median
        # and minimum.
        flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        for key, fn, fl in (("fwd_1x1x8192_d128_cold", run_fwd, flops),
                            ("fwd_1x1x8192_d128_causal_cold", run_fwd_c, flops / 2),
                            ("decode_B16_Hq32_Hkv8_L8192_cold", run_dec, None)):
            times = []
            for i in range(50):
                flush.amax()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b) * 1e-3)
            times.sort()
            med, best = times[len(times) // 2], times[0]
            if fl is None:
                extra[key] = {"us_median": round(med * 1e6, 2), "us_min": round(best * 1e6, 2),
                              "hbm_gbs_median": round(kv_bytes / med / 1e9, 1)}
            else:
                extra[key] = {"us_median": round(med * 1e6, 2), "us_min": round(best * 1e6, 2),
                              "tflops_median": round(fl / med / 1e12, 2)}
        del flush
        # The 32-head 4K forward both ways and the long-context 128K causal forward (each
        # call ~28 ms, so 3 timed calls).
        for case, nrep in ((si.HEADS32_4K, 10), (si.HEADS32_4K_CAUSAL, 10), (si.LONG_128K, 3)):
            fin3 = si.fwd_inputs(case)
            q3, k3, v3 = (up(x) for x in fin3)
            o3 = torch.empty_like(q3)
            l3 = torch.empty((case.B, case.Hq, case.N), dtype=torch.float32, device=dev)
            run3 = fa.prepare_fwd(q3, k3, v3, o3, l3, causal=case.causal, scale=case.scale)
            settle(run3, 0.2)
            t = per_call_s(run3, nrep)
            fl = 4.0 * case.N ** 2 * case.d * case.B * case.Hq / (2 if case.causal else 1)
            key = f"fwd_{case.B}x{case.Hq}x{case.N}_d{case.d}" + ("_causal" if case.causal else "")
            extra[key] = {"us": round(t * 1e6, 2), "tflops": round(fl / t / 1e12, 2),
                          "frac_peak": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4)}
            if not args.no_cpu_baseline:
                torch.cuda.synchronize()
                gpu_outputs[case.name] = (case, *sampled(case, o3, l3), fin3)
            del q3, k3, v3, o3, l3, fin3
        # FP8 forward at the 32-head 4K shape (E4M3 inputs quantised per tensor from
        # the same seeded draws); the peak it is quoted against is the FP8 one.
        for case in (si.HEADS32_4K, si.HEADS32_4K_CAUSAL):
            q8, k8, v8, qs, ks, vs = si.fwd_fp8_inputs(case)
            q3, k3, v3 = (torch.from_numpy(x).to(dev).view(torch.float8_e4m3fn) for x in (q8, k8, v8))
            o3 = torch.empty(q3.shape, dtype=torch.bfloat16, device=dev)
            l3 = torch.empty((case.B, case.Hq, case.N), dtype=torch.float32, device=dev)
            run8 = fa.prepare_fwd_fp8(q3, k3, v3, qs, ks, vs, o3, l3, causal=case.causal, scale=case.scale)
            settle(run8, 0.2)
            t = per_call_s(run8, 10)
            fl = 4.0 * case.N ** 2 * case.d * case.B * case.Hq / (2 if case.causal else 1)
            key = "fwd_fp8_1x32x4096_d128" + ("_causal" if case.causal else "")
            extra[key] = {"us": round(t * 1e6, 2), "tflops": round(fl / t / 1e12, 2),
                          "frac_fp8_peak": round(fl / t / 1e12 / PEAK_FP8_TFLOPS, 4)}
            del q3, k3, v3, o3, l3
        # Backward pass at the 32-head 4K shape: algorithmic FLOPs 10 N^2 d per head
        # (five N x N x d products; halved causal), upstream gradient seeded.
        for causal in (False, True):
            case = si.HEADS32_4K_CAUSAL if causal else si.HEADS32_4K
            q3, k3, v3 = (up(x) for x in si.fwd_inputs(case))
            g3 = up(si.normal_bf16(np.random.default_rng(case.seed + 10_000), (case.B, case.Hq, case.N, case.d)))
            o3, l3 = fa.fwd(q3, k3, v3, causal=causal, scale=case.scale)
            dq3, dk3, dv3 = torch.empty_like(q3), torch.empty_like(k3), torch.empty_like(v3)
            ws3 = torch.empty(fa.bwd_workspace_bytes(case.B, case.Hq, case.N, case.d), dtype=torch.uint8, device=dev)
            run_b = fa.prepare_bwd(q3, k3, v3, o3, l3, g3, dq3, dk3, dv3, ws3, causal=causal, scale=case.scale)
            settle(run_b, 0.2)
            t = per_call_s(run_b, 10)
            fl = 10.0 * case.N ** 2 * case.d * case.B * case.Hq / (2 if causal else 1)
            key = "bwd_1x32x4096_d128" + ("_causal" if causal else "")
            extra[key] = {"us": round(t * 1e6, 2), "tflops": round(fl / t / 1e12, 2),
                          "frac_peak": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4)}
            del q3, k3, v3, g3, o3, l3, dq3, dk3, dv3, ws3
        # Variable-length decode: the decode workload's shape, cache lengths drawn
        # uniformly from 1..8192 (seeded); bytes = the K/V rows actually read.
        vlens = np.random.default_rng(dcase.seed).integers(1, dcase.L + 1, size=dcase.B).astype(np.int32)
        vlens_t = torch.from_numpy(vlens).to(dev)
        run_vl = fa.prepare_decode(dq, dk, dv, do, dlse, ws, num_splits=dcase.num_splits, scale=dcase.scale,
                                   seq_lens=vlens_t)
        settle(run_vl, 0.2)
        t_vl = per_call_s(run_vl, 20)
        vl_bytes = 2 * int(vlens.astype(np.int64).sum()) * dcase.Hkv * dcase.d * 2
        extra["decode_varlen_B16_Hq32_Hkv8_Lmax8192"] = {
            "us": round(t_vl * 1e6, 2), "hbm_gbs": round(vl_bytes / t_vl / 1e9, 1),
            "frac_hbm_peak": round(vl_bytes / t_vl / 1e9 / PEAK_HBM_GBS, 4), "mean_len": float(vlens.mean())}

    traffic, call_traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fwd 1 head N=8192 d=128 non-causal (step also runs the causal fwd and a "
                               "B16 Hq32 Hkv8 L8192 16-split decode)",
                   "batch": 1, "heads": 1, "seq_len": 8192, "head_dim": 128, "causal": False},
        "roofline": {"bound": "mfma", "achieved": round(tflops_kernel, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops_kernel / PEAK_BF16_TFLOPS, 5), "traffic": traffic,
                     "kernel": "fa_fwd_kernel<128,false,8>", "kernel_us": round(t_kernel * 1e6, 2),
                     "call_frac": round(tflops / PEAK_BF16_TFLOPS, 5), "call_traffic": call_traffic},
        "fwd_us": round(t_fwd * 1e6, 2),
        "fwd_causal_tflops": round(tflops_c, 3),
        "fwd_causal_us": round(t_fwd_c * 1e6, 2),
        "decode_hbm_gbs": round(dec_gbs, 1),
        "decode_frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
        "decode_us": round(t_dec * 1e6, 2),
        "also": extra,
        "rocprof_counters": measured_counters(),
        "pages_h100_model": PAGES_H100_MODEL,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(fcase, args.cpu_seconds, gpu_outputs)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
