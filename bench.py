#!/usr/bin/env python3
"""Benchmark of the quantized attention forward on one MI355X.

One step = one whole forward pass (preprocessing: means, INT8/FP8 quantization, Delta S;
then the fused attention kernel) over one batch of seeded synthetic input already
resident in HBM, through the C ABI (sage_attn_fwd_ex with a preallocated workspace).

Metric: attention TOPS = 4 N^2 d H B / time, causal counted as half (the pages'
convention: "Quantization for Attention, in depth", "When attention compute is worth
quantizing"; "SageAttention2 Technical Report", kernel speed figures).  The default
workload is the LLM-prefill shape B=1, H=32, N=M=32768, d=128, bf16, causal.

Printed: ONE JSON line with the metric, a roofline object for the dominant kernel (the
fused attention kernel, timed with HIP events attached to every one of its launches in the
timed region: the launch itself sets them to the kernel's start and end times) and a cpu_baseline object (the CPU oracle on a bounded sample of the
same workload, rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TOPS = 5000.0     # MI355X dense INT8 / OCP-FP8 MFMA peak, 5.0 POPS
PEAK_TOPS_FP4 = 10100.0  # MI355X dense MXFP4 MFMA peak, 10.1 PFLOP/s (the MX variant's contractions)
# VALU issue peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-slots per second (the published
# FP32 vector 157.3 TFLOP/s counts 2 flops per FMA and 2 lanes per packed FP32 instruction,
# and the kernels use no packed FP32).  A half-rate instruction (v_exp_f32, the FP8 and FP4
# packs) takes two slots.
PEAK_VALU_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12

# The softmax's VALU work per score element, in lane-slots: the method's steps as the fewest
# gfx950 instructions that carry them out (INT8 path: convert the INT32 score, one FMA for
# dequantization and Delta S, half a v_max3 for the row max, the subtraction of the running
# max, exp2 (2 slots), the row sum, half of a two-value FP8 pack (2 slots); E4M3 QK: no
# convert; MX: no convert and no dequantization (the block scales and Delta S are summed by
# the matrix core), one FMA for sm_scale log2(e) and the running max, the FP4 pack of two
# values per instruction).
VALU_SLOTS_PER_SCORE = {"i8f8": 7.5, "qkfp8": 6.5, "mx": 5.5}

# Kernel-level HBM traffic of the fused attention kernel, one launch on the named workload:
# rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (KiB per dispatch) scaled by what the same
# counters read for a plain 1 GiB device copy (FETCH x2.000, WRITE x1.000).  Valid only for
# the kernel source it was taken on: the hash of that fused kernel's sources is checked,
# and a changed kernel reports traffic null until the counters are taken again.
TRAFFIC_BYTES = {
    "prefill32k": {"source_sha256_16": "f4b7745f9c66d9fa",
                   "fetch_bytes": 1834093315, "write_bytes": 268486042},
    "mxfp4_32k": {"source_sha256_16": "d4319ec4c6fe92b7",
                  "fetch_bytes": 1688355523, "write_bytes": 201327104},
    "video17k": {"source_sha256_16": "f4b7745f9c66d9fa",
                 "fetch_bytes": 2110387978, "write_bytes": 215654400},
}
# SQ counters of the fused attention kernel on the named workload (rocprofv3 --pmc, the summary
# under profiles/): VALU and matrix-core busy fractions of the SIMD cycles, instructions per
# (wave, 64-key tile) as SQ_INSTS_VALU (which counts the MFMA instructions too) and
# SQ_INSTS_MFMA report them, and the engine clock of the profiled dispatch (GRBM_GUI_ACTIVE
# cycles per XCD over its duration).  Keyed by the same source hash as the traffic; null once stale.
COUNTERS = {
    "prefill32k": {"source_sha256_16": "f4b7745f9c66d9fa", "valu_busy": 0.902, "mfma_busy": 0.405,
                   "valu_insts_per_wave_tile": 235.2, "mfma_insts_per_wave_tile": 12.0,
                   "clock_ghz_profiled": 1.779, "wave_tiles": 8404992, "waves_per_simd": 2.83,
                   "waves_per_simd_max": 3,
                   "summary": "profiles/attn_fwd_prefill32k_counters.md"},
    "mxfp4_32k": {"source_sha256_16": "d4319ec4c6fe92b7", "valu_busy": 0.943, "mfma_busy": 0.245,
                  "valu_insts_per_wave_tile": 184.9, "mfma_insts_per_wave_tile": 8.0,
                  "clock_ghz_profiled": 1.955, "wave_tiles": 12582912, "waves_per_simd": 2.82,
                  "waves_per_simd_max": 3,
                  "summary": "profiles/attn_fwd_mx_mxfp4_32k_counters.md"},
    "video17k": {"source_sha256_16": "f4b7745f9c66d9fa", "valu_busy": 1.033, "mfma_busy": 0.251,
                 "valu_insts_per_wave_tile": 214.2, "mfma_insts_per_wave_tile": 6.03,
                 "clock_ghz_profiled": 1.924, "wave_tiles": 14493600, "waves_per_simd": 3.72,
                 "waves_per_simd_max": 4,
                 "summary": "profiles/attn_fwd_video17k_counters.md"},
}
_COMMON_SOURCES = ("quantized_attention_amd/csrc/attn_device.hpp", "quantized_attention_amd/csrc/sage_common.hpp")
KERNEL_SOURCES = {
    False: ("quantized_attention_amd/csrc/attn_fwd.hip",) + _COMMON_SOURCES,    # INT8/FP8 path
    True: ("quantized_attention_amd/csrc/attn_fwd_mx.hip",) + _COMMON_SOURCES,  # MXFP4 variant
}


def kernel_source_hash(mx: bool = False) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[mx]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str, mx: bool = False):
    t = TRAFFIC_BYTES.get(name)
    if t is None or t["source_sha256_16"] != kernel_source_hash(mx):
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def measured_counters(name: str, mx: bool = False):
    c = COUNTERS.get(name)
    if c is None or c["source_sha256_16"] != kernel_source_hash(mx):
        return None
    return {k: v for k, v in c.items() if k != "source_sha256_16"}


def scores_of(cfg) -> float:
    """(query, key) score elements the fused kernel evaluates, with the metric's causal counting
    (half of N^2 for causal N = M; the visible pairs otherwise)."""
    return counted_ops(cfg) / (4.0 * cfg.d)


def host_info() -> dict:
    """The host the CPU baseline ran on: logical CPUs and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill32k",
                    help="one of: n4k, prefill32k, prefill32k_b, full32k, video17k, chunk4k_32k, prefill32k_gqa, "
                         "prefill32k_qkfp8, "
                         "mxfp4_32k, mxfp4_32k_p2l, train8k (default prefill32k)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-measured-peak", action="store_true",
                    help="skip the matrix-core rate probe (libsage_probe.so) after the timed steps")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the steps, copy a MIB-MiB device buffer twice (a plain copy kernel of "
                         "known size, the reference point for HBM byte counters)")
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls the timing needs (events), via ctypes."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventSynchronize(b) == 0
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def counted_ops(cfg) -> float:
    """4 d ops per (query, key) pair; causal with N = M counts half of N^2 (the pages'
    convention); causal with N != M counts the visible pairs."""
    ops = 4.0 * cfg.N * cfg.M * cfg.d * cfg.H * cfg.B
    if not cfg.causal:
        return ops
    if cfg.N == cfg.M:
        return ops / 2
    coff = cfg.M - cfg.N if cfg.causal == 2 else 0
    pairs = sum(min(cfg.M, r + coff + 1) for r in range(cfg.N))
    return 4.0 * pairs * cfg.d * cfg.H * cfg.B


def cpu_baseline(cfg, budget_s: float) -> dict:
    """The oracle (as it stands) on head 0 of the workload: batches of seeded random query
    rows until the time budget is spent; ops counted with the same convention per row
    (4 d x keys the row attends to)."""
    import oracle
    from quantized_attention_amd import synthetic as sy
    q, k, v = sy.make_qkv(cfg, heads=[0])
    rng = np.random.default_rng(7)
    s = 1.0 / math.sqrt(cfg.d)
    flags = (oracle.SMOOTH_V if cfg.smooth_v else 0) | (oracle.MXFP4 if cfg.mxfp4 else 0)
    flags |= oracle.QK_E4M3 if cfg.qk_fp8 else 0
    flags |= oracle.MX_P_TWO_LEVEL if cfg.mx_p_two_level else 0
    ops, t_used, nrows, batch, ncalls = 0.0, 0.0, 0, 8, 0
    while t_used < budget_s:
        rows = np.sort(rng.integers(0, cfg.N, batch))
        t0 = time.perf_counter()
        oracle.forward_head(q[0], k[0], v[0], cfg.fp16, cfg.causal, s, flags, rows=rows)
        dt = time.perf_counter() - t0
        t_used += dt
        nrows += batch
        ncalls += 1
        coff = cfg.M - cfg.N if cfg.causal == 2 else 0
        ops += sum(4.0 * cfg.d * (min(cfg.M, int(r) + coff + 1) if cfg.causal else cfg.M) for r in rows)
        if dt < budget_s / 8:
            batch = min(2 * batch, cfg.N)
    return {"value": ops / t_used / 1e12, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"head 0 of {cfg.B * cfg.H}: {ncalls} oracle calls on seeded random query rows of "
                      f"N={cfg.N} ({nrows} rows in all, drawn with replacement; every call includes the head's "
                      f"preprocessing and its Delta S rows), {t_used:.1f} s",
            "omp_threads": oracle.num_threads(), **host_info()}


def train_cpu_baseline(cfg, n=1024):
    """The SageBwd oracle (forward + backward) on head 0, cut to n queries and keys."""
    import oracle
    from quantized_attention_amd import synthetic as sy
    sub = cfg.with_shape(B=1, H=1, N=min(n, cfg.N), M=min(n, cfg.M))
    q, k, v = [x[0, 0] for x in sy.make_qkv(sub)]
    do = sy.f32_to_bf16_bits(np.random.default_rng(5).standard_normal(q.shape).astype(np.float32))
    t0 = time.perf_counter()
    oracle.sagebwd_backward(q, k, v, do, sub.fp16, sub.causal, 1.0 / math.sqrt(sub.d))
    dt = time.perf_counter() - t0
    ops = counted_ops(sub) * 14 / 4
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"head 0, first {sub.N} queries and keys (forward + backward, per-head preprocessing "
                      f"included), {dt:.1f} s", "omp_threads": oracle.num_threads(), **host_info()}


def main_train(args, cfg):
    """A SageBwd training step of the attention: forward (out, lse) then backward (dq, dk, dv), both on
    one workspace with SAGE_TRAIN_KEEP_QUANT: the forward quantizes Q, K and V once and leaves them
    there for the backward, as a training framework keeps the forward's activations."""
    import torch

    import quantized_attention_amd as qa
    from quantized_attention_amd import synthetic as sy
    qa.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] generating {cfg.name} B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d}", file=sys.stderr, flush=True)
    qb, kb, vb = sy.make_qkv(cfg)
    dob = sy.f32_to_bf16_bits(np.random.default_rng(5).standard_normal(qb.shape).astype(np.float32))
    dt = torch.bfloat16
    q, k, v, do = (torch.from_numpy(x.view(np.int16)).view(dt).to(dev) for x in (qb, kb, vb, dob))
    del qb, kb, vb, dob
    out = torch.empty_like(q)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device=dev)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    shape = qa.SageAttnShape(cfg.B, cfg.H, cfg.H, cfg.N, cfg.M, cfg.d, int(cfg.causal), 1.0 / math.sqrt(cfg.d),
                             qa.SAGE_IN_BF16 | qa.SAGE_TRAIN_KEEP_QUANT)
    ws_bytes = qa.sage_attn_train_workspace_bytes(shape)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    ws_ptr = (ws.data_ptr() + 255) // 256 * 256
    stream = torch.cuda.current_stream(dev).cuda_stream

    def fwd():
        rc = qa.sage_attn_train_fwd(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    ws_ptr, ws_bytes, stream)
        if rc != qa.SAGE_OK:
            raise qa.SageError(rc, "sage_attn_train_fwd")

    def bwd():
        rc = qa.sage_attn_train_bwd(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_bytes,
                                    stream)
        if rc != qa.SAGE_OK:
            raise qa.SageError(rc, "sage_attn_train_bwd")

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        fwd()
        bwd()
    t_stop.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_stop) / args.steps
    # the forward / backward split, from as many further steps with an event at each boundary
    # (outside the timed region: each event record adds a few microseconds to the stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b, c in ev:
        a.record()
        fwd()
        b.record()
        bwd()
        c.record()
    torch.cuda.synchronize()
    f_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    b_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    ops = counted_ops(cfg) * 14 / 4
    value = ops / (ms * 1e-3) / 1e12
    shape_s = f"N={cfg.N} d={cfg.d}" + (" causal" if cfg.causal else "")
    line = {
        "metric": f"training attention TOPS (SageBwd forward + backward, 14*N^2*d*H*B/time, causal counted as half) "
                  f"at {shape_s}, % of INT8 MFMA peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 (QK^T, P^T dO, dS K, dS^T Q, P V) + bf16 (dO V^T), fp32 softmax/accumulate",
        "data": "synthetic (seeded Gaussian + per-channel offsets; dO standard normal)",
        "config": {"workload": f"{cfg.name}: B={cfg.B} H={cfg.H} N=M={cfg.N} d={cfg.d} {cfg.dtype} "
                               f"{'causal' if cfg.causal else 'non-causal'}, forward + backward",
                   "global_batch": cfg.B, "seq_len": cfg.N, "heads": cfg.H, "head_dim": cfg.d,
                   "parallelism": "single GPU"},
        "frac_of_peak": round(value / PEAK_TOPS, 4),
        "forward_ms": round(f_ms, 4),
        "backward_ms": round(b_ms, 4),
        "train_mode": "the forward quantizes Q, K, V once and the backward reuses them (SAGE_TRAIN_KEEP_QUANT)",
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_TOPS, "unit": "TOPS",
                     "frac": round(value / PEAK_TOPS, 4), "traffic": None,
                     "note": "whole step (preprocessing included) against the INT8 peak; dO V^T runs at the bf16 rate"},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = train_cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); heads are independent, "
              "so a multi-GPU run would shard heads with no communication -- not measured here.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_attention_amd as qa
    from quantized_attention_amd import synthetic as sy

    cfg = sy.CONFIGS[args.workload]
    if cfg.train:
        return main_train(args, cfg)
    qa.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] generating {cfg.name} B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d}", file=sys.stderr, flush=True)
    qb, kb, vb = sy.make_qkv(cfg)
    dt = torch.float16 if cfg.fp16 else torch.bfloat16
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(dt).to(dev) for x in (qb, kb, vb))
    del qb, kb, vb
    out = torch.empty((cfg.B, cfg.H, cfg.N, cfg.d), dtype=dt, device=dev)
    var = (qa.SAGE_IN_FP16 if cfg.fp16 else qa.SAGE_IN_BF16) | (qa.SAGE_SMOOTH_V if cfg.smooth_v else 0)
    if cfg.mxfp4:
        var |= qa.SAGE_PATH_MXFP4
    if cfg.qk_fp8:
        var |= qa.SAGE_QK_FP8
    if cfg.mx_p_two_level:
        var |= qa.SAGE_MX_P_TWO_LEVEL
    peak = PEAK_TOPS_FP4 if cfg.mxfp4 else PEAK_TOPS
    shape = qa.SageAttnShape(cfg.B, cfg.H, cfg.hkv, cfg.N, cfg.M, cfg.d, int(cfg.causal), 1.0 / math.sqrt(cfg.d), var)
    ws_bytes = qa.sage_attn_workspace_bytes_ex(shape)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    ws_ptr = (ws.data_ptr() + 255) // 256 * 256
    stream = torch.cuda.current_stream(dev).cuda_stream
    scale = 1.0 / math.sqrt(cfg.d)
    hip = Hip()

    def step(evs=None):
        if evs is not None:
            qa.sage_attn_set_profile_events(evs[0], evs[1])
        rc = qa.sage_attn_fwd_ex(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), ws_ptr, ws_bytes,
                                 stream)
        if rc != qa.SAGE_OK:
            raise qa.SageError(rc, "sage_attn_fwd_ex")

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kev = [(hip.event(), hip.event()) for _ in range(args.steps)]
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(kev[i])
    t_stop.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_stop)
    kern_ms = [hip.elapsed(a, b) for a, b in kev]
    for a, b in kev:
        hip.destroy(a)
        hip.destroy(b)
    ms = total_ms / args.steps
    kms = float(np.mean(kern_ms))
    ops = counted_ops(cfg)
    value = ops / (ms * 1e-3) / 1e12
    achieved = ops / (kms * 1e-3) / 1e12
    traffic = measured_traffic(cfg.name, cfg.mxfp4)
    path = "mx" if cfg.mxfp4 else ("qkfp8" if cfg.qk_fp8 else "i8f8")
    slots = VALU_SLOTS_PER_SCORE[path] * scores_of(cfg) / (kms * 1e-3) / 1e12
    measured_peak = None
    if not args.no_measured_peak:
        from quantized_attention_amd import probe
        measured_peak = round(probe.mfma_rate(2 if cfg.mxfp4 else (1 if cfg.qk_fp8 else 0)), 1)
    # The fused kernel's binding resource is its vector work: per (wave, 64-key tile) the softmax
    # needs VALU_SLOTS_PER_SCORE x 32 x 4 cycles against 512 (INT8/FP8, d = 128) or 256 (FP4)
    # cycles of matrix-core work, so the roofline is the VALU issue rate; the metric's matrix-core
    # fraction is reported beside it.
    roofline = {
        "bound": "alu", "achieved": round(slots, 3), "peak": round(PEAK_VALU_TSLOTS, 3),
        "unit": "T VALU lane-slots/s", "frac": round(slots / PEAK_VALU_TSLOTS, 4), "traffic": traffic,
        "work": f"{VALU_SLOTS_PER_SCORE[path]} VALU lane-slots per score element x {scores_of(cfg):.4g} scores "
                f"per launch",
        "mfma": {"achieved": round(achieved, 2), "peak": peak, "unit": "TOPS", "frac": round(achieved / peak, 4),
                 "peak_measured": measured_peak,
                 "frac_of_measured": round(achieved / measured_peak, 4) if measured_peak else None},
        "counters": measured_counters(cfg.name, cfg.mxfp4),
    }
    dtype = ("e2m1 + e8m0 1x32 blocks (QK, PV), fp32 softmax/accumulate" if cfg.mxfp4
             else ("fp8e4m3(QK)+fp8e4m3(PV)" if cfg.qk_fp8 else "int8(QK)+fp8e4m3(PV)")
             + ", fp32 softmax/accumulate")
    shape = (f"N={cfg.N}" if cfg.N == cfg.M else f"N={cfg.N} M={cfg.M}") + f" d={cfg.d}" + (" causal" if cfg.causal else "")
    counting = ("4*N^2*d*H*B/time, causal counted as half" if cfg.N == cfg.M
                else "4*d*(visible query-key pairs)*H*B/time")
    metric = (f"attention TOPS ({counting}) at {shape}{', E4M3 QK' if cfg.qk_fp8 else ''}, % of INT8/FP8 MFMA peak"
              if not cfg.mxfp4 else
              f"attention TOPS ({counting}) at {shape}, MXFP4 variant"
              f"{' with two-level P' if cfg.mx_p_two_level else ''}, % of FP4 MFMA peak")
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded Gaussian + per-channel offsets)",
        "config": {"workload": f"{cfg.name}: B={cfg.B} H={cfg.H} " + (f"Hkv={cfg.hkv} " if cfg.hkv != cfg.H else "")
                               + (f"N=M={cfg.N}" if cfg.N == cfg.M else f"N={cfg.N} M={cfg.M}")
                               + f" d={cfg.d} {cfg.dtype} "
                               f"{('causal' if cfg.causal == 1 or cfg.N == cfg.M else 'causal (last query on last key)') if cfg.causal else 'non-causal'}"
                               f"{' smooth_v' if cfg.smooth_v else ''}",
                   "global_batch": cfg.B, "seq_len": cfg.N, "heads": cfg.H, "head_dim": cfg.d,
                   "parallelism": "single GPU"},
        "frac_of_peak": round(value / peak, 4),
        # the raw formula 4 N^2 d H B / time, without the causal halving (causal N = M only)
        "tops_raw_formula": round(2 * value, 2) if (cfg.causal and cfg.N == cfg.M) else round(value, 2),
        "attn_kernel_ms": round(kms, 4),
        "attn_kernel_ms_median": round(float(np.median(kern_ms)), 4),
        "attn_kernel_ms_min": round(float(np.min(kern_ms)), 4),
        "preprocess_ms": round(ms - kms, 4),
        "roofline": roofline,
    }
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline ({args.cpu_seconds:.0f} s budget)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
