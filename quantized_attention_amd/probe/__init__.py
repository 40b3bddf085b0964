"""ctypes binding of lib/libsage_probe.so: probes of the gfx950 instructions the attention kernels
rely on (matrix-core precision and rates, the E4M3 conversion).  A measurement aid beside the
attention library, used by the GPU unit tests and by bench.py's measured matrix-core peak; the
attention path never calls it.  Device buffers are torch tensors."""
from __future__ import annotations

import ctypes
import os

_LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "lib", "libsage_probe.so")
_lib = None

# VALU kinds of sage_probe_valu_rate: kind -> (name, VALU instructions per lane and step)
VALU_KINDS = {0: ("v_fma_f32", 8), 1: ("v_exp_f32", 8), 2: ("v_cvt_pk_fp8_f32", 8),
              3: ("v_cvt_scalef32_pk_fp4_f32", 8), 4: ("v_cvt_f32_i32 + v_cvt_i32_f32 + v_add_u32", 24),
              5: ("v_exp_f32 and v_fma_f32 interleaved", 16)}

# kind -> (name, operations per MFMA instruction: 2 x M x N x K)
RATE_KINDS = {0: ("int8 32x32x32", 2 * 32 * 32 * 32), 1: ("fp8 32x32x64", 2 * 32 * 32 * 64),
              2: ("fp4 32x32x64 block-scaled", 2 * 32 * 32 * 64)}


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is missing: build it with `python -m quantized_attention_amd.build`")
        L = ctypes.CDLL(_LIB)
        P, i, u = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint
        L.sage_probe_mfma_f8.argtypes = [P, P, P, P, P]
        L.sage_probe_mfma_i8.argtypes = [P, P, P, P, P]
        L.sage_probe_cvt_e4m3.argtypes = [u, u, P, P]
        L.sage_probe_mfma_rate.argtypes = [i, i, i, P, P]
        L.sage_probe_valu_rate.argtypes = [i, i, i, ctypes.c_float, P, P]
        L.sage_probe_stream.argtypes = [i, P, ctypes.c_ulonglong, P, P]
        L.sage_probe_cvt_u8.argtypes = [u, u, P, P]
        for f in (L.sage_probe_mfma_f8, L.sage_probe_mfma_i8, L.sage_probe_cvt_e4m3, L.sage_probe_mfma_rate,
                  L.sage_probe_valu_rate, L.sage_probe_stream, L.sage_probe_cvt_u8):
            f.restype = i
        _lib = L
    return _lib


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: HIP error {rc}")


def mfma_f8(a, b, c):
    """D = A B + C on the FP8 MFMA (one wave): a, b uint8 [64, 32] (E4M3 codes per lane), c float32
    [64, 16] (C registers per lane) -> float32 [64, 16]."""
    import torch
    d = torch.empty_like(c)
    _check(load().sage_probe_mfma_f8(a.data_ptr(), b.data_ptr(), c.data_ptr(), d.data_ptr(), _stream()), "mfma_f8")
    torch.cuda.synchronize()
    return d


def mfma_i8(a, b, c):
    """D = A B + C on the INT8 MFMA (one wave): a, b int8 [64, 16], c int32 [64, 16] -> int32 [64, 16]."""
    import torch
    d = torch.empty_like(c)
    _check(load().sage_probe_mfma_i8(a.data_ptr(), b.data_ptr(), c.data_ptr(), d.data_ptr(), _stream()), "mfma_i8")
    torch.cuda.synchronize()
    return d


def cvt_e4m3(start: int, count: int):
    """E4M3 codes (the kernels' clamp to +-448, then v_cvt_pk_fp8_f32) of the FP32 values with bit
    patterns start .. start + count - 1, as a uint8 device tensor."""
    import torch
    out = torch.empty(count, dtype=torch.uint8, device="cuda")
    _check(load().sage_probe_cvt_e4m3(start, count, out.data_ptr(), _stream()), "cvt_e4m3")
    torch.cuda.synchronize()
    return out


def cvt_u8(start: int, count: int):
    """The bytes v_cvt_pk_u8_f32 makes of the FP32 values with bit patterns start .. start + count - 1,
    as a uint8 device tensor."""
    import torch
    out = torch.empty(count, dtype=torch.uint8, device="cuda")
    _check(load().sage_probe_cvt_u8(start, count, out.data_ptr(), _stream()), "cvt_u8")
    torch.cuda.synchronize()
    return out


def mfma_rate(kind: int, blocks: int = 4096, iters: int = 512, repeats: int = 3) -> float:
    """Measured matrix-core rate in TOPS (best of `repeats` timed launches after one warm-up):
    every wave runs 4 x iters independent MFMAs of the given kind (see RATE_KINDS)."""
    import torch
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    s = _stream()
    _check(load().sage_probe_mfma_rate(kind, blocks, iters, sink.data_ptr(), s), "mfma_rate")
    best = float("inf")
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _check(load().sage_probe_mfma_rate(kind, blocks, iters, sink.data_ptr(), s), "mfma_rate")
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    ops = blocks * 4 * 4 * iters * RATE_KINDS[kind][1]
    return ops / (best * 1e-3) / 1e12


def valu_rate(kind: int, blocks: int = 2048, iters: int = 1024, repeats: int = 3) -> float:
    """Measured VALU rate of one instruction kind (see VALU_KINDS), in wave64 instructions per
    nanosecond over the whole chip (best of `repeats` timed launches after one warm-up)."""
    import torch
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    s = _stream()
    _check(load().sage_probe_valu_rate(kind, blocks, iters, 0.999, sink.data_ptr(), s), "valu_rate")
    best = float("inf")
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _check(load().sage_probe_valu_rate(kind, blocks, iters, 0.999, sink.data_ptr(), s), "valu_rate")
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    waves = blocks * 4
    return waves * iters * VALU_KINDS[kind][1] / (best * 1e6)


def stream_rate(kind: int, buf, nbytes: int) -> float:
    """Reads (kind 0) or writes (kind 1) the first nbytes of the device tensor buf once, timed with
    events on the current stream; returns TB/s.  Whatever ran before on the stream (a buffer read or
    written just before) is what the caller measures against."""
    import torch
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    sink = torch.zeros(1, dtype=torch.float32, device=buf.device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    _check(load().sage_probe_stream(kind, buf.data_ptr(), nbytes, sink.data_ptr(), _stream()), "stream")
    e1.record()
    e1.synchronize()
    return nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e12
