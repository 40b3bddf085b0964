"""Seeded synthetic attention inputs of the pages' workload shapes.

This module only draws numbers: it holds none of the method's arithmetic, and both the
GPU tests and the oracle-side checks take their inputs from it.

The pages measure on activations captured from real models (channel-biased Q and K,
V with per-channel stripes; "SageAttention2 Technical Report", section 3.4 "Smoothing Q",
"FP8 Quantization for P~V") and on N(0,1) inputs for kernel speed.  None of those tensors
are available, so each configuration draws Gaussian tokens plus a per-channel offset
vector shared by all tokens of a (batch, head) -- the structure the smoothing steps
exist for -- and, where asked, a few channels pinned to a large offset (the +8 channel of
"Quantization for Attention, in depth", "Worked example").

Generation: numpy PCG64 seeded with (seed, tensor id, batch, head); Gaussian draws in
FP32; the sum is rounded to bf16 (round-to-nearest-even on the FP32 bits) or fp16.
Arrays are returned as raw 16-bit patterns (uint16), shape [B, H, T, d].
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


@dataclass(frozen=True)
class Dist:
    """Value distribution of one configuration (all per (batch, head))."""
    q_off_std: float = 0.0       # Q += o_q, o_q[c] ~ N(0, q_off_std^2)
    k_off_std: float = 0.0       # K += o_k, o_k[c] ~ N(0, k_off_std^2)
    k_spike: float = 0.0         # value written into o_k at the spike channels
    k_spike_channels: tuple = () # channels whose K offset is set to k_spike
    v_bias_std: float = 0.0      # V += b_v, b_v[c] ~ N(0, v_bias_std^2)


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    N: int
    M: int
    d: int
    dtype: str          # "bf16" or "fp16"
    causal: int  # 0 none; 1 first query aligned with the first key; 2 last with the last
    dist: Dist
    seed: int
    smooth_v: bool = False
    mxfp4: bool = False
    note: str = ""
    Hkv: int = 0        # key/value heads (0: H); query head h reads key/value head h // (H // Hkv)
    qk_fp8: bool = False  # Q^, K^ in E4M3 instead of INT8
    train: bool = False   # SageBwd forward + backward (a training step of the attention)
    mx_p_two_level: bool = False  # MX variant with two-level P quantization (row-scaled by rowmax / 6)

    @property
    def fp16(self) -> bool:
        return self.dtype == "fp16"

    @property
    def hkv(self) -> int:
        return self.Hkv or self.H

    def with_shape(self, **kw) -> "Config":
        return replace(self, **kw)


def spike_channels(d: int) -> tuple:
    """Four channels spread over the head dimension (one per quarter)."""
    return (0, d // 4 + 1, d // 2 + 2, 3 * d // 4 + 3)


# The five workloads, in the order the benchmark description lists them.
CONFIGS = {
    "tiny": Config("tiny", 1, 1, 256, 256, 64, "fp16", False,
                   Dist(k_off_std=3.0, k_spike=8.0, k_spike_channels=spike_channels(64)), 1001,
                   note="oracle check; INT8 QK, FP8 PV"),
    "n4k": Config("n4k", 1, 32, 4096, 4096, 128, "bf16", False,
                  Dist(k_off_std=2.0, v_bias_std=0.5), 1002,
                  note="INT8 per-thread-group QK, FP8 E4M3 PV"),
    "prefill32k": Config("prefill32k", 1, 32, 32768, 32768, 128, "bf16", True,
                         Dist(k_off_std=4.0, k_spike=8.0, k_spike_channels=spike_channels(128)), 1003,
                         note="LLM prefill layer (8B-style), causal"),
    "prefill32k_b": Config("prefill32k_b", 1, 32, 32768, 32768, 128, "bf16", True,
                           Dist(k_off_std=4.0, v_bias_std=0.5), 1009,
                           note="the prefill layer with the N = 4096 workload's distribution and K offset std 4"),
    "video17k": Config("video17k", 2, 48, 17550, 17550, 64, "bf16", False,
                       Dist(q_off_std=3.0, k_off_std=3.0, v_bias_std=1.0), 1004, smooth_v=True,
                       note="video diffusion shape, ragged last tile, V smoothing"),
    "chunk4k_32k": Config("chunk4k_32k", 1, 32, 4096, 32768, 128, "bf16", 2,
                          Dist(k_off_std=4.0, k_spike=8.0, k_spike_channels=spike_channels(128)), 1006,
                          note="chunked prefill: the last 4096 queries over a 32768-token cache, causal"),
    "prefill32k_gqa": Config("prefill32k_gqa", 1, 32, 32768, 32768, 128, "bf16", 1,
                             Dist(k_off_std=4.0, k_spike=8.0, k_spike_channels=spike_channels(128)), 1007,
                             Hkv=8, note="LLM prefill with grouped key/value heads (32 query heads, 8 key/value)"),
    "full32k": Config("full32k", 1, 32, 32768, 32768, 128, "bf16", False,
                      Dist(k_off_std=4.0, k_spike=8.0, k_spike_channels=spike_channels(128)), 1003,
                      note="the prefill layer's shape and inputs without the causal mask (no counting convention)"),
    "prefill32k_qkfp8": Config("prefill32k_qkfp8", 1, 32, 32768, 32768, 128, "bf16", True,
                               Dist(k_off_std=4.0, k_spike=8.0, k_spike_channels=spike_channels(128)), 1003,
                               qk_fp8=True, note="the prefill layer with Q^, K^ in E4M3 (same inputs)"),
    "train8k": Config("train8k", 1, 32, 8192, 8192, 128, "bf16", True,
                      Dist(k_off_std=4.0, k_spike=8.0, k_spike_channels=spike_channels(128)), 1008, train=True,
                      note="SageBwd training step (forward + backward) of an 8k-token causal layer"),
    "mxfp4_32k": Config("mxfp4_32k", 1, 24, 32768, 32768, 128, "bf16", False,
                        Dist(k_off_std=2.0, v_bias_std=0.5), 1005, mxfp4=True,
                        note="MXFP4 variant"),
    "mxfp4_32k_p2l": Config("mxfp4_32k_p2l", 1, 24, 32768, 32768, 128, "bf16", False,
                            Dist(k_off_std=2.0, v_bias_std=0.5), 1005, mxfp4=True, mx_p_two_level=True,
                            note="MXFP4 variant with two-level P quantization (same inputs)"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    r = u >> 16
    r &= 1
    r += np.uint32(0x7FFF)
    u += r
    u >>= 16
    return u.astype(np.uint16)


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bits_to_f32(bits: np.ndarray, fp16: bool) -> np.ndarray:
    """Widen 16-bit patterns to FP32 (exact)."""
    if fp16:
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _head(cfg: Config, tensor: int, b: int, h: int, T: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64([cfg.seed, tensor, b, h]))
    d = cfg.d
    dist = cfg.dist
    off = np.zeros(d, np.float32)
    if tensor == TENSOR_Q and dist.q_off_std:
        off = (rng.standard_normal(d) * dist.q_off_std).astype(np.float32)
    if tensor == TENSOR_K:
        if dist.k_off_std:
            off = (rng.standard_normal(d) * dist.k_off_std).astype(np.float32)
        for c in dist.k_spike_channels:
            off[c] = dist.k_spike
    if tensor == TENSOR_V and dist.v_bias_std:
        off = (rng.standard_normal(d) * dist.v_bias_std).astype(np.float32)
    x = rng.standard_normal((T, d), dtype=np.float32)
    x += off[None, :]
    if cfg.fp16:
        return f32_to_fp16_bits(x)
    u = x.view(np.uint32)  # x is owned here: round to bf16 in place
    r = u >> 16
    r &= 1
    r += np.uint32(0x7FFF)
    u += r
    u >>= 16
    return u.astype(np.uint16)


def make_tensor(cfg: Config, tensor: int, heads=None) -> np.ndarray:
    """One of Q, K, V as uint16 bits [B, H, T, d] (K and V: [B, Hkv, T, d]), or
    [len(heads), T, d] for a subset of flattened (b*heads + h) head indices."""
    T = cfg.N if tensor == TENSOR_Q else cfg.M
    H = cfg.H if tensor == TENSOR_Q else cfg.hkv
    idx = list(range(cfg.B * H)) if heads is None else list(heads)
    out = np.empty((len(idx), T, cfg.d), np.uint16)

    def fill(i):  # each head has its own generator, so threads do not change the values
        bh = idx[i]
        out[i] = _head(cfg, tensor, bh // H, bh % H, T)

    with ThreadPoolExecutor(max_workers=min(8, len(idx))) as ex:
        list(ex.map(fill, range(len(idx))))
    if heads is None:
        return out.reshape(cfg.B, H, T, cfg.d)
    return out


def make_qkv(cfg: Config, heads=None):
    return tuple(make_tensor(cfg, t, heads) for t in (TENSOR_Q, TENSOR_K, TENSOR_V))
