"""GPU parity of the MXFP4 variant (SAGE_PATH_MXFP4) against the CPU oracle (needs an MI355X).

Sources: "SageAttention3" summary, 3.4 "The NVFP4 Microscaling Format and Quantization
Operator" (E2M1 values, one E8M0 scale per 32 elements along the reduction dimension of each
product); the smoothing and the online softmax of "SageAttention2 Technical Report" 3.4.

Bars: E2M1 codes and E8M0 exponents of gamma(Q), gamma(K), V' bit-exact (their decisions are
made from the same FP32 values on both sides); the output within max |err| <= 1e-2 and
mean |err| <= 1e-3 of the MX oracle (FP32 output).  The pages give no accuracy bar for the
MX variant against exact attention; its cosine against FP64 attention is reported, with a
floor of 0.95 only to catch a broken path (the oracle itself reaches 0.97-0.9994 on these
inputs).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from quantized_attention_amd import synthetic as sy

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, MIN_COS_SANITY = 1e-2, 1e-3, 0.95


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_attention_amd
    quantized_attention_amd.load_library()


from tests import gpu_util as gu  # noqa: E402

MX_CASES = [
    ("tiny-d64", sy.CONFIGS["tiny"]),
    ("mx-ragged", sy.CONFIGS["mxfp4_32k"].with_shape(H=2, N=600, M=600)),
    ("causal-700", sy.CONFIGS["prefill32k"].with_shape(H=2, N=700, M=700)),
    ("smoothv-d64", sy.CONFIGS["video17k"].with_shape(B=2, H=1, N=333, M=333)),
    ("fp16-d128-N!=M", sy.Config("fp16x", 1, 2, 300, 1000, 128, "fp16", False,
                                 sy.Dist(q_off_std=1.0, k_off_std=2.0, v_bias_std=0.5), 77)),
    ("one-token", sy.Config("one", 1, 1, 1, 1, 64, "bf16", False, sy.Dist(), 79)),
    ("few-tokens", sy.Config("few", 1, 3, 5, 3, 128, "fp16", False, sy.Dist(k_off_std=1.0), 80)),
    ("causal-br-N<M", sy.CONFIGS["mxfp4_32k"].with_shape(H=2, N=300, M=1000, causal=2)),
]


def flags(cfg):
    return oracle.MXFP4 | (oracle.SMOOTH_V if cfg.smooth_v else 0)


@pytest.mark.parametrize("name,cfg", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_mx_preprocess_bit_exact(name, cfg):
    q, k, v = sy.make_qkv(cfg)
    say(f"mx quantize {name} B={cfg.B} H={cfg.H} N={cfg.N} M={cfg.M} d={cfg.d}")
    g = gu.quantize_mx(q, k, v, cfg.fp16, cfg.causal, cfg.smooth_v)
    N, M, d = cfg.N, cfg.M, cfg.d
    nvb = -(-M // 32)
    for bh in range(cfg.B * cfg.H):
        b, h = bh // cfg.H, bh % cfg.H
        o = oracle.preprocess_mx_head(q[b, h], k[b, h], v[b, h], cfg.fp16, oracle.SMOOTH_V if cfg.smooth_v else 0)
        assert np.array_equal(g["qcode"][bh, :N], o["qcode"])
        assert np.array_equal(g["qexp"][bh, :N], o["qexp"])
        assert np.array_equal(g["kcode"][bh, :M], o["kcode"])
        assert np.array_equal(g["kexp"][bh, :M], o["kexp"])
        assert np.array_equal(g["vcode"][bh, :M], o["vcode"])
        assert np.array_equal(g["vexp"][bh, :nvb], o["vexp"])
        # padding: codes 0, scale byte 0 (2^-127)
        assert not g["qcode"][bh, N:].any() and (g["qexp"][bh, N:] == -127).all()
        assert not g["kcode"][bh, M:].any() and (g["kexp"][bh, M:] == -127).all()
        assert not g["vcode"][bh, M:].any() and (g["vexp"][bh, nvb:] == -127).all()
        p = oracle.preprocess_head(q[b, h], k[b, h], v[b, h], cfg.fp16, oracle.SMOOTH_V if cfg.smooth_v else 0)
        assert np.array_equal(g["k_mean"][bh].view(np.uint32), p["kmean"].view(np.uint32))
        assert np.array_equal(g["v_mean"][bh].view(np.uint32), p["vmean"].view(np.uint32))
        assert np.array_equal(g["q_mean"][bh].view(np.uint32), p["qmean"].view(np.uint32))
    # scale bytes beyond d/64 (K) and d/32 (V) are documented as 0
    if d == 64:
        ks = g["mx_scales_k"]
        assert not ks[..., 1].any() and not ks[..., 3].any()
        assert not g["mx_scales_v"][..., 2:].any()


def run_mx(cfg, q, k, v, acc_valu=False):
    return gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, acc_valu=acc_valu, mxfp4=True).cpu().numpy()


def cosine(a, b):
    return float((a * b).sum() / math.sqrt((a * a).sum() * (b * b).sum()))


@pytest.mark.parametrize("name,cfg", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_mx_forward_parity_small(name, cfg):
    q, k, v = sy.make_qkv(cfg)
    say(f"mx forward {name} B={cfg.B} H={cfg.H} N={cfg.N} M={cfg.M} d={cfg.d} causal={cfg.causal}")
    out = run_mx(cfg, q, k, v)
    s = 1 / math.sqrt(cfg.d)
    got, ref, ex = [], [], []
    for bh in range(cfg.B * cfg.H):
        b, h = bh // cfg.H, bh % cfg.H
        got.append(out[b, h].astype(np.float64))
        ref.append(oracle.forward_head(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, s, flags(cfg)))
        ex.append(oracle.exact_head(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, s))
    g, r, e = np.stack(got), np.stack(ref), np.stack(ex)
    err = np.abs(g - r)
    say(f"  max abs {err.max():.3g} mean abs {err.mean():.3g} cos(gpu, fp64) {cosine(g, e):.5f} "
        f"cos(oracle, fp64) {cosine(r, e):.5f}")
    assert np.isfinite(g).all()
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
    if cfg.N > 1:
        assert cosine(g, e) >= MIN_COS_SANITY


@pytest.mark.parametrize("name", ["mx-ragged", "causal-700", "smoothv-d64"])
def test_mx_literal_two_level(name):
    cfg = dict(MX_CASES)[name]
    q, k, v = sy.make_qkv(cfg)
    say(f"mx literal two-level {name}")
    a = run_mx(cfg, q, k, v, acc_valu=True)
    b = run_mx(cfg, q, k, v)
    assert np.abs(a - b).max() <= 1e-5 * max(1.0, np.abs(b).max())


def test_mx_full_size_sampled():
    cfg = sy.CONFIGS["mxfp4_32k"]
    q, k, v = sy.make_qkv(cfg)
    say(f"mx full-size forward B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, mxfp4=True)
    BH = cfg.B * cfg.H
    s = 1 / math.sqrt(cfg.d)
    rng = np.random.default_rng(5)
    for bh in sorted({0, BH // 2, BH - 1}):
        b, h = bh // cfg.H, bh % cfg.H
        rows = np.array(sorted(set([0, 1, 127, 128, cfg.N // 2, cfg.N - 1] + list(rng.integers(0, cfg.N, 16)))))
        got = out[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        ref = oracle.forward_head(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, s, flags(cfg), rows=rows)
        err = np.abs(got - ref)
        say(f"  head {bh}: max abs {err.max():.3g}")
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


def test_mx_long_sequence_sampled():
    """One head of 262144 tokens on the MX path (causal, prefill-shaped): Delta S is 2 GiB, so the
    workspace and tile offsets pass 2^31 bytes; rows at both ends and around the middle."""
    cfg = sy.CONFIGS["mxfp4_32k"].with_shape(H=1, N=262144, M=262144, causal=1)
    q, k, v = sy.make_qkv(cfg)
    say(f"mx long forward N={cfg.N} d={cfg.d} causal={cfg.causal}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, mxfp4=True)
    N = cfg.N
    rows = np.array(sorted(set([0, 1, 127, 128, N // 2 - 1, N // 2, N - 2, N - 1]
                               + list(np.random.default_rng(9).integers(0, N, 6)))))
    got = out[0, 0, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    ref = oracle.forward_head(q[0, 0], k[0, 0], v[0, 0], cfg.fp16, cfg.causal, 1 / math.sqrt(cfg.d), flags(cfg),
                              rows=rows)
    err = np.abs(got - ref)
    say(f"  max abs {err.max():.3g}")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
