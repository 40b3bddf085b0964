"""GPU parity of the E4M3 QK knob (SAGE_QK_FP8) against the CPU oracle (needs an MI355X).

Source: "SageAttention2 Technical Report" summary, "Critical Assessment" (the FP8-QK form of
SageAttention2-8b that the pages name and do not run); 3.3 "FP8 Quantization for P~V" fixes
the E4M3 range that sets the scale.

Bars:
  * Q^ and K^ codes (E4M3 bytes), dQ and dK bit-exact with the oracle's QK_E4M3 quantizer;
    the rest of the preprocessing (means, V^, Delta S) as in the INT8 path;
  * the output within mean |err| <= 1e-3 of the oracle (FP32 output), and its cosine
    against FP64 attention within 1e-4 of the oracle's own (0.9985 - 0.9999 on these
    inputs), with a floor of 0.998;
  * every row within max |err| <= 1e-2 plus the oracle's margin bound for that row (0 on rows
    with no P~ near an E4M3 rounding midpoint), and within one P^ step: max |err| <= max|V| / 8.
    Why a margin: the oracle sums Q^ K^ exactly, while the FP8 MFMA sums each 64-channel step
    with an error of up to FP8_MFMA_STEP_ERR times the step's largest code product (measured
    by tests/test_gpu_probes.py: worst 2^-11.4, typical 2^-15).  A score can then differ from
    the oracle's by that times dQ dK sm_scale, and where 448 P~ lies that close (relative) to an
    E4M3 rounding midpoint the two sides store neighbouring P^ codes.  The oracle's margin for
    each decision is 2^-16 (FP32 rounding) plus the error bounds of the key's score and of the
    row maximum, computed from the pair's own codes and scales; the row's bound is the output
    move of one E4M3 step (at most 1/8 of the value) of every flagged key: invisible in a long
    row, up to a few 1e-2 in a short causal one.  The INT8 MFMA sums exactly (also checked by
    tests/test_gpu_probes.py), so the INT8 path needs no such margin.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from quantized_attention_amd import synthetic as sy

pytestmark = pytest.mark.gpu

ROW_ABS, MEAN_ABS, MIN_COS, COS_MATCH = 1e-2, 1e-3, 0.998, 1e-4


def check_rows(got, ref, bound, vmax):
    """got, ref: [..., rows, d]; bound: [..., rows].  Mean bar on all elements; every row within
    the max bar plus its margin bound, and within the one-step bound."""
    err = np.abs(got - ref)
    row = err.reshape(-1, err.shape[-1]).max(axis=1)
    bd = np.asarray(bound, np.float64).reshape(-1)
    over = int((row > ROW_ABS).sum())
    say(f"  rows over {ROW_ABS}: {over} of {row.size}; worst {row.max():.3g}; rows with a margin: {(bd > 0).sum()}; "
        f"worst beyond 1e-2 + margin {(row - ROW_ABS - bd).max():.3g} (one-step bound {vmax / 8:.3g})")
    assert err.mean() <= MEAN_ABS
    assert (row <= ROW_ABS + bd).all()
    assert row.max() <= vmax / 8


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_attention_amd
    quantized_attention_amd.load_library()


from tests import gpu_util as gu  # noqa: E402
from tests.test_gpu_probes import FP8_MFMA_STEP_ERR  # noqa: E402

CASES = [
    ("causal-d128-ragged", sy.CONFIGS["prefill32k"].with_shape(H=2, N=700, M=700)),
    ("noncausal-d64-smoothv", sy.CONFIGS["video17k"].with_shape(B=2, H=1, N=333, M=333)),
    ("fp16-d128-N!=M", sy.Config("fp16x", 1, 2, 300, 1000, 128, "fp16", False,
                                 sy.Dist(q_off_std=1.0, k_off_std=2.0, v_bias_std=0.5), 77)),
    ("bottom-right-N<M", sy.CONFIGS["prefill32k"].with_shape(H=2, N=300, M=1000, causal=2)),
    ("gqa-G4", sy.CONFIGS["prefill32k_gqa"].with_shape(B=1, H=8, Hkv=2, N=256, M=256)),
    ("one-token", sy.Config("one", 1, 1, 1, 1, 64, "bf16", False, sy.Dist(), 79)),
    ("few-tokens", sy.Config("few", 1, 3, 5, 3, 128, "fp16", False, sy.Dist(k_off_std=1.0), 80)),
]


def heads(cfg):
    """(b, query head h, key/value head g) for every query head."""
    G = cfg.H // cfg.hkv
    return [(bh // cfg.H, bh % cfg.H, (bh % cfg.H) // G) for bh in range(cfg.B * cfg.H)]


def vflags(cfg):
    return oracle.SMOOTH_V if cfg.smooth_v else 0


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_qk_fp8_preprocess_bit_exact(name, cfg):
    q, k, v = sy.make_qkv(cfg)
    say(f"qk-fp8 quantize {name} B={cfg.B} H={cfg.H} Hkv={cfg.hkv} N={cfg.N} M={cfg.M} d={cfg.d}")
    g = gu.quantize(q, k, v, cfg.fp16, cfg.causal, cfg.smooth_v, qk_fp8=True)
    N, M = cfg.N, cfg.M
    for bh, (b, h, gh) in enumerate(heads(cfg)):
        bk = b * cfg.hkv + gh
        o = oracle.preprocess_head(q[b, h], k[b, gh], v[b, gh], cfg.fp16, vflags(cfg) | oracle.QK_E4M3)
        assert np.array_equal(g["dq"][bh, :N].view(np.uint32), o["dq"].view(np.uint32))
        assert np.array_equal(g["q_hat"][bh, :N].view(np.uint8), o["qhat"])
        assert not g["q_hat"][bh, N:].any()
        assert np.array_equal(g["dk"][bk].view(np.uint32), o["dk"].view(np.uint32))
        assert np.array_equal(g["k_hat"][bk, :M].view(np.uint8), o["khat"])
        assert not g["k_hat"][bk, M:].any()
        assert np.array_equal(g["v_nat"][bk, :M], o["vhat"])
        assert np.array_equal(g["q_mean"][bh].view(np.uint32), o["qmean"].view(np.uint32))


def cosine(a, b):
    return float((a * b).sum() / math.sqrt((a * a).sum() * (b * b).sum()))


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_qk_fp8_forward_parity_small(name, cfg):
    q, k, v = sy.make_qkv(cfg)
    say(f"qk-fp8 forward {name} B={cfg.B} H={cfg.H} N={cfg.N} M={cfg.M} d={cfg.d} causal={cfg.causal}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, qk_fp8=True).cpu().numpy()
    s = 1 / math.sqrt(cfg.d)
    got, ref, ex, bnd = [], [], [], []
    for b, h, gh in heads(cfg):
        got.append(out[b, h].astype(np.float64))
        o, _, bd = oracle.forward_head_ties(q[b, h], k[b, gh], v[b, gh], cfg.fp16, cfg.causal, s,
                                            vflags(cfg) | oracle.QK_E4M3, qk_step_err=FP8_MFMA_STEP_ERR)
        ref.append(o)
        bnd.append(bd)
        ex.append(oracle.exact_head(q[b, h], k[b, gh], v[b, gh], cfg.fp16, cfg.causal, s))
    g, r, e = np.stack(got), np.stack(ref), np.stack(ex)
    err = np.abs(g - r)
    say(f"  max abs {err.max():.3g} mean abs {err.mean():.3g} cos(gpu, fp64) {cosine(g, e):.6f} "
        f"cos(oracle, fp64) {cosine(r, e):.6f}")
    assert np.isfinite(g).all()
    vmax = max(np.abs(sy.bits_to_f32(v, cfg.fp16)).max(), 1.0)
    check_rows(g, r, np.stack(bnd), vmax)
    if cfg.N > 8:
        assert cosine(g, e) >= MIN_COS
        assert abs(cosine(g, e) - cosine(r, e)) <= COS_MATCH


@pytest.mark.parametrize("name", ["causal-d128-ragged", "noncausal-d64-smoothv"])
def test_qk_fp8_literal_two_level(name):
    cfg = dict(CASES)[name]
    q, k, v = sy.make_qkv(cfg)
    say(f"qk-fp8 literal two-level {name}")
    a = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, acc_valu=True, qk_fp8=True).cpu().numpy()
    b = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, qk_fp8=True).cpu().numpy()
    assert np.abs(a - b).max() <= 1e-5 * max(1.0, np.abs(b).max())


@pytest.mark.parametrize("name", ["prefill32k", "video17k"])
def test_qk_fp8_full_size_sampled(name):
    cfg = sy.CONFIGS[name]
    q, k, v = sy.make_qkv(cfg)
    say(f"qk-fp8 full-size forward {name} B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} causal={cfg.causal}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, qk_fp8=True)
    BH = cfg.B * cfg.H
    s = 1 / math.sqrt(cfg.d)
    rng = np.random.default_rng(7)
    for bh in sorted({0, BH // 2, BH - 1}):
        b, h = bh // cfg.H, bh % cfg.H
        rows = np.array(sorted(set([0, 1, 127, 128, cfg.N // 2, cfg.N - 1] + list(rng.integers(0, cfg.N, 16)))))
        got = out[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        ref, _, bd = oracle.forward_head_ties(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, s,
                                              vflags(cfg) | oracle.QK_E4M3, rows=rows,
                                              qk_step_err=FP8_MFMA_STEP_ERR)
        say(f"  head {bh}:")
        check_rows(got, ref, bd, max(np.abs(sy.bits_to_f32(v[b, h], cfg.fp16)).max(), 1.0))
