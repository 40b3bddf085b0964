"""Seeded sweep over the forward's configuration space against the CPU oracle (needs an MI355X).

Each case draws, from one seeded generator, a path (INT8/FP8; the literal two-level
accumulation; E4M3 QK; MXFP4; MXFP4 with two-level P), a head dimension, batch, grouped
key/value heads (groups of 1, 2 or 3 query heads), sequence lengths (uniform, or next to a
multiple of the 128-query / 64-key tiles), the causal alignment (bottom-right only with
N <= M, as the C ABI requires), the input dtype, V smoothing and the input distribution
(per-channel offsets and spike channels of random size).  Every query head is compared
with the oracle run on (that query head, its key/value head):

  * mean |err| <= 1e-3 over the case, and every row within 1e-2 plus the oracle's bound for
    the P rounding decisions of that row which lie within 2^-16 of a boundary (where an
    FP32 kernel may round the other way), widened on the E4M3-QK path by the FP8 matrix
    core's measured score error (the bar the per-path tests use);
  * finite outputs everywhere.

The draws are fixed by the seed, so a failure names a reproducible case.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from quantized_attention_amd import synthetic as sy

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3
PATHS = {
    "int8": ({}, 0),
    "int8_acc_valu": ({"acc_valu": True}, 0),
    "qk_fp8": ({"qk_fp8": True}, oracle.QK_E4M3),
    "mxfp4": ({"mxfp4": True}, oracle.MXFP4),
    "mxfp4_p2l": ({"mxfp4": True, "mx_p_two_level": True}, oracle.MXFP4 | oracle.MX_P_TWO_LEVEL),
}
N_CASES = 30


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_attention_amd
    quantized_attention_amd.load_library()


from tests import gpu_util as gu  # noqa: E402


def _length(rng, tile):
    kind = rng.integers(3)
    if kind == 0:
        return int(rng.integers(1, 701))
    base = tile * int(rng.integers(1, 6))
    return max(1, base + int(rng.integers(-1, 2)))  # a multiple of the tile, or one off it


def draw_case(i):
    rng = np.random.default_rng(20261202 + i)
    path = sorted(PATHS)[i % len(PATHS)]
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    hkv = int(rng.integers(1, 3))
    G = int(rng.integers(1, 4))
    causal = int(rng.integers(0, 3))
    M = _length(rng, 64)
    N = _length(rng, 128)
    if causal == 2 and N > M:
        N = max(1, M - int(rng.integers(0, min(M, 200))))
    dist = sy.Dist(q_off_std=float(rng.uniform(0, 2)), k_off_std=float(rng.uniform(0, 6)),
                   k_spike=float(rng.choice([0.0, 8.0, 20.0])),
                   k_spike_channels=sy.spike_channels(d), v_bias_std=float(rng.uniform(0, 1)))
    cfg = sy.Config(f"sweep{i}", B, hkv * G, N, M, d, str(rng.choice(["bf16", "fp16"])), causal, dist,
                    1000 + i, smooth_v=bool(rng.integers(2)), Hkv=hkv)
    return path, cfg


CASES = [draw_case(i) for i in range(N_CASES)]


@pytest.mark.parametrize("i", range(N_CASES), ids=[f"{i}-{CASES[i][0]}" for i in range(N_CASES)])
def test_sweep(i):
    from tests.test_gpu_probes import FP8_MFMA_STEP_ERR
    path, cfg = CASES[i]
    kw, flags = PATHS[path]
    say(f"sweep case {i}: path={path} B={cfg.B} H={cfg.H} Hkv={cfg.hkv} N={cfg.N} M={cfg.M} d={cfg.d} "
        f"causal={cfg.causal} {cfg.dtype} smooth_v={cfg.smooth_v}")
    q, k, v = sy.make_qkv(cfg)
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, **kw).cpu().numpy().astype(np.float64)
    assert np.isfinite(out).all()
    s = 1 / math.sqrt(cfg.d)
    G = cfg.H // cfg.hkv
    errs, worst = [], -np.inf
    for b in range(cfg.B):
        for h in range(cfg.H):
            ref, _, bound = oracle.forward_head_ties(
                q[b, h], k[b, h // G], v[b, h // G], cfg.fp16, cfg.causal, s,
                flags | (oracle.SMOOTH_V if cfg.smooth_v else 0),
                qk_step_err=FP8_MFMA_STEP_ERR if path == "qk_fp8" else 0.0)
            err = np.abs(out[b, h] - ref)
            errs.append(err)
            worst = max(worst, float((err.max(axis=1) - MAX_ABS - bound).max()))
    err = np.concatenate([e.ravel() for e in errs])
    say(f"  max abs {err.max():.3g}, mean abs {err.mean():.3g}, worst row beyond 1e-2 + margin {worst:.3g}")
    assert err.mean() <= MEAN_ABS
    assert worst <= 0.0


# ---- SageBwd (sage_attn_train_forward / _backward): the same kind of draws, ungrouped heads ----
N_TRAIN = 16


def draw_train_case(i):
    rng = np.random.default_rng(20261203 + i)
    d = int(rng.choice([64, 128]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    causal = int(rng.integers(0, 3))
    M = _length(rng, 64)
    N = _length(rng, 128)
    if causal == 2 and N > M:
        N = max(1, M - int(rng.integers(0, min(M, 200))))
    dist = sy.Dist(q_off_std=float(rng.uniform(0, 2)), k_off_std=float(rng.uniform(0, 6)),
                   k_spike=float(rng.choice([0.0, 8.0])), k_spike_channels=sy.spike_channels(d),
                   v_bias_std=float(rng.uniform(0, 1)))
    cfg = sy.Config(f"train_sweep{i}", B, H, N, M, d, str(rng.choice(["bf16", "fp16"])), causal, dist, 2000 + i)
    return cfg, bool(rng.integers(4) > 0)


TRAIN_CASES = [draw_train_case(i) for i in range(N_TRAIN)]


@pytest.mark.parametrize("i", range(N_TRAIN), ids=[f"train{i}" for i in range(N_TRAIN)])
def test_train_sweep(i):
    """Forward: out within 1e-2 max / 1e-3 mean of the oracle, lse within 1e-4.  Backward: dQ, dK,
    dV within 1e-2 max(1, max |ref|) and 1e-3 max(1, mean |ref|) (the SageBwd bars)."""
    import quantized_attention_amd as qa
    cfg, smooth_k = TRAIN_CASES[i]
    say(f"train sweep case {i}: B={cfg.B} H={cfg.H} N={cfg.N} M={cfg.M} d={cfg.d} causal={cfg.causal} "
        f"{cfg.dtype} smooth_k={smooth_k}")
    q, k, v = sy.make_qkv(cfg)
    rng = np.random.default_rng(3000 + i)
    x = rng.standard_normal(q.shape).astype(np.float32)
    do = x.astype(np.float16).view(np.uint16) if cfg.fp16 else sy.f32_to_bf16_bits(x)
    tq, tk, tv, tdo = (gu.to_dev(a, cfg.fp16) for a in (q, k, v, do))
    out, lse = qa.sage_attn_train_forward(tq, tk, tv, cfg.causal, None, out_fp32=True, smooth_k=smooth_k)
    dq, dk, dv = qa.sage_attn_train_backward(tq, tk, tv, out, tdo, lse, cfg.causal, None, smooth_k=smooth_k)
    torch.cuda.synchronize()
    got = {"out": out.cpu().numpy(), "lse": lse.cpu().numpy(), "dq": dq.cpu().numpy(),
           "dk": dk.cpu().numpy(), "dv": dv.cpu().numpy()}
    s = 1 / math.sqrt(cfg.d)
    flags = 0 if smooth_k else oracle.SB_NO_SMOOTH_K
    for b in range(cfg.B):
        for h in range(cfg.H):
            ro, rl = oracle.sagebwd_forward(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, s, flags)
            eo = np.abs(got["out"][b, h].astype(np.float64) - ro)
            el = np.abs(got["lse"][b, h].astype(np.float64) - rl)
            assert np.isfinite(got["out"][b, h]).all() and np.isfinite(got["lse"][b, h]).all()
            assert eo.max() <= MAX_ABS and eo.mean() <= MEAN_ABS, (b, h, eo.max(), eo.mean())
            assert el.max() <= 1e-4, (b, h, el.max())
            ref = oracle.sagebwd_backward(q[b, h], k[b, h], v[b, h], do[b, h], cfg.fp16, cfg.causal, s, flags)
            for nm in ("dq", "dk", "dv"):
                g = got[nm][b, h].astype(np.float64)
                e = np.abs(g - ref[nm])
                assert np.isfinite(g).all(), nm
                assert e.max() <= 1e-2 * max(1.0, np.abs(ref[nm]).max()), (nm, b, h, e.max())
                assert e.mean() <= 1e-3 * max(1.0, np.abs(ref[nm]).mean()), (nm, b, h, e.mean())
