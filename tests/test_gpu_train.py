"""GPU parity of SageBwd, the trainable INT8 attention (sage_attn_train_fwd / _bwd), against the
CPU oracle (needs an MI355X).

Source: "SageAttention3: Microscaling FP4 Attention for Inference and An Exploration of
8-Bit Training" summary, "SageBwd Forward Pass: INT8 Quantization for Training" and "SageBwd
Backward Pass and the Critical dOV^T Decision".

Bars (FP32 outputs):
  * forward: out within max |err| <= 1e-2 and mean |err| <= 1e-3 of the oracle; the
    log-sum-exp within 1e-4 (its scores carry only FP32 rounding against the oracle's exact
    integer dot products, and P^ rounds against the row's block max on both sides);
  * backward: dQ, dK, dV within max |err| <= 1e-2 max(1, max |ref|) and mean |err| <=
    1e-3 max(1, mean |ref|) of the oracle (the gradients' scale varies with the inputs; the
    two sides differ by FP32 against FP64 rounding of S, L, dP and D, and by the rare P^ /
    dS^ code that this moves across a rounding midpoint); the autograd wrapper returns the
    same gradients in the input dtype.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from quantized_attention_amd import synthetic as sy

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 1e-2, 1e-3, 1e-4


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_attention_amd
    quantized_attention_amd.load_library()


import quantized_attention_amd as qa  # noqa: E402
from tests import gpu_util as gu  # noqa: E402

CASES = [
    ("causal-d128-ragged", sy.CONFIGS["prefill32k"].with_shape(H=2, N=300, M=300), True),
    ("noncausal-d64", sy.CONFIGS["video17k"].with_shape(B=2, H=1, N=333, M=333), True),
    ("fp16-d128-N!=M", sy.Config("fp16x", 1, 2, 200, 500, 128, "fp16", False,
                                 sy.Dist(q_off_std=1.0, k_off_std=2.0, v_bias_std=0.5), 77), True),
    ("bottom-right", sy.CONFIGS["prefill32k"].with_shape(H=2, N=100, M=300, causal=2), True),
    ("no-smooth-k", sy.CONFIGS["n4k"].with_shape(H=2, N=256, M=256), False),
    ("one-token", sy.Config("one", 1, 1, 1, 1, 64, "bf16", False, sy.Dist(), 79), True),
]


def train_fwd(cfg, q, k, v, smooth_k):
    tq, tk, tv = gu.to_dev(q, cfg.fp16), gu.to_dev(k, cfg.fp16), gu.to_dev(v, cfg.fp16)
    out, lse = qa.sage_attn_train_forward(tq, tk, tv, cfg.causal, None, out_fp32=True, smooth_k=smooth_k)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("name,cfg,smooth_k", CASES, ids=[c[0] for c in CASES])
def test_train_forward_parity(name, cfg, smooth_k):
    q, k, v = sy.make_qkv(cfg)
    say(f"train forward {name} B={cfg.B} H={cfg.H} N={cfg.N} M={cfg.M} d={cfg.d} causal={cfg.causal}")
    out, lse = train_fwd(cfg, q, k, v, smooth_k)
    s = 1 / math.sqrt(cfg.d)
    flags = 0 if smooth_k else oracle.SB_NO_SMOOTH_K
    eo, el = [], []
    for bh in range(cfg.B * cfg.H):
        b, h = bh // cfg.H, bh % cfg.H
        ro, rl = oracle.sagebwd_forward(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, s, flags)
        eo.append(np.abs(out[b, h].astype(np.float64) - ro).ravel())
        el.append(np.abs(lse[b, h].astype(np.float64) - rl))
    eo, el = np.concatenate(eo), np.concatenate(el)
    say(f"  out max {eo.max():.3g} mean {eo.mean():.3g}; lse max {el.max():.3g}")
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert eo.max() <= MAX_ABS and eo.mean() <= MEAN_ABS
    assert el.max() <= LSE_ABS


def rand_bits(shape, fp16, seed):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return x.astype(np.float16).view(np.uint16) if fp16 else sy.f32_to_bf16_bits(x)


def rel_err(got, ref):
    e = np.abs(got.astype(np.float64) - ref)
    return e.max() / max(1.0, np.abs(ref).max()), e.mean() / max(1.0, np.abs(ref).mean())


@pytest.mark.parametrize("recompute", [False, True], ids=["stored_ds", "recomputed_ds"])
@pytest.mark.parametrize("name,cfg,smooth_k", CASES, ids=[c[0] for c in CASES])
def test_train_backward_parity(name, cfg, smooth_k, recompute):
    q, k, v = sy.make_qkv(cfg)
    do = rand_bits(q.shape, cfg.fp16, 41)
    say(f"train backward {name} B={cfg.B} H={cfg.H} N={cfg.N} M={cfg.M} d={cfg.d} causal={cfg.causal} "
        f"recompute_ds={recompute}")
    tq, tk, tv, tdo = (gu.to_dev(x, cfg.fp16) for x in (q, k, v, do))
    out, lse = qa.sage_attn_train_forward(tq, tk, tv, cfg.causal, None, out_fp32=True, smooth_k=smooth_k)
    dq, dk, dv = qa.sage_attn_train_backward(tq, tk, tv, out, tdo, lse, cfg.causal, None, smooth_k=smooth_k,
                                             recompute_ds=recompute)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    s = 1 / math.sqrt(cfg.d)
    flags = 0 if smooth_k else oracle.SB_NO_SMOOTH_K
    worst = {}
    for bh in range(cfg.B * cfg.H):
        b, h = bh // cfg.H, bh % cfg.H
        ref = oracle.sagebwd_backward(q[b, h], k[b, h], v[b, h], do[b, h], cfg.fp16, cfg.causal, s, flags)
        ex = oracle.sagebwd_backward(q[b, h], k[b, h], v[b, h], do[b, h], cfg.fp16, cfg.causal, s,
                                     flags | oracle.SB_IDENTITY)
        for nm, got in (("dq", dq[b, h]), ("dk", dk[b, h]), ("dv", dv[b, h])):
            mx, mn = rel_err(got, ref[nm])
            g = got.astype(np.float64).ravel()
            e = ex[nm].ravel()
            cos = float((g * e).sum() / max(1e-300, math.sqrt((g * g).sum() * (e * e).sum())))
            w = worst.setdefault(nm, [0.0, 0.0, 1.0])
            w[0], w[1], w[2] = max(w[0], mx), max(w[1], mn), min(w[2], cos)
    for nm, (mx, mn, cos) in worst.items():
        say(f"  {nm}: max rel {mx:.3g} mean rel {mn:.3g} cos vs exact {cos:.5f}")
        assert np.isfinite(mx) and mx <= 1e-2 and mn <= 1e-3, nm


@pytest.mark.parametrize("name,cfg,smooth_k", CASES, ids=[c[0] for c in CASES])
def test_stored_and_recomputed_ds_agree(name, cfg, smooth_k):
    """The two backward forms compute the same dS^ codes: dK and dV bit-identical; dQ equal up to the
    FP32 order of the K-mean term's row sums (bit-identical without K smoothing)."""
    q, k, v = sy.make_qkv(cfg)
    do = rand_bits(q.shape, cfg.fp16, 43)
    tq, tk, tv, tdo = (gu.to_dev(x, cfg.fp16) for x in (q, k, v, do))
    out, lse = qa.sage_attn_train_forward(tq, tk, tv, cfg.causal, None, out_fp32=True, smooth_k=smooth_k)
    a = qa.sage_attn_train_backward(tq, tk, tv, out, tdo, lse, cfg.causal, None, smooth_k=smooth_k)
    b = qa.sage_attn_train_backward(tq, tk, tv, out, tdo, lse, cfg.causal, None, smooth_k=smooth_k,
                                    recompute_ds=True)
    torch.cuda.synchronize()
    (dqa, dka, dva), (dqb, dkb, dvb) = ([t.cpu().numpy() for t in x] for x in (a, b))
    assert np.array_equal(dka, dkb) and np.array_equal(dva, dvb)
    if smooth_k:
        assert np.abs(dqa.astype(np.float64) - dqb).max() <= 1e-5 * max(1.0, np.abs(dqb).max())
    else:
        assert np.array_equal(dqa, dqb)


@pytest.mark.parametrize("recompute", [False, True], ids=["stored_ds", "recomputed_ds"])
@pytest.mark.parametrize("name,cfg,smooth_k", CASES, ids=[c[0] for c in CASES])
def test_kept_quantization_gives_identical_results(name, cfg, smooth_k, recompute):
    """SAGE_TRAIN_KEEP_QUANT: the forward leaves its INT8 Q, K, V in the step's workspace and the
    backward takes them from there instead of quantizing again; the same codes, so out, lse, dq,
    dk and dv are bit-identical to the two calls without it."""
    q, k, v = sy.make_qkv(cfg)
    do = rand_bits(q.shape, cfg.fp16, 47)
    tq, tk, tv, tdo = (gu.to_dev(x, cfg.fp16) for x in (q, k, v, do))
    say(f"kept quantization {name} recompute={recompute}")
    o1, l1 = qa.sage_attn_train_forward(tq, tk, tv, cfg.causal, None, out_fp32=True, smooth_k=smooth_k)
    g1 = qa.sage_attn_train_backward(tq, tk, tv, o1, tdo, l1, cfg.causal, None, smooth_k=smooth_k,
                                     recompute_ds=recompute)
    o2, l2, ctx = qa.sage_attn_train_forward(tq, tk, tv, cfg.causal, None, out_fp32=True, smooth_k=smooth_k,
                                             keep=True)
    g2 = qa.sage_attn_train_backward(tq, tk, tv, o2, tdo, l2, cfg.causal, None, smooth_k=smooth_k,
                                     recompute_ds=recompute, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_train_full_size():
    """The train8k workload (B=1 H=32 N=M=8192 d=128 bf16 causal) in the launch configuration the
    benchmark times, FP32 outputs: the forward (out, lse) and all three gradients of the first
    and the last head against the oracle, whole heads, to the bars above."""
    cfg = sy.CONFIGS["train8k"]
    q, k, v = sy.make_qkv(cfg)
    do = rand_bits(q.shape, cfg.fp16, 45)
    say(f"train full size B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} causal={cfg.causal}")
    tq, tk, tv, tdo = (gu.to_dev(x, cfg.fp16) for x in (q, k, v, do))
    out, lse = qa.sage_attn_train_forward(tq, tk, tv, cfg.causal, None, out_fp32=True)
    dq, dk, dv = qa.sage_attn_train_backward(tq, tk, tv, out, tdo, lse, cfg.causal, None)
    torch.cuda.synchronize()
    s = 1 / math.sqrt(cfg.d)
    for h in (0, cfg.H - 1):
        ref = oracle.sagebwd_backward(q[0, h], k[0, h], v[0, h], do[0, h], cfg.fp16, cfg.causal, s)
        o = out[0, h].cpu().numpy().astype(np.float64)
        err = np.abs(o - ref["out"])
        lerr = np.abs(lse[0, h].cpu().numpy().astype(np.float64) - ref["lse"]).max()
        say(f"  head {h}: out max {err.max():.3g} mean {err.mean():.3g}; lse {lerr:.3g}")
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS and lerr <= LSE_ABS
        for nm, got in (("dq", dq[0, h]), ("dk", dk[0, h]), ("dv", dv[0, h])):
            mx, mn = rel_err(got.cpu().numpy(), ref[nm])
            say(f"  head {h} {nm}: max rel {mx:.3g} mean rel {mn:.3g}")
            assert np.isfinite(mx) and mx <= 1e-2 and mn <= 1e-3, nm


def test_train_autograd_function():
    cfg = sy.CONFIGS["prefill32k"].with_shape(H=2, N=200, M=200)
    q, k, v = sy.make_qkv(cfg)
    do = rand_bits(q.shape, cfg.fp16, 43)
    tq, tk, tv, tdo = (gu.to_dev(x, cfg.fp16) for x in (q, k, v, do))
    say("train autograd function")
    leaves = [t.clone().requires_grad_(True) for t in (tq, tk, tv)]
    out = qa.SageBwdAttention.apply(*leaves, 1, None)
    out.backward(tdo)
    o2, lse = qa.sage_attn_train_forward(tq, tk, tv, 1, None)
    dq, dk, dv = qa.sage_attn_train_backward(tq, tk, tv, o2, tdo, lse, 1, None)
    torch.cuda.synchronize()
    assert torch.equal(out, o2)
    for leaf, ref in zip(leaves, (dq, dk, dv)):
        assert leaf.grad.dtype == leaf.dtype
        assert torch.equal(leaf.grad, ref.to(leaf.dtype))

