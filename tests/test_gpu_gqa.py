"""GPU checks of grouped key/value heads (sage_attn_fwd_ex / sage_attn_quantize_ex with
Hkv < Hq; needs an MI355X).

Grouped heads are the plain extension of the method: query head h attends with key/value
head h // (Hq // Hkv), every per-head quantity keeps its owner (K mean, V_m, K^, V^ and
their scales: the key/value head; Q block means, Q^, its scales and Delta S: the query
head).  So
  * the output equals, bit for bit, the output of ungrouped attention on K and V with each
    key/value head repeated for its query heads (same kernels, same per-head data);
  * each query head matches the oracle run on (that query head, its key/value head) within
    the usual bars (max |err| <= 1e-2, mean <= 1e-3, FP32 output);
  * the quantize views hold the key/value-side tensors once per key/value head, bit-exact.
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


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_attention_amd
    quantized_attention_amd.load_library()


from tests import gpu_util as gu  # noqa: E402

BASE = sy.CONFIGS["prefill32k_gqa"]
CASES = [
    ("causal-d128-G4", BASE.with_shape(B=2, H=8, Hkv=2, N=300, M=300)),
    ("noncausal-d64-G2-smoothv", sy.CONFIGS["video17k"].with_shape(B=1, H=4, Hkv=2, N=333, M=333)),
    ("bottom-right-G8", BASE.with_shape(B=1, H=8, Hkv=1, N=200, M=700, causal=2)),
    ("mx-G4", sy.CONFIGS["mxfp4_32k"].with_shape(B=1, H=8, Hkv=2, N=256, M=400)),
]


def kv_of(cfg, bh):
    G = cfg.H // cfg.hkv
    b, h = bh // cfg.H, bh % cfg.H
    return b, h, h // G


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_grouped_equals_repeated_kv(name, cfg):
    q, k, v = sy.make_qkv(cfg)
    G = cfg.H // cfg.hkv
    say(f"gqa vs repeated {name} B={cfg.B} H={cfg.H} Hkv={cfg.hkv} N={cfg.N} M={cfg.M}")
    grouped = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, mxfp4=cfg.mxfp4)
    rep = gu.fwd(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), cfg.fp16, cfg.causal, None, cfg.smooth_v,
                 mxfp4=cfg.mxfp4)
    assert torch.equal(grouped.view(torch.int32), rep.view(torch.int32))


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_grouped_parity_vs_oracle(name, cfg):
    q, k, v = sy.make_qkv(cfg)
    say(f"gqa forward {name}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, mxfp4=cfg.mxfp4).cpu().numpy()
    flags = (oracle.SMOOTH_V if cfg.smooth_v else 0) | (oracle.MXFP4 if cfg.mxfp4 else 0)
    s = 1 / math.sqrt(cfg.d)
    errs = []
    for bh in range(cfg.B * cfg.H):
        b, h, g = kv_of(cfg, bh)
        ref = oracle.forward_head(q[b, h], k[b, g], v[b, g], cfg.fp16, cfg.causal, s, flags)
        errs.append(np.abs(out[b, h].astype(np.float64) - ref))
    e = np.stack(errs)
    say(f"  max abs {e.max():.3g} mean abs {e.mean():.3g}")
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS


def test_grouped_quantize_views():
    cfg = CASES[0][1]
    q, k, v = sy.make_qkv(cfg)
    say("gqa quantize views")
    g = gu.quantize(q, k, v, cfg.fp16, cfg.causal, cfg.smooth_v)
    N, M = cfg.N, cfg.M
    assert g["k_hat"].shape[0] == cfg.B * cfg.hkv and g["q_hat"].shape[0] == cfg.B * cfg.H
    for bh in range(cfg.B * cfg.H):
        b, h, gh = kv_of(cfg, bh)
        bk = b * cfg.hkv + gh
        o = oracle.preprocess_head(q[b, h], k[b, gh], v[b, gh], cfg.fp16, 0)
        assert np.array_equal(g["q_hat"][bh, :N], o["qhat"])
        assert np.array_equal(g["dq"][bh, :N].view(np.uint32), o["dq"].view(np.uint32))
        assert np.array_equal(g["q_mean"][bh].view(np.uint32), o["qmean"].view(np.uint32))
        assert np.array_equal(g["k_hat"][bk, :M], o["khat"])
        assert np.array_equal(g["dk"][bk].view(np.uint32), o["dk"].view(np.uint32))
        assert np.array_equal(g["k_mean"][bk].view(np.uint32), o["kmean"].view(np.uint32))
        assert np.array_equal(g["v_nat"][bk, :M], o["vhat"])
        ds, ref = g["delta_s"][bh][:, :M].astype(np.float64), o["ds"]
        tile0 = 64 * (np.arange(M) // 64)
        mask = tile0[None, :] < 128 * (np.arange(ds.shape[0])[:, None] + 1)
        assert np.abs(ds[mask] - ref[mask]).max() <= 1e-5 * max(1.0, np.abs(ref).max())


def test_grouped_full_size_sampled():
    cfg = sy.CONFIGS["prefill32k_gqa"]
    q, k, v = sy.make_qkv(cfg)
    say(f"gqa full-size forward B={cfg.B} H={cfg.H} Hkv={cfg.hkv} N={cfg.N} causal={cfg.causal}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v)
    s = 1 / math.sqrt(cfg.d)
    rng = np.random.default_rng(11)
    for bh in sorted({0, 5, cfg.B * cfg.H - 1}):
        b, h, g = kv_of(cfg, bh)
        rows = np.array(sorted(set([0, 127, 128, cfg.N // 2, cfg.N - 1] + list(rng.integers(0, cfg.N, 12)))))
        got = out[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        ref = oracle.forward_head(q[b, h], k[b, g], v[b, g], cfg.fp16, cfg.causal, s, 0, rows=rows)
        err = np.abs(got - ref)
        say(f"  head {bh} (kv {b * cfg.hkv + g}): max abs {err.max():.3g}")
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
