"""Direction tests: the oracle's ablation knobs reproduce the orderings and the worked
figures the pages report.  The pages measured on real model tensors that are not
available, so only directions (and, where a page works an example by hand, its figures)
are checked -- these are not parity tests.

  * "Quantization for Attention, in depth": "Worked example" (INT8 scale and level count
    before/after K smoothing) and "Simulate the error" (smoothing K halves the INT8 QK
    relative L1, about 2.5% -> 1.3%, on N(0,1) data with a +8 K channel).
  * "SageAttention2" review tables: Table 4 (smooth Q+K < Q < K < none in error), Table 6
    (per-thread ~ per-token < per-block < per-tensor), Table 7 (E4M3 < E5M2 << INT8 for
    P~ and V).
"""
import json
import os

import numpy as np
import pytest

import oracle as O
from quantized_attention_amd import synthetic as sy

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rel_l1(o, r):
    return np.abs(o - r).sum() / np.abs(r).sum()


def cosine(o, r):
    return (o * r).sum() / np.sqrt((o * o).sum() * (r * r).sum())


def test_worked_example_smoothing_k():
    g = json.load(open(os.path.join(GOLD, "qa_worked_example.json")))
    rng = np.random.default_rng(3)
    M, d = 64, 64
    K = np.stack([rng.permutation(np.linspace(-1, 1, M)) for _ in range(d)], axis=1)
    K[:, 5] = rng.permutation(np.linspace(7, 9, M))        # offset ~8, spread ~+-1
    K[:, 9] = rng.permutation(np.linspace(-0.3, 0.3, M))   # the probe channel
    k = sy.f32_to_bf16_bits(K.astype(np.float32))
    q = sy.f32_to_bf16_bits(rng.standard_normal((M, d)).astype(np.float32))
    for key, flags in (("before_smoothing", O.NO_SMOOTH_K | O.QK_PER_BLOCK), ("after_smoothing", O.QK_PER_BLOCK)):
        p = O.preprocess_head(q, k, k, False, flags)
        scale = float(p["dk"][0, 0])
        levels = int(p["khat"][:, 9].max()) - int(p["khat"][:, 9].min()) + 1
        want = g[key]
        assert abs(scale - want["scale"]) <= 0.15 * want["scale"], (key, scale)
        assert abs(levels - want["probe_levels"]) <= 0.15 * want["probe_levels"] + 1, (key, levels)


def test_simulator_smoothing_k_halves_int8_error():
    g = json.load(open(os.path.join(GOLD, "qa_simulator_expectations.json")))
    rng = np.random.default_rng(5)
    N = d = None
    N, d = 1024, 128
    x = rng.standard_normal((3, N, d)).astype(np.float32)
    x[1][:, 7] += 8.0
    q, k, v = [sy.f32_to_bf16_bits(t) for t in x]
    s = 1 / np.sqrt(d)
    ref = O.exact_head(q, k, v, False, False, s)
    base = O.QK_PER_BLOCK | O.PV_IDENTITY | O.NO_SMOOTH_Q
    e0 = rel_l1(O.forward_head(q, k, v, False, False, s, base | O.NO_SMOOTH_K), ref)
    e1 = rel_l1(O.forward_head(q, k, v, False, False, s, base), ref)
    assert e0 / e1 >= 1.5
    assert abs(e0 - g["int8_qk_rel_l1_without_smoothing"]) < 0.5 * g["int8_qk_rel_l1_without_smoothing"]
    assert abs(e1 - g["int8_qk_rel_l1_with_smooth_k"]) < 0.5 * g["int8_qk_rel_l1_with_smooth_k"]


@pytest.fixture(scope="module")
def biased_case():
    cfg = sy.CONFIGS["video17k"].with_shape(N=1024, M=1024, B=1, H=1, d=128)
    q, k, v = [a[0, 0] for a in sy.make_qkv(cfg)]
    s = 1 / np.sqrt(128)
    return q, k, v, s, O.exact_head(q, k, v, False, False, s)


def test_table4_smoothing_order(biased_case):
    q, k, v, s, ref = biased_case
    err = {}
    for name, fl in (("none", O.NO_SMOOTH_Q | O.NO_SMOOTH_K), ("K", O.NO_SMOOTH_Q), ("Q", O.NO_SMOOTH_K), ("QK", 0)):
        err[name] = rel_l1(O.forward_head(q, k, v, False, False, s, fl | O.PV_IDENTITY), ref)
    assert err["QK"] < err["Q"] < err["K"] < err["none"]


def test_table6_granularity_order(biased_case):
    q, k, v, s, ref = biased_case
    err = {}
    for name, fl in (("thread", 0), ("token", O.QK_PER_TOKEN), ("block", O.QK_PER_BLOCK), ("tensor", O.QK_PER_TENSOR)):
        err[name] = rel_l1(O.forward_head(q, k, v, False, False, s, fl | O.PV_IDENTITY), ref)
    assert err["thread"] < err["block"] < err["tensor"]
    assert err["token"] < err["block"]
    assert err["thread"] < 1.25 * err["token"]      # per-thread is close to per-token


def test_table7_pv_format_order():
    """Attention with a sink key: most P~ are ~1e-4, collectively large (the distribution
    the FP8 choice is made for); INT8 with a static 1/127 scale zeroes them."""
    rng = np.random.default_rng(6)
    N, M, d = 512, 2048, 128
    Q = rng.standard_normal((N, d)).astype(np.float32)
    K = rng.standard_normal((M, d)).astype(np.float32) * 0.5
    V = rng.standard_normal((M, d)).astype(np.float32) + rng.standard_normal(d).astype(np.float32) * 2
    Q[:, 3] += 4.0
    K[0, 3] = 24.0
    q, k, v = [sy.f32_to_bf16_bits(t) for t in (Q, K, V)]
    s = 1 / np.sqrt(d)
    ref = O.exact_head(q, k, v, False, False, s)
    err = {name: rel_l1(O.forward_head(q, k, v, False, False, s, O.QK_IDENTITY | fl), ref)
           for name, fl in (("e4m3", 0), ("e5m2", O.PV_E5M2), ("int8", O.PV_INT8))}
    assert err["e4m3"] < err["e5m2"] < err["int8"]
    assert err["int8"] > 5 * err["e5m2"]
    assert cosine(O.forward_head(q, k, v, False, False, s, O.QK_IDENTITY | O.PV_INT8), ref) < 0.99


def test_default_path_cosine_on_tiny_config():
    """The INT8/FP8 path stays above cosine 0.999 vs FP64 attention on the tiny workload."""
    cfg = sy.CONFIGS["tiny"]
    q, k, v = [a[0, 0] for a in sy.make_qkv(cfg)]
    s = 1 / np.sqrt(cfg.d)
    for causal in (False, True):
        ex = O.exact_head(q, k, v, True, causal, s)
        assert cosine(O.forward_head(q, k, v, True, causal, s), ex) >= 0.999
