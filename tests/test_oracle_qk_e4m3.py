"""Pins of the oracle's E4M3 QK knob (oracle.QK_E4M3): Q^ and K^ as OCP E4M3 with the
per-thread groups of the INT8 path and the scale amax / 448.

Source: "SageAttention2 Technical Report" summary, "Critical Assessment" (the missing ablation
of SageAttention2-8b with FP8 instead of INT8 for Q K^T) and 3.3 "FP8 Quantization for P~V"
(the E4M3 range 448 that sets the scale, as for V).

  * a lossless construction: smoothed Q and K built on the E4M3 grid times a power of two
    with every group's largest magnitude at 448 * 2^e, so the scales are exactly 2^e, the
    codes are exactly the grid values, and the forward equals textbook attention (P and V
    unquantized) and equals the identity-QK forward (P and V quantized);
  * on the synthetic prefill distribution the codes are torch's float8_e4m3fn conversion of
    the FP32 quotient and the scales follow the group maxima;
  * the knob is rejected together with the MX variant and the identity quantizer.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_attention_amd import synthetic as sy


def f16(x):
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def e4m3_grid():
    dec = oracle.e4m3_decode_table()
    return np.array([dec[c] for c in range(1, 0x7F)])  # every positive finite magnitude, 2^-9 .. 448


def qk_e4m3_lossless_case(seed, N, M, d):
    """fp16 inputs whose smoothed Q and K lie exactly on the per-token / per-group E4M3 grids.
    Keys of a group and rows of a query block come in (y, -y) pairs, so every mean is 0."""
    rng = np.random.default_rng(seed)
    grid = e4m3_grid()
    Y = np.zeros((M, d))
    eg = {}
    for u in range(-(-M // 64)):
        keys = list(range(64 * u, min(64 * u + 64, M)))
        for g in range(4):
            grp = [t for t in keys if oracle.lib().orc_k_group(t) == g]
            if not grp:
                continue
            e = int(rng.integers(-3, 1))
            eg[(u, g)] = e
            assert len(grp) % 2 == 0
            for a, b in zip(grp[0::2], grp[1::2]):
                Y[a] = rng.choice(grid, d) * rng.choice([-1.0, 1.0], d) * 2.0 ** e
                Y[a, rng.integers(d)] = 0.0
                Y[b] = -Y[a]
            Y[grp[0], rng.integers(d)] = 448.0 * 2.0 ** e
            Y[grp[1]] = -Y[grp[0]]
    Yq = np.zeros((N, d))
    er = np.zeros(N, int)
    for i in range(-(-N // 128)):
        rows = list(range(128 * i, min(128 * i + 128, N)))
        assert len(rows) % 2 == 0
        for a, b in zip(rows[0::2], rows[1::2]):
            e = int(rng.integers(-2, 1))
            n = rng.choice(grid, d) * rng.choice([-1.0, 1.0], d)
            n[rng.integers(d)] = 448.0 * rng.choice([-1.0, 1.0])
            Yq[a] = n * 2.0 ** e
            Yq[b] = -Yq[a]
            er[a] = er[b] = e
    V = rng.standard_normal((M, d)).astype(np.float16).astype(np.float64)
    assert np.array_equal(f16(Y).view(np.float16).astype(np.float64), Y)
    assert np.array_equal(f16(Yq).view(np.float16).astype(np.float64), Yq)
    return f16(Yq), f16(Y), f16(V), dict(Y=Y, eg=eg, Yq=Yq, er=er)


def decode(codes):
    dec = np.array(oracle.e4m3_decode_table())
    return dec[codes.astype(np.int64)]


@pytest.mark.parametrize("N,causal", [(200, 0), (200, 1), (256, 0)])
def test_qk_e4m3_lossless_construction(N, causal):
    d = 64
    q, k, v, c = qk_e4m3_lossless_case(30 + N, N, N, d)
    p = oracle.preprocess_head(q, k, v, fp16=True, flags=oracle.QK_E4M3)
    assert not p["kmean"].any() and not p["qmean"].any()
    for (u, g), e in c["eg"].items():
        assert p["dk"][u, g] == 2.0 ** e
    ek = np.array([c["eg"][(t // 64, oracle.lib().orc_k_group(t))] for t in range(N)])
    assert np.array_equal(decode(p["khat"]), c["Y"] / 2.0 ** ek[:, None])
    assert np.array_equal(p["dq"], (2.0 ** c["er"]).astype(np.float32))
    assert np.array_equal(decode(p["qhat"]), c["Yq"] / 2.0 ** c["er"][:, None])
    assert not p["ds"].any()
    s = 1 / 256
    ex = oracle.exact_head(q, k, v, True, causal, s)
    got = oracle.forward_head(q, k, v, True, causal, s, oracle.QK_E4M3 | oracle.PV_IDENTITY)
    assert np.abs(got - ex).max() < 1e-11
    # with P and V quantized, lossless E4M3 QK equals the identity QK exactly
    a = oracle.forward_head(q, k, v, True, causal, s, oracle.QK_E4M3)
    b = oracle.forward_head(q, k, v, True, causal, s, oracle.QK_IDENTITY)
    assert np.abs(a - b).max() < 1e-12


def test_qk_e4m3_codes_follow_torch_conversion():
    cfg = sy.CONFIGS["prefill32k"].with_shape(H=1, N=300, M=300)
    q, k, v = [x[0, 0] for x in sy.make_qkv(cfg)]
    p = oracle.preprocess_head(q, k, v, fp16=False, flags=oracle.QK_E4M3)
    K = sy.bits_to_f32(k, False)
    Q = sy.bits_to_f32(q, False)
    gk = (K - p["kmean"][None, :]).astype(np.float32)
    grp = np.array([oracle.lib().orc_k_group(t) for t in range(K.shape[0])])
    tile = np.arange(K.shape[0]) // 64
    for (u, g) in {(a, b) for a, b in zip(tile, grp)}:
        sel = (tile == u) & (grp == g)
        want = np.float32(max(np.abs(gk[sel]).max(), np.float32(1e-8))) / np.float32(448)
        assert p["dk"][u, g] == want
    dk_key = p["dk"][tile, grp]
    quot = np.clip(gk / dk_key[:, None].astype(np.float32), -448, 448).astype(np.float32)
    ref = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(p["khat"], ref)
    qm = np.repeat(p["qmean"], 128, axis=0)[:Q.shape[0]]
    gq = (Q - qm).astype(np.float32)
    dq = (np.maximum(np.abs(gq).max(axis=1), np.float32(1e-8)) / np.float32(448)).astype(np.float32)
    assert np.array_equal(p["dq"], dq)
    quot = np.clip(gq / dq[:, None], -448, 448).astype(np.float32)
    ref = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(p["qhat"], ref)
    # every group reaches the top code 448 (0x7E) in magnitude
    for u in range(tile.max() + 1):
        for g in range(4):
            sel = (tile == u) & (grp == g)
            assert ((p["khat"][sel] & 0x7F) == 0x7E).any()


def test_qk_e4m3_close_to_exact_attention():
    cfg = sy.CONFIGS["video17k"].with_shape(B=1, H=1, N=512, M=512)
    q, k, v = [x[0, 0] for x in sy.make_qkv(cfg)]
    s = 1 / math.sqrt(cfg.d)
    ex = oracle.exact_head(q, k, v, cfg.fp16, cfg.causal, s)
    got = oracle.forward_head(q, k, v, cfg.fp16, cfg.causal, s, oracle.QK_E4M3)
    cos = float((got * ex).sum() / math.sqrt((got * got).sum() * (ex * ex).sum()))
    assert cos > 0.999


def test_qk_e4m3_rejected_with_mx_and_identity():
    q = np.zeros((4, 64), np.uint16)
    for f in (oracle.MXFP4, oracle.QK_IDENTITY):
        with pytest.raises(ValueError):
            oracle.forward_head(q, q, q, False, 0, 0.1, oracle.QK_E4M3 | f)


def qk_margin_case(delta, qk_step_err):
    """Two rows Q = +-e0 and two keys K = +-e0 (d = 64): the smoothing means are 0, every code is
    +-448 with the scales 1/448, so each score is +-sm_scale and one step's largest code product
    is 448^2 for every (row, key).  A score's error bound is then e = qk_step_err x 448^2 x dQ dK x
    sm_scale (= qk_step_err sm_scale up to the FP32 rounding of 1/448), and the low key of each row
    has 448 P~ = 448 exp(-2 sm_scale); sm_scale is set so that this is 17 (1 + delta), delta above
    the E4M3 midpoint between 16 and 18.  That decision's margin is e (the key) + e (the row
    maximum)."""
    Q = np.zeros((2, 64)); Q[0, 0], Q[1, 0] = 1.0, -1.0
    K = Q.copy()
    V = np.zeros((2, 64)); V[:, 0] = [1.0, 2.0]
    sm = -math.log(17 * (1 + delta) / 448) / 2
    out, ties, bound = oracle.forward_head_ties(f16(Q), f16(K), f16(V), True, 0, sm, oracle.QK_E4M3,
                                                tie_eps=1e-12, qk_step_err=qk_step_err)
    return ties, 2 * qk_step_err * sm


def test_qk_margin_widens_by_the_score_errors():
    eps = 2.0 ** -10
    _, e2 = qk_margin_case(0.0, eps)  # twice the per-score bound, for this sm_scale
    for frac, flagged in ((0.9, 1), (1.1, 0)):
        ties, e2 = qk_margin_case(frac * e2, eps)
        assert (ties == flagged).all(), (frac, ties)
    ties, _ = qk_margin_case(0.5 * e2, 0.0)  # no kernel error model: no margin beyond tie_eps
    assert (ties == 0).all()


@pytest.mark.parametrize("old,new", [
    ("  return qk_step_err * e * (double)h->dq[r] * (double)h->dk_key[t] * sm_scale;",
     "  return qk_step_err * e * (double)h->dk_key[t] * sm_scale;"),
    ("tie_eps + (qk_err ? E[x] + emax : 0.0)", "tie_eps + (qk_err ? E[x] : 0.0)"),
])
def test_qk_margin_catches_planted_mistake(old, new):
    with oracle.planted_mistake(("sage_oracle.c", old, new)):
        with pytest.raises(AssertionError):
            test_qk_margin_widens_by_the_score_errors()
