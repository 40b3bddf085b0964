"""Pins of the SageBwd oracle (oracle.sagebwd_forward / sagebwd_backward / sagebwd_quantize).

Source: "SageAttention3: Microscaling FP4 Attention for Inference and An Exploration of
8-Bit Training" summary, "SageBwd Forward Pass: INT8 Quantization for Training" and
"SageBwd Backward Pass and the Critical dOV^T Decision".

  * identity quantizers: the forward and all three gradients equal torch's FP64 autograd of
    textbook attention (causal alignments, ragged blocks, N != M, d 64/128); the log-sum-exp
    equals torch's after the K-smoothing shift;
  * closed forms that exercise every quantizer scale: one key per row (P = 1, dQ = dK = 0,
    dV = column sums of dO), two keys with equal scores (dS = +-a, dQ = 2 a sm w, dK = +-a sm q,
    L = ln 2), the backward's per-block P^ (a split row beside a peaked row of its block) and
    the forward's P scale taken from the row's block maximum;
  * a lossless construction for the exported codes (Q and dO per 128 rows, K and V per 64
    keys, scales 2^e);
  * the quantized method close to exact attention on zero-mean dO (a sanity bound).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_attention_amd import synthetic as sy


def f16(x):
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def widen(bits, fp16):
    return sy.bits_to_f32(bits, fp16).astype(np.float64)


def torch_reference(q, k, v, do, fp16, causal, sm):
    Q, K, V, dO = (torch.tensor(widen(x, fp16), dtype=torch.float64, requires_grad=i < 3)
                   for i, x in enumerate((q, k, v, do)))
    S = sm * Q @ K.T
    N, M = S.shape
    if causal:
        off = M - N if causal == 2 else 0
        mask = torch.arange(M)[None, :] > torch.arange(N)[:, None] + off
        S = S.masked_fill(mask, float("-inf"))
    lse = torch.logsumexp(S, dim=-1)
    O = torch.softmax(S, dim=-1) @ V
    (O * dO).sum().backward()
    return dict(out=O.detach().numpy(), lse=lse.detach().numpy(), dq=Q.grad.numpy(), dk=K.grad.numpy(),
                dv=V.grad.numpy())


SHAPES = [(200, 333, 64, 0, True), (300, 300, 128, 1, False), (130, 500, 64, 2, True), (1, 7, 128, 0, False),
          (65, 65, 64, 1, True), (260, 70, 128, 1, False)]


@pytest.mark.parametrize("N,M,d,causal,fp16", SHAPES)
def test_identity_equals_torch_autograd(N, M, d, causal, fp16):
    cfg = sy.Config("t", 1, 1, N, M, d, "fp16" if fp16 else "bf16", causal,
                    sy.Dist(q_off_std=1.0, k_off_std=3.0, v_bias_std=0.5), 5000 + N)
    q, k, v = [x[0, 0] for x in sy.make_qkv(cfg)]
    do = f16(np.random.default_rng(N).standard_normal((N, d))) if fp16 else \
        sy.f32_to_bf16_bits(np.random.default_rng(N).standard_normal((N, d)).astype(np.float32))
    sm = 1 / math.sqrt(d)
    got = oracle.sagebwd_backward(q, k, v, do, fp16, causal, sm, oracle.SB_IDENTITY)
    ref = torch_reference(q, k, v, do, fp16, causal, sm)
    for name in ("out", "dq", "dk", "dv"):
        scale = max(1.0, np.abs(ref[name]).max())
        assert np.abs(got[name] - ref[name]).max() <= 1e-10 * scale, name
    # L is taken after K smoothing: it differs from torch's by sm * q . kmean per row
    kmean = oracle.sagebwd_quantize(q, k, v, None, fp16)["kmean"].astype(np.float64)
    assert np.abs(got["lse"] - (ref["lse"] - sm * widen(q, fp16) @ kmean)).max() <= 1e-10 * max(1, np.abs(ref["lse"]).max())
    nosm = oracle.sagebwd_backward(q, k, v, do, fp16, causal, sm, oracle.SB_IDENTITY | oracle.SB_NO_SMOOTH_K)
    assert np.abs(nosm["lse"] - ref["lse"]).max() <= 1e-10 * max(1, np.abs(ref["lse"]).max())
    assert np.abs(nosm["dq"] - ref["dq"]).max() <= 1e-10 * max(1, np.abs(ref["dq"]).max())


def grid_rows(rng, T, d, e, peak=True):
    """Rows on the INT8 grid of scale 2^e (integers up to 127 times 2^e), one 127 per block."""
    n = rng.integers(-100, 101, (T, d)).astype(np.float64)
    if peak:
        n[0, rng.integers(d)] = 127
    return n * 2.0 ** e


def test_single_key_closed_form():
    """M = 1: P = 1 for every row, so out = v, dQ = dK = 0 and dV = sum of dO."""
    rng = np.random.default_rng(1)
    N, d = 100, 64
    q = f16(rng.integers(-8, 9, (N, d)))
    k = f16(rng.integers(-8, 9, (1, d)))
    v = f16(grid_rows(rng, 1, d, -4))
    do = f16(grid_rows(rng, N, d, -6))
    o = oracle.sagebwd_backward(q, k, v, do, True, 0, 0.125)
    V, dO = widen(v, True), widen(do, True)
    assert np.abs(o["out"] - V).max() <= 1e-14
    assert np.abs(o["lse"] - 0.125 * widen(q, True) @ (widen(k, True)[0] - widen(k, True)[0])).max() == 0  # S' = 0
    assert np.abs(o["dq"]).max() <= 1e-12 and np.abs(o["dk"]).max() <= 1e-12
    assert np.abs(o["dv"][0] - dO.sum(axis=0)).max() <= 1e-12


def test_two_equal_score_keys_closed_form():
    """N = 1, K' = +-w with w orthogonal to q: P = 1/2 each, dS = +-a, a = (dO.(v1 - v2)) / 4."""
    rng = np.random.default_rng(2)
    d, sm = 64, 0.25
    qv = np.zeros(d); qv[0] = 127 * 2.0 ** -3
    w = np.zeros(d); w[1:] = rng.integers(-20, 21, d - 1); w[5] = 127  # w . q = 0, on the grid of scale 1
    kbar = rng.integers(-4, 5, d).astype(np.float64)
    K = np.stack([kbar + w, kbar - w])
    V = grid_rows(rng, 2, d, -5)
    dO = grid_rows(rng, 1, d, -2)
    q, k, v, do = f16(qv[None]), f16(K), f16(V), f16(dO)
    o = oracle.sagebwd_backward(q, k, v, do, True, 0, sm)
    assert np.abs(o["out"][0] - V.mean(axis=0)).max() <= 1e-13
    assert abs(o["lse"][0] - math.log(2)) <= 1e-15
    a = dO[0] @ (V[0] - V[1]) / 4
    assert np.abs(o["dv"] - 0.5 * dO[0][None, :]).max() <= 1e-13
    assert np.abs(o["dq"][0] - 2 * sm * a * w).max() <= 1e-12 * max(1, abs(a) * 127)
    assert np.abs(o["dk"][0] - sm * a * qv).max() <= 1e-12 * max(1, abs(a) * 16)
    assert np.abs(o["dk"][1] + sm * a * qv).max() <= 1e-12 * max(1, abs(a) * 16)


def test_smoothing_k_term_of_dq_closed_form():
    """The smoothing-K term of dQ, sm rowsum(dS) k, in isolation.  N = 1, two keys
    kbar +- w with w along channel 0 only and kbar = 8 on channel 1 (so gamma K and K^ are 0
    there): the main term sm dS^ K^ contributes nothing to dQ[1], and
    dQ[1] = sm * 8 * rowsum(dS).  The backward's P = exp(S - L) sums to 1 and dP = dO V^T is
    exact on 16-bit inputs, so rowsum(dS) = dO . O_exact - D with D = dO . O from the forward,
    whose INT8 P^ is lossy here (127 e^-delta is not an integer).  O_exact is numpy's softmax
    of the scores times V.  Dropping the term, its sign or its sm_scale fails this."""
    rng = np.random.default_rng(3)
    d, sm = 64, 0.2
    qv = np.zeros(d); qv[0] = 127 * 2.0 ** -7
    w = np.zeros(d); w[0] = 127 * 2.0 ** -6  # scales 2^-7, 2^-6: exact; P~ ratio e^-(2 sm q0 w0), lossy in INT8
    kbar = np.zeros(d); kbar[1] = 8.0
    K = np.stack([kbar + w, kbar - w])
    V = grid_rows(rng, 2, d, -5)
    dO = grid_rows(rng, 1, d, -2)
    q, k, v, do = f16(qv[None]), f16(K), f16(V), f16(dO)
    o = oracle.sagebwd_backward(q, k, v, do, True, 0, sm)
    s = sm * (K @ qv)
    p = np.exp(s - s.max())
    o_exact = (p / p.sum()) @ V
    rs = dO[0] @ o_exact - dO[0] @ o["out"][0]
    assert abs(rs) > 1e-4  # the forward's P^ is lossy: the term does not vanish
    # rowsum(dS) is a difference of terms near D (~3e2 here), so FP64 rounding leaves ~1e-13 on it
    assert abs(o["dq"][0, 1] - sm * 8.0 * rs) <= 1e-9 * abs(sm * 8.0 * rs)


def test_backward_p_scale_is_per_block():
    """Rows 0 (peaked, P ~ [1, 0]) and 1 (split, P = [1/2, 1/2]) share one block: the split row's
    P^ is coded against the block max P_00, so 0.5 becomes rne(63.5 / P_00) * P_00 / 127."""
    d, sm = 64, 1.0
    a, b, c = 127 / 32, 127 / 64, 127 / 128  # magnitudes 127 * 2^e: every block scale is 2^e
    w = np.zeros(d); w[1] = a
    q0 = np.zeros(d); q0[1] = b            # S_0 = +-a b
    q1 = np.zeros(d); q1[2] = b            # S_1 = 0, 0
    K = np.stack([w, -w])                  # mean 0
    dO = np.zeros((2, d)); dO[0, 3] = c; dO[1, 4] = c
    V = np.eye(2, d)
    q, k, v, do = f16(np.stack([q0, q1])), f16(K), f16(V), f16(dO)
    o = oracle.sagebwd_backward(q, k, v, do, True, 0, sm)
    e = math.exp(-2 * a * b)
    P = np.array([[1 / (1 + e), e / (1 + e)], [0.5, 0.5]])
    sp = P.max() / 127
    Ph = np.round(P / sp) * sp             # no ties here (63.5 / P_00 > 63.5)
    want = Ph.T @ dO                       # dV = P^^T dO (dO exact on its grid)
    assert np.abs(o["dv"] - want).max() <= 1e-15
    assert abs(o["dv"][0, 4] - 64 * P.max() / 127 * c) <= 1e-15  # not the per-row 0.5 c


def test_forward_p_scale_from_block_row_max():
    """One row, keys in two 64-key blocks: block 0 holds the row max, block 1's largest P is
    e^-(S_0 - S_64) < 1.  Block 1 is coded against its own max (-> 127), not the static 1/127."""
    d, M, sm = 64, 128, 1.0
    rng = np.random.default_rng(4)
    q = np.zeros((1, d)); q[0, 0] = 127 / 128        # every block scale below is a power of two
    K = np.zeros((M, d))
    K[0, 0] = 127 / 64            # block 0: the row max
    K[64, 0] = 127 / 128          # block 1: its max, and one more key
    K[65, 0] = 64 / 128
    V = np.zeros((M, d)); V[:, 2] = rng.integers(-100, 101, M) / 32
    V[0, 2] = V[64, 2] = 127 / 32
    o, lse = oracle.sagebwd_forward(f16(q), f16(K), f16(V), True, 0, sm, oracle.SB_NO_SMOOTH_K)
    s = q[0, 0] * K[:, 0]         # scores: Q, K and V are exact on their grids
    p = np.exp(s - s.max())
    ph = np.empty(M)
    for j in range(2):
        blk = slice(64 * j, 64 * j + 64)
        sp = p[blk].max() / 127
        ph[blk] = np.round(p[blk] / sp) * sp
    want = (ph * V[:, 2]).sum() / p.sum()
    assert abs(o[0, 2] - want) <= 1e-13
    assert abs(lse[0] - (s.max() + math.log(p.sum()))) <= 1e-13
    static = np.round(p * 127) / 127          # the static 1/127 scale the pages reject
    assert abs((static * V[:, 2]).sum() / p.sum() - want) > 1e-5


def test_quantize_lossless_construction():
    rng = np.random.default_rng(3)
    N, M, d = 300, 200, 128
    eq = [-3, -5, -2]                  # per 128-row block
    ek = [-4, -1, -6, -2]              # per 64-key block
    Q = np.concatenate([grid_rows(rng, min(128, N - 128 * i), d, eq[i]) for i in range(3)])
    Ky = np.concatenate([grid_rows(rng, min(64, M - 64 * j), d, ek[j]) for j in range(4)])
    Ky = np.concatenate([Ky[:100], -Ky[:100]])                 # mean exactly 0
    Ky = Ky * 1.0
    V = np.concatenate([grid_rows(rng, min(64, M - 64 * j), d, ek[j] - 1) for j in range(4)])
    dO = np.concatenate([grid_rows(rng, min(128, N - 128 * i), d, eq[i] - 2) for i in range(3)])
    o = oracle.sagebwd_quantize(f16(Q), f16(Ky), f16(V), f16(dO), True)
    assert np.array_equal(o["sq"], np.float32(2.0) ** np.array(eq, np.float32))
    assert np.array_equal(o["qcode"].astype(np.float64), Q / np.repeat(2.0 ** np.array(eq), 128)[:N, None])
    assert np.array_equal(o["sdo"], np.float32(2.0) ** np.array(eq, np.float32) / 4)
    assert np.array_equal(o["docode"].astype(np.float64), dO / np.repeat(2.0 ** (np.array(eq) - 2), 128)[:N, None])
    assert not o["kmean"].any()
    amax = np.array([np.abs(Ky[64 * j:64 * j + 64]).max() for j in range(4)])
    assert np.array_equal(o["sk"], (amax.astype(np.float32) / np.float32(127)))
    assert np.array_equal(o["vcode"].astype(np.float64), V / np.repeat(2.0 ** (np.array(ek) - 1), 64)[:M, None])


def test_quantized_close_to_exact():
    """The quantized method stays close to exact attention and its gradients on zero-mean dO
    (a sanity bound, not a pin: the pages report accuracy on real tensors only).  The INT8
    dO V^T ablation runs; its direction against the 16-bit form depends on the inputs here
    (D = rowsum(dO o O) takes the quantized forward's O, which the pages' form keeps)."""
    cfg = sy.CONFIGS["video17k"].with_shape(B=1, H=1, N=512, M=512)
    q, k, v = [x[0, 0] for x in sy.make_qkv(cfg)]
    do = sy.f32_to_bf16_bits(np.random.default_rng(9).standard_normal((512, cfg.d)).astype(np.float32))
    sm = 1 / math.sqrt(cfg.d)
    ex = oracle.sagebwd_backward(q, k, v, do, False, 0, sm, oracle.SB_IDENTITY)
    a = oracle.sagebwd_backward(q, k, v, do, False, 0, sm)
    b = oracle.sagebwd_backward(q, k, v, do, False, 0, sm, oracle.SB_DP_INT8)

    def cos(x, y):
        return float((x * y).sum() / math.sqrt((x * x).sum() * (y * y).sum()))

    for name in ("out", "dq", "dk", "dv"):
        assert cos(a[name], ex[name]) > 0.99, name
        assert cos(b[name], ex[name]) > 0.98, name
    assert np.array_equal(a["dv"], b["dv"]) and np.array_equal(a["out"], b["out"])  # dV, out do not use dP


def test_arguments_rejected():
    z = np.zeros((4, 64), np.uint16)
    with pytest.raises(ValueError):
        oracle.sagebwd_forward(z, z, z, False, 3, 0.1)
    with pytest.raises(ValueError):
        oracle.sagebwd_forward(z, z[:2], z[:2], False, 2, 0.1)  # causal = 2 with N > M
    with pytest.raises(ValueError):
        oracle.sagebwd_backward(z, z, z, z, False, 0, 0.1, 0x100)
