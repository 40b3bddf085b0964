"""Pins of the oracle against what the pages and the mathematics fix.

Sources: "SageAttention2 Technical Report" summary, 3.4 ("Smoothing Q": softmax shift
invariance and the Delta S decomposition; "Per-Thread INT4 Quantization"; "FP8 Quantization
for P~V"; "Two-Level Accumulation"; "Optional Smoothing of V": P~ V_m = V_m; "The Complete
Algorithm (Algorithm 1)"); "Quantization for Attention, in depth" ("The datapath and its
quantize points").

The pins, and the mistakes they are built to catch:
  * textbook attention vs torch FP64 and a pure-Python brute force (mask, scale, softmax);
  * identity quantizers reduce the tile loop to textbook attention (online softmax, alpha
    rescale, two-level sum, causal skip, ragged tiles, epilogue, V smoothing add-back);
  * a QK-lossless construction: inputs whose smoothed Q and K sit exactly on their INT8
    grids, with a different scale exponent per token / per key group, so the quantized
    forward must equal textbook attention (group map, per-token dQ, dQ dK dequant, the sign
    and definition of Delta S, both means);
  * a PV-lossless construction: scores that are integer multiples of ln 2 and V on the
    E4M3 grid with per-channel exponents (448 static scale, per-channel dV, P^ relative to
    the running max, alpha rescale, V smoothing);
  * a closed form for l: one key with P~ = 1 and 64 keys with P~ = 0.3 (E4M3(134.4) = 128),
    which pins "l sums the unquantized P~" and the RNE cast;
  * invariants of the quantizers and the means.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_attention_amd import synthetic as sy


def f16(x):
    x = np.asarray(x, np.float64)
    b = x.astype(np.float16)
    assert np.array_equal(b.astype(np.float64), x), "construction is not fp16-exact"
    return b.view(np.uint16)


def rel_err(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# ---------------------------------------------------------------- textbook attention
def test_exact_matches_torch_and_bruteforce():
    rng = np.random.default_rng(0)
    for causal, (N, M, d) in itertools.product([False, True], [(37, 37, 64), (5, 5, 8)]):
        if not causal:
            M = M + 11
        q, k, v = rng.standard_normal((N, d)), rng.standard_normal((M, d)), rng.standard_normal((M, d))
        s = 0.37
        got = oracle.exact_f64(q, k, v, causal, s)
        S = torch.from_numpy(q) @ torch.from_numpy(k).T * s
        if causal:
            S = S.masked_fill(torch.ones(N, M, dtype=torch.bool).triu(1), float("-inf"))
        ref = (torch.softmax(S, dim=-1) @ torch.from_numpy(v)).numpy()
        assert np.abs(got - ref).max() < 1e-13
    # brute force, pure Python, tiny
    q, k, v = rng.standard_normal((3, 2)), rng.standard_normal((4, 2)), rng.standard_normal((4, 2))
    got = oracle.exact_f64(q, k, v, False, 0.5)
    for r in range(3):
        w = [math.exp(0.5 * sum(q[r, c] * k[t, c] for c in range(2))) for t in range(4)]
        for c in range(2):
            assert abs(sum(w[t] * v[t, c] for t in range(4)) / sum(w) - got[r, c]) < 1e-14


def test_softmax_shift_invariance_under_k_mean():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((64, 64)) + 2.0
    k = rng.standard_normal((80, 64)) + rng.standard_normal(64) * 5.0
    v = rng.standard_normal((80, 64))
    a = oracle.exact_f64(q, k, v, False, 0.125)
    b = oracle.exact_f64(q, k - k.mean(0), v, False, 0.125)
    assert np.abs(a - b).max() < 1e-12


def test_v_mean_passes_through_attention():
    """Rows of softmax sum to one, so a V whose rows all equal V_m returns V_m."""
    rng = np.random.default_rng(2)
    vm = rng.standard_normal(64) * 3
    out = oracle.exact_f64(rng.standard_normal((50, 64)), rng.standard_normal((70, 64)),
                           np.tile(vm, (70, 1)), False, 0.2)
    assert np.abs(out - vm).max() < 1e-12


# ---------------------------------------------------------------- Delta S decomposition
def test_delta_s_decomposition_is_row_constant():
    cfg = sy.CONFIGS["tiny"].with_shape(N=300, M=200)
    q, k, v = [x[0, 0] for x in sy.make_qkv(cfg)]
    p = oracle.preprocess_head(q, k, v, fp16=True)
    Q = sy.bits_to_f32(q, True).astype(np.float64)
    K = sy.bits_to_f32(k, True).astype(np.float64)
    gk = (sy.bits_to_f32(k, True) - p["kmean"][None, :]).astype(np.float64)
    for i in range(p["qmean"].shape[0]):
        rows = slice(128 * i, min(128 * i + 128, 300))
        gq = (sy.bits_to_f32(q, True)[rows] - p["qmean"][i][None, :]).astype(np.float64)
        diff = Q[rows] @ K.T - (gq @ gk.T + p["ds"][i][None, :])
        # constant along each row (the dropped q_i k^T + gamma(Q_i) k^T terms)
        assert np.abs(diff - diff[:, :1]).max() < 2e-3 * np.abs(Q[rows] @ K.T).max() * 1e-2
        # and not trivially so: Delta S itself is O(1)
        assert np.abs(p["ds"][i]).max() > 0.1


# ---------------------------------------------------------------- identity quantizers
@pytest.mark.parametrize("fp16,d,N,M,causal,flags", [
    (True, 64, 256, 256, False, 0),
    (True, 64, 300, 300, True, 0),
    (False, 128, 200, 333, False, 0),
    (False, 128, 130, 130, True, oracle.SMOOTH_V),
    (True, 64, 77, 190, False, oracle.SMOOTH_V),
])
def test_identity_quantizers_equal_textbook_attention(fp16, d, N, M, causal, flags):
    cfg = sy.CONFIGS["video17k"].with_shape(N=N, M=M, d=d, dtype="fp16" if fp16 else "bf16", H=1, B=1)
    q, k, v = [x[0, 0] for x in sy.make_qkv(cfg)]
    s = 1 / math.sqrt(d)
    ex = oracle.exact_head(q, k, v, fp16, causal, s)
    idm = oracle.forward_head(q, k, v, fp16, causal, s, flags | oracle.QK_IDENTITY | oracle.PV_IDENTITY)
    assert np.abs(idm - ex).max() < 1e-10
    # sampled rows give the same rows
    rows = np.array([0, N - 1, N // 2, 5])
    sub = oracle.forward_head(q, k, v, fp16, causal, s, flags | oracle.QK_IDENTITY | oracle.PV_IDENTITY, rows=rows)
    assert np.array_equal(sub, idm[rows])


# ---------------------------------------------------------------- causal alignments, N != M
@pytest.mark.parametrize("N,M", [(37, 37), (20, 53), (53, 20), (1, 9)])
def test_causal_alignments_match_torch_masks(N, M):
    """causal = 1: key t visible to row r iff t <= r (the upper triangle of the N x M score
    matrix masked, as the pages' reference code does); causal = 2: iff t <= r + M - N (the
    last query aligned with the last key).  Masks built independently with torch.tril."""
    rng = np.random.default_rng(N * 100 + M)
    d = 16
    q, k, v = rng.standard_normal((N, d)), rng.standard_normal((M, d)), rng.standard_normal((M, d))
    S = torch.from_numpy(q) @ torch.from_numpy(k).T * 0.41
    for causal, diag in [(1, 0), (2, M - N)]:
        if causal == 2 and N > M:
            with pytest.raises(ValueError):
                oracle.exact_f64(q, k, v, causal, 0.41)
            continue
        keep = torch.ones(N, M, dtype=torch.bool).tril(diag)
        ref = (torch.softmax(S.masked_fill(~keep, float("-inf")), dim=-1) @ torch.from_numpy(v)).numpy()
        got = oracle.exact_f64(q, k, v, causal, 0.41)
        assert np.abs(got - ref).max() < 1e-13


def test_bottom_right_equals_suffix_of_full_causal():
    """The last N queries of a causal sequence of M tokens, attending under causal = 2, give the
    last N rows of causal attention over all M queries."""
    cfg = sy.CONFIGS["tiny"].with_shape(N=150, M=150)
    q, k, v = [x[0, 0] for x in sy.make_qkv(cfg)]
    s = 1 / 8
    full = oracle.exact_head(q, k, v, True, 1, s)
    tail = oracle.exact_head(q[100:], k, v, True, 2, s)
    assert np.abs(tail - full[100:]).max() < 1e-13


@pytest.mark.parametrize("N,M,causal,flags", [(90, 300, 2, 0), (90, 300, 1, oracle.SMOOTH_V),
                                              (300, 90, 1, 0), (200, 200, 2, oracle.SMOOTH_V)])
def test_identity_quantizers_causal_alignments(N, M, causal, flags):
    cfg = sy.CONFIGS["video17k"].with_shape(N=N, M=M, d=64, H=1, B=1)
    q, k, v = [x[0, 0] for x in sy.make_qkv(cfg)]
    s = 1 / 8
    ex = oracle.exact_head(q, k, v, False, causal, s)
    idm = oracle.forward_head(q, k, v, False, causal, s, flags | oracle.QK_IDENTITY | oracle.PV_IDENTITY)
    assert np.abs(idm - ex).max() < 1e-10


def test_causal_argument_rejected():
    q = np.zeros((5, 64), np.uint16)
    k = np.zeros((3, 64), np.uint16)
    with pytest.raises(ValueError):
        oracle.forward_head(q, k, k, False, 2, 0.1)  # bottom-right needs N <= M
    with pytest.raises(ValueError):
        oracle.forward_head(q, q, q, False, 3, 0.1)


# ---------------------------------------------------------------- QK-lossless construction
def qk_lossless_case(seed, N, M, d):
    """fp16 inputs whose smoothed Q, K are exactly on the per-token / per-group INT8 grids."""
    rng = np.random.default_rng(seed)
    kb = 8.0 * rng.integers(-4, 5, d)
    Y = np.zeros((M, d))
    eg = {}
    for u in range(-(-M // 64)):
        keys = [t for t in range(64 * u, min(64 * u + 64, M))]
        for g in range(4):
            grp = [t for t in keys if oracle.lib().orc_k_group(t) == g]
            if not grp:
                continue
            e = int(rng.integers(-3, 1))
            eg[(u, g)] = e
            assert len(grp) % 2 == 0
            for a, b in zip(grp[0::2], grp[1::2]):
                n = rng.integers(-20, 21, d).astype(np.float64)
                Y[a] = n * 2.0 ** e
                Y[b] = -Y[a]
            Y[grp[0], rng.integers(d)] = 127 * 2.0 ** e
            Y[grp[1]] = -Y[grp[0]]
    K = kb[None, :] + Y
    Yq = np.zeros((N, d))
    qb = np.zeros((-(-N // 128), d))
    er = np.zeros(N, int)
    for i in range(qb.shape[0]):
        qb[i] = 4.0 * rng.integers(-4, 5, d)
        rows = list(range(128 * i, min(128 * i + 128, N)))
        assert len(rows) % 2 == 0
        for a, b in zip(rows[0::2], rows[1::2]):
            e = int(rng.integers(-2, 1))
            n = rng.integers(-20, 21, d).astype(np.float64)
            n[rng.integers(d)] = 127 * rng.choice([-1, 1])
            Yq[a] = n * 2.0 ** e
            Yq[b] = -Yq[a]
            er[a] = er[b] = e
    Q = np.repeat(qb, 128, axis=0)[:N] + Yq
    V = rng.standard_normal((M, d)).astype(np.float16).astype(np.float64)
    return f16(Q), f16(K), f16(V), dict(kb=kb, Y=Y, eg=eg, qb=qb, Yq=Yq, er=er)


@pytest.mark.parametrize("N,causal", [(200, False), (200, True), (256, False)])
def test_qk_lossless_construction(N, causal):
    d = 64
    q, k, v, c = qk_lossless_case(10 + N, N, N, d)
    p = oracle.preprocess_head(q, k, v, fp16=True)
    assert np.array_equal(p["kmean"], c["kb"].astype(np.float32))
    for (u, g), e in c["eg"].items():
        assert p["dk"][u, g] == 2.0 ** e
    assert np.array_equal(p["khat"].astype(np.float64), c["Y"] / np.array(
        [2.0 ** c["eg"][(t // 64, oracle.lib().orc_k_group(t))] for t in range(N)])[:, None])
    assert np.array_equal(p["qmean"], c["qb"].astype(np.float32))
    assert np.array_equal(p["dq"], (2.0 ** c["er"]).astype(np.float32))
    assert np.array_equal(p["qhat"].astype(np.float64), c["Yq"] / 2.0 ** c["er"][:, None])
    assert np.array_equal(p["ds"], c["qb"] @ c["Y"].T)
    s = 1 / 64
    ex = oracle.exact_head(q, k, v, True, causal, s)
    got = oracle.forward_head(q, k, v, True, causal, s, oracle.PV_IDENTITY)
    assert np.abs(got - ex).max() < 1e-11


# ---------------------------------------------------------------- PV-lossless construction
def pv_lossless_case(seed, N, M, d, smooth_v):
    rng = np.random.default_rng(seed)
    dec = oracle.e4m3_decode_table()
    grid = np.array([dec[c] for c in range(0x30, 0x7F)])  # magnitudes 0.5 .. 448
    Q = np.zeros((N, d))
    Q[np.arange(N), rng.integers(0, d, N)] = 8.0
    # one more per 64-key tile: every tile raises the running maximum by exactly one octave, so
    # each one rescales O and l by alpha = 1/2 (P~ stays within 2^-15 of its tile's maximum)
    K = (rng.integers(0, 13, (M, d)) + (np.arange(M) // 64)[:, None]).astype(np.float64)
    ev = rng.integers(-6, -1, d)
    Z = np.zeros((M, d))
    for c in range(d):
        z = rng.choice(grid, M) * rng.choice([-1, 1], M)
        z[2 * rng.integers(M // 2)] = 448.0  # an even slot, so the pairing below keeps it
        if smooth_v:
            z[1::2] = -z[0::2]
        Z[:, c] = z * 2.0 ** ev[c]
    vm = 16.0 * 2.0 ** ev * rng.integers(-3, 4, d) if smooth_v else np.zeros(d)
    V = vm[None, :] + Z
    return f16(Q), f16(K), f16(V), math.log(2.0) / 8.0


@pytest.mark.parametrize("N,causal,smooth_v", [(150, False, False), (150, True, False),
                                               (150, False, True), (192, True, True)])
def test_pv_lossless_construction(N, causal, smooth_v):
    q, k, v, s = pv_lossless_case(20 + N, N, N, 64, smooth_v)
    flags = oracle.QK_IDENTITY | (oracle.SMOOTH_V if smooth_v else 0)
    ex = oracle.exact_head(q, k, v, True, causal, s)
    got = oracle.forward_head(q, k, v, True, causal, s, flags)
    assert np.abs(got - ex).max() < 1e-11 * max(1.0, np.abs(ex).max())
    p = oracle.preprocess_head(q, k, v, True, oracle.SMOOTH_V if smooth_v else 0)
    # every nonzero V channel has a code of magnitude 448
    assert np.all(np.any((p["vhat"] & 0x7F) == 0x7E, axis=0))


# ---------------------------------------------------------------- closed form for l
@pytest.mark.parametrize("n", [64, 10])
def test_row_sum_uses_unquantized_p(n):
    """One key at P~ = 1, n keys at P~ = 0.3, V constant 1: O = (448 + 128 n) / (448 (1 + 0.3 n))."""
    d, M = 64, n + 1
    Q = np.zeros((1, d)); Q[0, 0] = 1.0
    K = np.zeros((M, d)); K[0, 0] = 1.0
    V = np.ones((M, d))
    s = -math.log(0.3)
    q, k, v = f16(Q), f16(K), f16(V)
    got = oracle.forward_head(q, k, v, True, False, s, oracle.QK_IDENTITY)
    assert oracle.lib().orc_e4m3_decode(oracle.lib().orc_e4m3_encode(448 * 0.3)) == 128.0
    dv = float(np.float32(1.0) / np.float32(448.0))  # dV = amax / 448 rounded to FP32
    want = (448 + 128 * n) / (448 * (1 + 0.3 * n)) * 448 * dv
    assert np.abs(got - want).max() < 1e-12
    ex = oracle.exact_head(q, k, v, True, False, s)
    assert np.abs(ex - 1.0).max() < 1e-12


# ---------------------------------------------------------------- quantizer invariants
def test_quantizer_invariants_and_means():
    cfg = sy.CONFIGS["prefill32k"].with_shape(N=700, M=700, H=1)
    q, k, v = [x[0, 0] for x in sy.make_qkv(cfg)]
    p = oracle.preprocess_head(q, k, v, fp16=False, flags=oracle.SMOOTH_V)
    K = sy.bits_to_f32(k, False)
    Q = sy.bits_to_f32(q, False)
    V = sy.bits_to_f32(v, False)
    # means: within one FP32 rounding of the FP64 mean
    for X, m in ((K, p["kmean"]), (V, p["vmean"])):
        ref = X.astype(np.float64).mean(0)
        assert np.all(np.abs(m - ref) <= np.spacing(np.abs(ref).astype(np.float32)) * 1.0 + 1e-30)
    gk = K - p["kmean"][None, :]
    for t0 in range(0, 700, 64):
        for g in range(4):
            keys = [t for t in range(t0, min(t0 + 64, 700)) if oracle.lib().orc_k_group(t) == g]
            if not keys:
                continue
            dk = p["dk"][t0 // 64, g]
            assert np.abs(p["khat"][keys]).max() == 127
            err = np.abs(gk[keys] - p["khat"][keys].astype(np.float32) * dk)
            assert err.max() <= dk * 0.5 * (1 + 1e-5)
    assert np.all(np.abs(p["qhat"]).max(1) == 127)
    for i in range(p["qmean"].shape[0]):
        rows = slice(128 * i, min(128 * i + 128, 700))
        ref = Q[rows].astype(np.float64).mean(0)
        assert np.all(np.abs(p["qmean"][i] - ref) <= np.spacing(np.abs(ref).astype(np.float32)))
    assert np.all(np.any((p["vhat"] & 0x7F) == 0x7E, axis=0))
    dec = oracle.e4m3_decode_table()
    vp = V - p["vmean"][None, :]
    rel = np.abs(dec[p["vhat"]] * p["dv"][None, :] - vp) / np.maximum(np.abs(vp), 1e-30)
    normal = np.abs(vp) / p["dv"][None, :] >= 2.0 ** -6
    assert rel[normal].max() <= 2.0 ** -4 * (1 + 1e-6)


def test_empty_key_group_has_floor_scale():
    """M = 600: the last tile holds 24 keys, all in its first 32-key half, so groups 2, 3
    are empty and take amax 0 -> scale max(0, 1e-8) / 127."""
    cfg = sy.CONFIGS["n4k"].with_shape(H=1, N=128, M=600)
    q, k, v = [x[0, 0] for x in sy.make_qkv(cfg)]
    p = oracle.preprocess_head(q, k, v, fp16=False)
    floor = np.float32(1e-8) / np.float32(127.0)
    assert p["dk"][-1, 2] == floor and p["dk"][-1, 3] == floor
    assert p["dk"][-1, 0] > 1e-3 and p["dk"][-1, 1] > 1e-3
