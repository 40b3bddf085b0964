"""Pins of the oracle's MXFP4 variant.

Sources: "SageAttention3" summary, 3.4 "The NVFP4 Microscaling Format and Quantization
Operator" (the E2M1 value set; one E8M0 power-of-two scale per 1x32 block along the
reduction dimension of each product; P~ quantized per block of keys, V per block of
tokens); "SageAttention2 Technical Report" summary, 3.4 ("Smoothing Q", "Optional Smoothing
of V", "The Complete Algorithm").

The lossless construction: fp16 inputs whose smoothed Q and K sit exactly on the E2M1 grid
of their own 32-channel blocks (with a different exponent per token and block), V' exactly
on the grid of each 32-token block of each channel, and scores that are multiples of ln 2,
so that every P~ is a power of two within three octaves of its 32-key block's maximum.
Then every quantizer in the MX forward is exact and the result must equal textbook FP64
attention.  A mistake in the block axis of any operand, in the E8M0 rule (the smallest e
with amax <= 6 * 2^e), in the scale arithmetic 2^(e_a + e_b), in the V smoothing
add-back or in the P~ blocks (per 32 keys of the row, relative to the block maximum) breaks
one of the equalities below.
"""
import math

import numpy as np
import pytest

import oracle

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def f16(x):
    x = np.asarray(x, np.float64)
    b = x.astype(np.float16)
    assert np.array_equal(b.astype(np.float64), x), "construction is not fp16-exact"
    return b.view(np.uint16)


def grid_block(rng, n, e):
    """n values on the E2M1 grid times 2^e whose largest magnitude is 4 or 6 times 2^e,
    so that the block's E8M0 exponent is exactly e."""
    z = rng.choice(E2M1, n) * rng.choice([-1.0, 1.0], n)
    z[rng.integers(n)] = rng.choice([4.0, 6.0]) * rng.choice([-1.0, 1.0])
    return z * 2.0 ** e


def mx_lossless_case(seed, N, M, d, smooth_v):
    assert N % 2 == 0 and M % 2 == 0
    rng = np.random.default_rng(seed)
    nb = d // 32
    score_ch = [32 * b + 1 for b in range(nb)]                       # the only channels scores use
    dead_ch = [32 * b + c for b in range(nb) for c in range(2, 10)]  # K constant there (gamma K = 0)
    free_ch = [c for c in range(d) if c not in score_ch and c not in dead_ch]
    # ---- K = kb + Y, Y paired (t, t+1) -> mean(K) = kb exactly
    kb = 2.0 * rng.integers(-3, 4, d)
    Y = np.zeros((M, d))
    kexp = np.zeros((M, nb), int)
    for t in range(0, M, 2):
        for b in range(nb):
            f = int(rng.integers(-2, 2))
            kexp[t, b] = kexp[t + 1, b] = f
            blk = [c for c in free_ch if c // 32 == b]
            Y[t, blk] = grid_block(rng, len(blk), f)
            Y[t, score_ch[b]] = rng.integers(-1, 2)  # 1 = 2^-f * 2^f is on every grid f in -2..1
        Y[t + 1] = -Y[t]
    # ---- Q = qb_i + Yq, Yq paired within each 128-row block; qb only on dead channels
    nqb = -(-N // 128)
    qb = np.zeros((nqb, d))
    Yq = np.zeros((N, d))
    qexp = np.zeros((N, nb), int)
    for i in range(nqb):
        qb[i, dead_ch] = 2.0 * rng.integers(-3, 4, len(dead_ch))
        for r in range(128 * i, min(128 * i + 128, N), 2):
            cr = int(rng.integers(nb))
            for b in range(nb):
                blk = [c for c in dead_ch if c // 32 == b]
                g = int(rng.integers(1, 5)) if b == cr else int(rng.integers(-2, 5))
                qexp[r, b] = qexp[r + 1, b] = g
                Yq[r, blk] = grid_block(rng, len(blk), g)
            Yq[r, score_ch[cr]] = 8.0 * rng.choice([-1.0, 1.0])  # 8 = (8 / 2^g) 2^g, g in 1..4
            Yq[r + 1] = -Yq[r]
    # ---- V = vm + Z; Z on the grid of each 32-token block (pairs keep mean(V) = vm)
    nvb = -(-M // 32)
    vm = 0.25 * rng.integers(-8, 9, d) if smooth_v else np.zeros(d)
    Z = np.zeros((M, d))
    vexp = np.zeros((nvb, d), int)
    for vb in range(nvb):
        toks = np.arange(32 * vb, min(32 * vb + 32, M))
        for c in range(d):
            h = int(rng.integers(-3, 1))
            vexp[vb, c] = h
            z = grid_block(rng, len(toks), h)
            if smooth_v:
                z[1::2] = -z[0::2]
                z[0] = rng.choice([4.0, 6.0]) * 2.0 ** h
                z[1] = -z[0]
            Z[toks, c] = z
    Q = np.repeat(qb, 128, axis=0)[:N] + Yq
    K = kb[None, :] + Y
    V = vm[None, :] + Z
    c = dict(Y=Y, Yq=Yq, Z=Z, kexp=kexp, qexp=qexp, vexp=vexp, qb=qb, kb=kb, vm=vm)
    return f16(Q), f16(K), f16(V), math.log(2.0) / 8.0, c


def codes_of(x, e_per_elem):
    """E2M1 codes of values on the grid; zeros are +0, as the smoothing subtraction leaves them."""
    y = (x + 0.0) / 2.0 ** e_per_elem
    mag = np.abs(y)
    idx = np.array([np.flatnonzero(E2M1 == m)[0] for m in mag.ravel()]).reshape(y.shape)
    return (np.signbit(y).astype(np.uint8) << 3) | idx.astype(np.uint8)


@pytest.mark.parametrize("N,d,smooth_v", [(192, 128, False), (192, 64, True), (130, 128, True)])
def test_mx_codes_and_exponents_match_construction(N, d, smooth_v):
    q, k, v, _, c = mx_lossless_case(30 + N + d, N, N, d, smooth_v)
    p = oracle.preprocess_mx_head(q, k, v, True, oracle.SMOOTH_V if smooth_v else 0)
    nb = d // 32
    qe = np.repeat(c["qexp"], 32, axis=1)
    ke = np.repeat(c["kexp"], 32, axis=1)
    ve = np.repeat(c["vexp"], 32, axis=0)[:N]
    # blocks that are entirely zero take the floor exponent -127 (their codes are zeros)
    zq = np.repeat(np.abs(c["Yq"]).reshape(N, nb, 32).max(axis=2) == 0, 32, axis=1)
    zk = np.repeat(np.abs(c["Y"]).reshape(N, nb, 32).max(axis=2) == 0, 32, axis=1)
    assert np.array_equal(p["qexp"], np.where(zq[:, ::32], -127, c["qexp"]))
    assert np.array_equal(p["kexp"], np.where(zk[:, ::32], -127, c["kexp"]))
    assert np.array_equal(p["vexp"], c["vexp"])
    assert np.array_equal(p["qcode"], codes_of(c["Yq"], np.where(zq, 0, qe)))
    assert np.array_equal(p["kcode"], codes_of(c["Y"], np.where(zk, 0, ke)))
    assert np.array_equal(p["vcode"], codes_of(c["Z"], ve))


@pytest.mark.parametrize("N,d,causal,smooth_v", [(192, 128, False, False), (192, 128, True, True),
                                                 (160, 64, False, True), (130, 128, True, False)])
def test_mx_lossless_construction_equals_textbook(N, d, causal, smooth_v):
    q, k, v, s, c = mx_lossless_case(40 + N + d, N, N, d, smooth_v)
    flags = oracle.MXFP4 | (oracle.SMOOTH_V if smooth_v else 0)
    got = oracle.forward_head(q, k, v, True, causal, s, flags)
    ex = oracle.exact_head(q, k, v, True, causal, s)
    assert np.abs(got - ex).max() < 1e-11 * max(1.0, np.abs(ex).max())


def test_mx_p_block_exponent_follows_block_max_not_row_max():
    """One 64-key tile, scores (ln 2) * {-2 for keys 0..31 except -4 for key 3; 0 for keys
    32..63}: row 0 sees P~ = 2^-2 and 2^-4 in its first 32-key block and 1 in the second.
    With one exponent per 32-key block (e = -4 for block max 2^-2) both 2^-2 = 4 * 2^-4 and
    2^-4 = 1 * 2^-4 are on the grid, and only key 3 carries a value, so O = exact attention.
    A single exponent per row (e = -2 for row max 1) would put 2^-4 = 0.25 * 2^-2 on a tie
    and round it to 0, losing the whole output.  K is left unsmoothed (its mean would move
    the values off the grid); row 1 = -row 0 keeps the Q block mean at 0."""
    d, M = 64, 64
    Q = np.zeros((2, d)); Q[0, 0] = 1.0; Q[1, 0] = -1.0
    K = np.zeros((M, d))
    K[:32, 0] = -2.0
    K[3, 0] = -4.0
    V = np.zeros((M, d))
    V[3, :] = 4.0
    q, k, v = f16(Q), f16(K), f16(V)
    s = math.log(2.0)
    got = oracle.forward_head(q, k, v, True, False, s, oracle.MXFP4 | oracle.NO_SMOOTH_K)
    ex = oracle.exact_head(q, k, v, True, False, s)
    l0 = 31 * 2.0 ** -2 + 2.0 ** -4 + 32
    assert abs(ex[0, 0] - 4 * 2.0 ** -4 / l0) < 1e-15
    assert np.abs(got - ex).max() < 1e-12


# ---- two-level quantization of P~ (knob MX_P_TWO_LEVEL) ----
# "SageAttention3" summary, 3.4 "Two-Level Quantization for the Attention Map P": each row of
# a tile's P~ is first divided by an FP32 factor s1 from the row maximum (the maximum of P~ is
# exp(rowmax S - m), the softmax's own maximum), then block-quantized; the tile's product is
# multiplied back by s1.  With E8M0 block scales the reading is s1 = rowmax / 6, so that the
# row maximum is exactly the largest E2M1 value.

def two_level_case(seed, N, M, d):
    """All query rows equal (so Q^ = 0 and S = Delta S * sm_scale exactly), K channel 0 in {0, 1}
    (so gamma K takes two values one apart), every other channel zero, and V on the E2M1 grid of
    every 32-token block (M a power of two keeps mean(K) exact).  With sm_scale = ln(3/2) a row's visible scores sit on two levels whose
    P~ ratio is exactly 2/3; the first two tiles hold low keys only, so the running maximum
    rises later.  Level one maps a tile's larger level to 6 and the smaller to 4, both on the
    grid, so every quantizer is exact; quantizing P~ directly puts 2/3 of the block maximum
    (16/3 or 8/3 times the block scale) off the grid."""
    rng = np.random.default_rng(seed)
    Q = np.zeros((N, d)); Q[:, 0] = 1.0
    K = np.zeros((M, d))
    hi = rng.random(M) < 0.4
    hi[:128] = False
    hi[min(M - 1, 130)] = True
    K[hi, 0] = 1.0
    V = rng.choice([0.0, 0.5, 1.0, 1.5, 2.0, 3.0], (M, d)) * rng.choice([-1.0, 1.0], (M, d))
    return Q, K, V


def textbook(Q, K, V, sm, causal):
    """softmax(Q K^T sm) V in FP64 with numpy (top-left causal mask)."""
    s = (Q @ K.T) * sm
    if causal:
        s = np.where(np.arange(K.shape[0])[None, :] <= np.arange(Q.shape[0])[:, None], s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)) @ V


@pytest.mark.parametrize("N,M,d,causal", [(256, 256, 64, False), (256, 256, 64, True), (192, 512, 128, False)])
def test_mx_two_level_p_lossless_on_two_levels(N, M, d, causal):
    Q, K, V = two_level_case(50 + N + d, N, M, d)
    q, k, v = f16(Q), f16(K), f16(V)
    sm = math.log(1.5)
    ex = textbook(Q, K, V, sm, causal)
    two = oracle.forward_head(q, k, v, True, causal, sm, oracle.MXFP4 | oracle.MX_P_TWO_LEVEL)
    direct = oracle.forward_head(q, k, v, True, causal, sm, oracle.MXFP4)
    assert np.abs(two - ex).max() < 1e-12
    assert np.abs(direct - ex).max() > 1e-3  # the construction tells the two apart


def test_mx_two_level_p_is_mx_only():
    q = k = v = np.zeros((64, 64), np.uint16)
    with pytest.raises(ValueError):
        oracle.forward_head(q, k, v, True, 0, 0.125, oracle.MX_P_TWO_LEVEL)


@pytest.mark.parametrize("name", ["mxfp4_32k", "prefill32k", "video17k"])
def test_mx_two_level_p_lowers_error(name):
    """Direction of the pages' Table 1(b): against exact attention, two-level P has a lower
    mean error than direct P quantization (here with E8M0 block scales, on the synthetic
    stand-ins for the pages' workloads, 2 heads of 2048 tokens, every 7th row)."""
    from quantized_attention_amd import synthetic as sy
    cfg = sy.CONFIGS[name].with_shape(B=1, H=2, N=2048, M=2048)
    qb, kb, vb = sy.make_qkv(cfg)
    sm = 1 / math.sqrt(cfg.d)
    rows = np.arange(0, 2048, 7)
    for h in range(2):
        args = (qb[0, h], kb[0, h], vb[0, h], cfg.fp16, 1 if cfg.causal else 0, sm)
        ex = oracle.exact_head(*args, rows=rows)
        e_two = np.abs(oracle.forward_head(*args, oracle.MXFP4 | oracle.MX_P_TWO_LEVEL, rows=rows) - ex).mean()
        e_dir = np.abs(oracle.forward_head(*args, oracle.MXFP4, rows=rows) - ex).mean()
        assert e_two < e_dir


def test_tie_diagnostic_counts_exact_midpoints():
    """The rounding-boundary diagnostic: with the two-level construction's scores (two levels one
    unit apart, all rows equal) and sm_scale = ln(448 / 17), every low key has 448 P~ = 17, the
    midpoint between the E4M3 values 16 and 18, and every high key 448; so a row's count is the
    number of low keys it sees after the first high one (non-causal: the same for every row),
    and its bound is those keys' P^ gap (2, of 448) times their largest dequantized V value,
    over l = (high keys) + (low keys) 17 / 448."""
    N = M = 256
    Q, K, V = two_level_case(7, N, M, 64)
    q, k, v = f16(Q), f16(K), f16(V)
    out, ties, bound = oracle.forward_head_ties(q, k, v, True, False, math.log(448 / 17), 0)
    hi = K[:, 0] == 1
    # low keys before the first high one were quantized relative to their own (lower) maximum:
    # there 448 P~ = 448 exactly, not a tie
    lead = (int(np.flatnonzero(hi)[0]) // 64) * 64
    late_low = ~hi & (np.arange(M) >= lead)
    assert (ties == late_low.sum()).all()
    p = oracle.preprocess_head(q, k, v, True)
    vdq = oracle.e4m3_decode_table()[p["vhat"]] * p["dv"].astype(np.float64)[None, :]
    vm = np.abs(vdq).max(axis=1)
    l = hi.sum() + (~hi).sum() * 17 / 448
    assert np.allclose(bound, (2 / 448) * vm[late_low].sum() / l, rtol=1e-12, atol=0)
    assert np.array_equal(out, oracle.forward_head(q, k, v, True, False, math.log(448 / 17), 0))


# ---- the MX branch of the rounding-decision margin (orc_forward_head_ties) ----
# The diagnostic counts, per output row, the P quantization decisions whose input lies within a
# relative tie_eps of a rounding boundary, and bounds the output change should every one of
# them round the other way.  In the MX form there are two kinds of decision ("SageAttention3"
# summary, 3.4 "The NVFP4 Microscaling Format and Quantization Operator"): an element's E2M1
# code (boundaries at the midpoints 0.25, 0.75, ..., 5 of the value set, times the block
# scale 2^e; the code then moves by the gap between its neighbours) and a 32-key block's E8M0
# exponent (the block maximum against 6 2^e from below or 6 2^(e-1) from above; the whole
# block is then quantized one octave coarser or finer, each value moving by less than 4 2^e).
# The construction below puts every late P~ on one of these boundaries, up to a relative
# offset of 1e-9 chosen so that the FP64 side of each decision is fixed, and states the count
# and the bound in closed form.

TIE_EPS = 2.0 ** -16
HI_KEYS = (70, 130, 200)  # one high key in 32-key blocks 2, 4 and 6; blocks 0, 1 lie before the first


def mx_tie_case():
    """All query rows equal (Q^ = 0, so S = Delta S * sm_scale), K channel 0 equal to 1 on the
    high keys and 0 elsewhere (M = 256, so mean(K) = 3/256 and gamma K are exact), V on the
    E2M1 grid of every 32-token block.  A low key's P~ relative to a high maximum is then
    r = exp(-sm_scale); the tile of the first high key and every later tile hold a high key,
    so every low key from key 64 on is quantized against the high maximum."""
    rng = np.random.default_rng(11)
    N = M = 256
    d = 64
    Q = np.zeros((N, d)); Q[:, 0] = 1.0
    K = np.zeros((M, d)); K[list(HI_KEYS), 0] = 1.0
    V = rng.choice([0.0, 0.5, 1.0, 1.5, 2.0, 3.0], (M, d)) * rng.choice([-1.0, 1.0], (M, d))
    return f16(Q), f16(K), f16(V), V


def check_mx_ties(two_level=False):
    """Counts and bounds of the MX margin diagnostic in closed form (raises AssertionError)."""
    q, k, v, V = mx_tie_case()
    M = 256
    vmax = np.abs(V).max(axis=1)                       # the largest dequantized V' value of each key
    hi = np.zeros(M, bool); hi[list(HI_KEYS)] = True
    late_low = ~hi & (np.arange(M) >= 64)
    low_blocks = [3, 5, 7]                             # late 32-key blocks without a high key
    flags = oracle.MXFP4 | (oracle.MX_P_TWO_LEVEL if two_level else 0)

    def run(r):
        out, ties, bound = oracle.forward_head_ties(q, k, v, True, 0, -math.log(r), flags, tie_eps=TIE_EPS)
        l = hi.sum() + (~hi).sum() * r                 # l in the final frame (high maximum)
        return out, ties, bound, l

    if not two_level:
        # (a) element midpoints: block scale 2^-2 (block maximum 1 or 7/8), every late low value
        # at 3.5 (1 + 1e-9) times it, gap 1; no exponent decision near a boundary
        out, ties, bound, l = run(0.875 * (1 + 1e-9))
        assert (ties == late_low.sum()).all(), ties
        assert np.allclose(bound, 0.25 * vmax[late_low].sum() / l, rtol=1e-7, atol=0)
        # (b) a low-only block's maximum r just below 6 2^-3 = 0.75: exponent -3, its values
        # at 6 (1 - 1e-9) 2^-3 (on the grid); the exponent decision is near 6 2^e
        out, ties, bound, l = run(0.75 * (1 - 1e-9))
        blk = sum(vmax[32 * b:32 * b + 32].sum() for b in low_blocks)
        assert (ties == len(low_blocks)).all(), ties
        assert np.allclose(bound, 4 * 2.0 ** -3 * blk / l, rtol=1e-7, atol=0)
        # (c) the maximum just above 0.75 = 6 2^(e-1): exponent -2, values at 3 (1 + 1e-9) 2^-2
        out, ties, bound, l = run(0.75 * (1 + 1e-9))
        assert (ties == len(low_blocks)).all(), ties
        assert np.allclose(bound, 4 * 2.0 ** -2 * blk / l, rtol=1e-7, atol=0)
        assert np.array_equal(out, oracle.forward_head(q, k, v, True, 0, -math.log(0.75 * (1 + 1e-9)), flags))
    else:
        # two-level P: every late tile holds a high key, so s1 = 1/6 and the high keys map to 6
        # exactly (not a rounded input: no exponent decision); low keys at 6 r = 3.5 (1 + 1e-9)
        # with block scale 2^0, gap 1, weighted by s1
        out, ties, bound, l = run((7.0 / 12.0) * (1 + 1e-9))
        assert (ties == late_low.sum()).all(), ties
        assert np.allclose(bound, (1.0 / 6.0) * vmax[late_low].sum() / l, rtol=1e-7, atol=0)


@pytest.mark.parametrize("two_level", [False, True])
def test_mx_tie_diagnostic_closed_form(two_level):
    check_mx_ties(two_level)


# Plausible mistakes in the MX branch of the margin bound, each planted in a copy of the oracle:
# the octave move of an exponent decision bounded by 2 instead of 4 steps; the exponent decision
# dropped; only one side of it checked; the element gap table off; the block scale 2^e left out;
# the two-level factor s1 left out.
MX_TIE_MISTAKES = {
    "octave_x2": ("blk += 4.0 * S[x];", "blk += 2.0 * S[x];"),
    "no_exponent_decision": ("if (am > 0.0 && !(two && am == 6.0) &&", "if (0 && am > 0.0 && !(two && am == 6.0) &&"),
    "exponent_one_side": ("|| near_rel(am, 6.0 * ldexp(1.0, ep - 1), tie_eps))", ")"),
    "gap_table": ("static const double gap[7] = {0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0};",
                  "static const double gap[7] = {0.5, 0.5, 0.5, 0.5, 1.0, 0.5, 2.0};"),
    "no_block_scale": ("mg.mass += s1 * ldexp(blk, ep);", "mg.mass += s1 * blk;"),
    "no_s1": ("mg.mass += s1 * ldexp(blk, ep);", "mg.mass += ldexp(blk, ep);"),
}


@pytest.mark.parametrize("name", sorted(MX_TIE_MISTAKES))
def test_mx_tie_diagnostic_catches_planted_mistake(name):
    old, new = MX_TIE_MISTAKES[name]
    with oracle.planted_mistake(("sage_oracle.c", old, new)):
        with pytest.raises(AssertionError):
            check_mx_ties(False)
            check_mx_ties(True)
