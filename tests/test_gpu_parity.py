"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Bars (stated by the method's acceptance criteria): quantized tensors, scales and means
bit-exact; the output within max |err| <= 1e-2 and mean |err| <= 1e-3 of the oracle
(FP32 output, so output rounding is not part of the error) and cosine >= 0.999 against
textbook FP64 attention.  Delta S is FP32 on the GPU and FP64 in the oracle, so it is
compared with a relative tolerance.

Sizes: small cases the oracle finishes in seconds that span several tiles with ragged
tails; the full workload shapes in the launch configuration the benchmark times, checked
on sampled rows the oracle computes one by one.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from quantized_attention_amd import synthetic as sy

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, MIN_COS = 1e-2, 1e-3, 0.999


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_attention_amd  # noqa: F401  (fails loudly if the library is missing)
    quantized_attention_amd.load_library()


from tests import gpu_util as gu  # noqa: E402


def small(name, **kw):
    return sy.CONFIGS[name].with_shape(**kw)


SMALL_CASES = [
    ("tiny", sy.CONFIGS["tiny"]),
    ("n4k-ragged", small("n4k", H=2, N=600, M=600)),
    ("prefill-causal", small("prefill32k", H=2, N=700, M=700)),
    ("video-smoothv", small("video17k", B=2, H=1, N=333, M=333)),
    ("video-nosmooth", small("video17k", B=1, H=2, N=333, M=333, smooth_v=False)),
    ("fp16-d128-N!=M", sy.Config("fp16x", 1, 2, 300, 1000, 128, "fp16", False,
                                 sy.Dist(q_off_std=1.0, k_off_std=2.0, v_bias_std=0.5), 77)),
    ("bf16-d64-causal", sy.Config("bf16c", 1, 1, 250, 250, 64, "bf16", True,
                                  sy.Dist(k_off_std=3.0, k_spike=8.0, k_spike_channels=sy.spike_channels(64)), 78)),
    ("one-token", sy.Config("one", 1, 1, 1, 1, 64, "bf16", False, sy.Dist(), 79)),
    ("few-tokens", sy.Config("few", 1, 3, 5, 3, 128, "fp16", False, sy.Dist(k_off_std=1.0), 80)),
    ("causal-br-N<M", small("prefill32k", H=2, N=300, M=1000, causal=2)),
    ("causal-tl-N<M", small("prefill32k", H=2, N=300, M=700, causal=1)),
    ("causal-tl-N>M", small("prefill32k", H=1, N=700, M=300, causal=1)),
    ("causal-br-d64-smoothv", small("video17k", B=1, H=2, N=200, M=900, causal=2)),
]


def oracle_head(cfg, q, k, v, bh, flags=0, rows=None):
    b, h = bh // cfg.H, bh % cfg.H
    return oracle.forward_head(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, 1 / math.sqrt(cfg.d),
                               flags | (oracle.SMOOTH_V if cfg.smooth_v else 0), rows=rows)


def check_preprocess_head(cfg, g, q, k, v, bh):
    """Every quantize view of head bh against the oracle's preprocessing: means, scales and codes
    bit for bit; Delta S (FP32 against FP64) within 1e-5 relative, on the tiles that are written."""
    N, M = cfg.N, cfg.M
    b, h = bh // cfg.H, bh % cfg.H
    o = oracle.preprocess_head(q[b, h], k[b, h], v[b, h], cfg.fp16, oracle.SMOOTH_V if cfg.smooth_v else 0)
    assert np.array_equal(g["k_mean"][bh].view(np.uint32), o["kmean"].view(np.uint32))
    assert np.array_equal(g["v_mean"][bh].view(np.uint32), o["vmean"].view(np.uint32))
    assert np.array_equal(g["q_mean"][bh].view(np.uint32), o["qmean"].view(np.uint32))
    assert np.array_equal(g["dq"][bh, :N].view(np.uint32), o["dq"].view(np.uint32))
    assert np.array_equal(g["dk"][bh].view(np.uint32), o["dk"].view(np.uint32))
    assert np.array_equal(g["dv"][bh].view(np.uint32), o["dv"].view(np.uint32))
    assert np.array_equal(g["q_hat"][bh, :N], o["qhat"])
    assert not g["q_hat"][bh, N:].any()
    assert np.array_equal(g["k_hat"][bh, :M], o["khat"])
    assert not g["k_hat"][bh, M:].any()
    assert np.array_equal(g["v_nat"][bh, :M], o["vhat"])
    assert not g["v_nat"][bh, M:].any()
    ds, ref = g["delta_s"][bh][:, :M].astype(np.float64), o["ds"]
    if cfg.causal:
        # written: the 64-key tiles whose first key is < 128 (i + 1) + coff
        coff = cfg.M - cfg.N if cfg.causal == 2 else 0
        tile0 = 64 * (np.arange(M) // 64)
        mask = tile0[None, :] - coff < 128 * (np.arange(ds.shape[0])[:, None] + 1)
        ds, ref = ds[mask], ref[mask]
    assert np.abs(ds - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("name,cfg", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_preprocess_bit_exact(name, cfg):
    q, k, v = sy.make_qkv(cfg)
    say(f"quantize {name} B={cfg.B} H={cfg.H} N={cfg.N} M={cfg.M} d={cfg.d}")
    g = gu.quantize(q, k, v, cfg.fp16, cfg.causal, cfg.smooth_v)
    for bh in range(cfg.B * cfg.H):
        check_preprocess_head(cfg, g, q, k, v, bh)


@pytest.mark.parametrize("name,heads", [("n4k", None), ("prefill32k", (0, 31)), ("video17k", (0, 95))])
def test_preprocess_bit_exact_full_size(name, heads):
    """The full workload through the same launches as the benchmark's forward (all heads on the
    GPU): every head of the 4096-token workload, and the first and last heads of the 32768-token
    prefill (512 K-mean chunks, 256 query blocks, 8 groups of 32 query blocks in the Delta S
    operand, the causal Delta S of the whole triangle) and of the ragged 17550-token video shape."""
    cfg = sy.CONFIGS[name]
    q, k, v = sy.make_qkv(cfg)
    say(f"quantize full {name} B={cfg.B} H={cfg.H} N={cfg.N} M={cfg.M} d={cfg.d}")
    g = gu.quantize(q, k, v, cfg.fp16, cfg.causal, cfg.smooth_v)
    for bh in (range(cfg.B * cfg.H) if heads is None else heads):
        check_preprocess_head(cfg, g, q, k, v, bh)


def check_output(got, ref, exact=None):
    err = np.abs(got - ref)
    assert np.isfinite(got).all()
    assert err.max() <= MAX_ABS, f"max abs err {err.max()}"
    assert err.mean() <= MEAN_ABS, f"mean abs err {err.mean()}"
    if exact is not None:
        cos = (got * exact).sum() / math.sqrt((got * got).sum() * (exact * exact).sum())
        assert cos >= MIN_COS, f"cosine {cos}"


@pytest.mark.parametrize("name,cfg", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_forward_parity_small(name, cfg):
    q, k, v = sy.make_qkv(cfg)
    say(f"forward {name} B={cfg.B} H={cfg.H} N={cfg.N} M={cfg.M} d={cfg.d} causal={cfg.causal}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v).cpu().numpy()
    s = 1 / math.sqrt(cfg.d)
    allg, allr, alle = [], [], []
    for bh in range(cfg.B * cfg.H):
        b, h = bh // cfg.H, bh % cfg.H
        allg.append(out[b, h].astype(np.float64))
        allr.append(oracle_head(cfg, q, k, v, bh))
        alle.append(oracle.exact_head(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, s))
    g, r, e = np.stack(allg), np.stack(allr), np.stack(alle)
    check_output(g, r, e if cfg.N > 1 else None)


@pytest.mark.parametrize("name", ["n4k-ragged", "prefill-causal", "video-smoothv"])
def test_forward_parity_literal_two_level(name):
    """The SAGE_ACC_VALU variant (tile sum from a zero accumulator, VALU add into O) meets
    the same bars, and differs from the default only by FP32 rounding."""
    cfg = dict(SMALL_CASES)[name]
    q, k, v = sy.make_qkv(cfg)
    say(f"forward literal two-level {name}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, acc_valu=True).cpu().numpy()
    dflt = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v).cpu().numpy()
    s = 1 / math.sqrt(cfg.d)
    g = np.stack([out[bh // cfg.H, bh % cfg.H].astype(np.float64) for bh in range(cfg.B * cfg.H)])
    r = np.stack([oracle_head(cfg, q, k, v, bh) for bh in range(cfg.B * cfg.H)])
    e = np.stack([oracle.exact_head(q[bh // cfg.H, bh % cfg.H], k[bh // cfg.H, bh % cfg.H],
                                    v[bh // cfg.H, bh % cfg.H], cfg.fp16, cfg.causal, s)
                  for bh in range(cfg.B * cfg.H)])
    check_output(g, r, e)
    assert np.abs(out - dflt).max() <= 1e-5 * max(1.0, np.abs(dflt).max())


def test_output_dtype_is_rounded_fp32():
    cfg = small("n4k", H=2, N=300, M=300)
    q, k, v = sy.make_qkv(cfg)
    say("bf16 vs fp32 output")
    o32 = gu.fwd(q, k, v, False, False, None, out_fp32=True).cpu()
    o16 = gu.fwd(q, k, v, False, False, None, out_fp32=False).cpu()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))


def test_deterministic():
    cfg = small("prefill32k", H=2, N=1000, M=1000)
    q, k, v = sy.make_qkv(cfg)
    say("determinism")
    a = gu.fwd(q, k, v, False, True, None).cpu()
    b = gu.fwd(q, k, v, False, True, None).cpu()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_nan_propagates():
    cfg = small("n4k", H=1, N=200, M=200)
    q, k, v = sy.make_qkv(cfg)
    v = v.copy()
    v[0, 0, 3, :] = 0x7FC0  # bf16 quiet NaN in one value row
    say("nan propagation")
    out = gu.fwd(q, k, v, False, False, None).cpu().numpy()
    assert np.isnan(out).all(axis=-1).all()


def test_sm_scale_argument():
    cfg = small("n4k", H=1, N=256, M=256)
    q, k, v = sy.make_qkv(cfg)
    say("explicit sm_scale")
    out = gu.fwd(q, k, v, False, False, 0.05).cpu().numpy()[0, 0].astype(np.float64)
    ref = oracle.forward_head(q[0, 0], k[0, 0], v[0, 0], False, False, 0.05)
    check_output(out, ref)


# ---------------------------------------------------------------- full workload shapes
FULL = ["n4k", "prefill32k", "prefill32k_b", "full32k", "video17k", "chunk4k_32k"]


def sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    edge = [0, 1, 127, 128, N // 2, N - 129, N - 128, N - 2, N - 1]
    rows = sorted(set([r for r in edge if 0 <= r < N] + list(rng.integers(0, N, 24))))
    return np.array(rows)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    cfg = sy.CONFIGS[name]
    q, k, v = sy.make_qkv(cfg)
    say(f"full-size forward {name} B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} causal={cfg.causal}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v)
    BH = cfg.B * cfg.H
    heads = sorted({0, BH - 1, BH // 2})
    s = 1 / math.sqrt(cfg.d)
    for bh in heads:
        b, h = bh // cfg.H, bh % cfg.H
        rows = sample_rows(cfg.N, 100 + bh)
        got = out[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        ref = oracle_head(cfg, q, k, v, bh, rows=rows)
        ex = oracle.exact_head(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, s, rows=rows)
        say(f"  head {bh}: max abs {np.abs(got - ref).max():.3g}")
        check_output(got, ref, ex)


# ---------------------------------------------------------------- the longest sequences
# One head of 262144 tokens: Delta S alone is 2 GiB (2048 query blocks x 262144 keys x 4 bytes),
# so every byte offset of the workspace and of the tiles passes 2^31; the rows sampled include
# both ends of the sequence and of the blocks around its middle.
LONG = [
    ("long256k-causal", sy.CONFIGS["prefill32k"].with_shape(H=1, N=262144, M=262144)),
    ("long256k-d64-smoothv", sy.CONFIGS["video17k"].with_shape(B=1, H=1, N=262144, M=262144)),
]


@pytest.mark.parametrize("name,cfg", LONG, ids=[n for n, _ in LONG])
def test_long_sequence_sampled(name, cfg):
    q, k, v = sy.make_qkv(cfg)
    say(f"long forward {name} N={cfg.N} d={cfg.d} causal={cfg.causal}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v)
    N = cfg.N
    rows = np.array(sorted(set([0, 1, 127, 128, N // 2 - 1, N // 2, N - 129, N - 128, N - 2, N - 1]
                               + list(np.random.default_rng(7).integers(0, N, 6)))))
    got = out[0, 0, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    ref = oracle_head(cfg, q, k, v, 0, rows=rows)
    ex = oracle.exact_head(q[0, 0], k[0, 0], v[0, 0], cfg.fp16, cfg.causal, 1 / math.sqrt(cfg.d), rows=rows)
    say(f"  max abs {np.abs(got - ref).max():.3g}")
    check_output(got, ref, ex)


# ---------------------------------------------------------------- the most heads
# B*H at the C ABI's bound (65535; the K/V kernels take the head from the grid's second
# dimension): 65535 heads of a short ragged causal sequence, in the plain head order (B*H not a
# multiple of 8), and 65528 heads of one batch in the XCD-grouped order.  Heads at both ends and
# in the middle are compared with the oracle, whole.
MANY = [
    ("B3-H21845", sy.CONFIGS["video17k"].with_shape(B=3, H=21845, N=130, M=130, causal=1, smooth_v=False)),
    ("B1-H65528", sy.CONFIGS["video17k"].with_shape(B=1, H=65528, N=130, M=130, causal=1, smooth_v=True)),
]


@pytest.mark.parametrize("path", ["int8", "mxfp4"])
@pytest.mark.parametrize("name,cfg", MANY, ids=[n for n, _ in MANY])
def test_most_heads(name, cfg, path):
    import quantized_attention_amd as qa
    BH = cfg.B * cfg.H
    checked = sorted({0, 1, cfg.H - 1, cfg.H, BH // 2, BH - 2, BH - 1} & set(range(BH)))
    # the checked heads hold the workload's seeded inputs; every other head a seeded normal fill
    # (heads are independent, so the fill only has to be valid data)
    sub = sy.make_qkv(cfg, heads=checked)
    gen = torch.Generator(device="cuda").manual_seed(4242)
    dev = []
    for t, x in enumerate(sub):
        full = torch.randn((BH, cfg.N if t == 0 else cfg.M, cfg.d), generator=gen, device="cuda").to(torch.bfloat16)
        full[torch.tensor(checked, device="cuda")] = gu.to_dev(x, cfg.fp16)
        dev.append(full.view(cfg.B, cfg.H, -1, cfg.d))
    kw = {"mxfp4": True} if path == "mxfp4" else {}
    say(f"most heads {name} path={path} B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d}")
    out = qa.sage_attn(*dev, causal=cfg.causal, smooth_v=cfg.smooth_v, out_fp32=True, **kw)
    torch.cuda.synchronize()
    flags = oracle.MXFP4 if path == "mxfp4" else 0
    s = 1 / math.sqrt(cfg.d)
    for j, bh in enumerate(checked):
        b, h = bh // cfg.H, bh % cfg.H
        got = out[b, h].cpu().numpy().astype(np.float64)
        ref, _, bound = oracle.forward_head_ties(sub[0][j], sub[1][j], sub[2][j], cfg.fp16, cfg.causal, s,
                                                 flags | (oracle.SMOOTH_V if cfg.smooth_v else 0))
        err = np.abs(got - ref)
        assert np.isfinite(got).all()
        assert err.mean() <= MEAN_ABS, (bh, err.mean())
        assert (err.max(axis=1) <= MAX_ABS + bound).all(), (bh, err.max())


# ---------------------------------------------------------------- degenerate inputs
# Inputs where the quantizers meet their edge cases: every scale at its floor (all zeros), gamma(K)
# exactly 0 (all keys equal: K^ = 0, Delta S = 0, every visible score equal), gamma(Q) and the
# block means 0 (Q = 0: the same uniform rows), and V' exactly 0 (every value row equal, with V
# smoothing: the output is V_m itself).  Each path is compared with the oracle; the zeros case
# must give exact zeros and the constant-value case with smoothing exactly the value row.
DEGENERATE = ["zeros", "equal_keys", "zero_queries", "constant_values"]
PATHS = {"int8": {}, "mxfp4": {"mxfp4": True}, "qk_fp8": {"qk_fp8": True}}


def degenerate_inputs(kind, N, M, d, seed):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((N, d)) + rng.standard_normal(d)
    K = rng.standard_normal((M, d)) + 3.0 * rng.standard_normal(d)
    V = rng.standard_normal((M, d)) + 0.5 * rng.standard_normal(d)
    if kind == "zeros":
        Q[:], K[:], V[:] = 0.0, 0.0, 0.0
    elif kind == "equal_keys":
        K[:] = K[0]
    elif kind == "zero_queries":
        Q[:] = 0.0
    elif kind == "constant_values":
        V[:] = V[0]
    bits = [sy.f32_to_bf16_bits(x.astype(np.float32))[None, None] for x in (Q, K, V)]
    return bits


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("kind", DEGENERATE)
def test_degenerate_inputs(kind, path):
    """Against the oracle with the bars of each path: mean <= 1e-3 and every row within 1e-2 plus
    the oracle's bound for its P rounding decisions near a boundary (with the FP8 matrix core's
    score error on the E4M3-QK path)."""
    from tests.test_gpu_probes import FP8_MFMA_STEP_ERR
    N, M, d = 300, 333, 128
    q, k, v = degenerate_inputs(kind, N, M, d, 91)
    s = 1 / math.sqrt(d)
    flags_of = {"int8": 0, "mxfp4": oracle.MXFP4, "qk_fp8": oracle.QK_E4M3}
    for causal in (0, 1):
        for smooth_v in (False, True):
            say(f"degenerate {kind} path={path} causal={causal} smooth_v={smooth_v}")
            got = gu.fwd(q, k, v, False, causal, None, smooth_v, **PATHS[path])[0, 0].cpu().numpy().astype(np.float64)
            ref, _, bound = oracle.forward_head_ties(
                q[0, 0], k[0, 0], v[0, 0], False, causal, s, flags_of[path] | (oracle.SMOOTH_V if smooth_v else 0),
                qk_step_err=FP8_MFMA_STEP_ERR if path == "qk_fp8" else 0.0)
            err = np.abs(got - ref)
            row = err.max(axis=1)
            say(f"  max abs {err.max():.3g}; rows with a margin {(bound > 0).sum()}; "
                f"worst beyond 1e-2 + margin {(row - MAX_ABS - bound).max():.3g}")
            assert np.isfinite(got).all()
            assert err.mean() <= MEAN_ABS
            assert (row <= MAX_ABS + bound).all()
            if kind == "zeros":
                assert (got == 0.0).all()
            if kind == "constant_values" and smooth_v:
                row_v = sy.bits_to_f32(v[0, 0, 0], False).astype(np.float64)
                assert (got == row_v[None, :]).all()
