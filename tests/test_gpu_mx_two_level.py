"""GPU parity of the MXFP4 variant with two-level P quantization (SAGE_MX_P_TWO_LEVEL) against
the CPU oracle (needs an MI355X).

Source: "SageAttention3" summary, 3.4 "Two-Level Quantization for the Attention Map P" (level
one: each row of a tile's P~ divided by an FP32 factor from the row maximum; level two: the
E2M1 block quantizer; the tile's product multiplied back by the factor), with the reading
s1 = rowmax / 6 for E8M0 block scales.

Bars: the output within mean |err| <= 1e-3 of the oracle run with the same knob (FP32
output), and every row within max |err| <= 1e-2 plus the oracle's bound for that row's
near-boundary decisions: P rounding decisions whose input lies within 2^-16 (relative) of a
rounding boundary, where the kernel's FP32 exponentials may round the other way (either code
is a correct rounding of the method's value; one step at the top of the E2M1 grid, 4 <-> 6, is
a third of the row maximum).  The bound is the change of each such P^ value times its key's
largest V value, carried through the tile loop like O; it is 0 on rows without such a
decision.  On the lossless two-level construction (every quantizer exact), the output equals
textbook attention up to FP32 arithmetic, while the direct P quantizer does not.
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
from tests.test_oracle_mx import f16, textbook, two_level_case  # noqa: E402

CASES = [
    ("tiny-d64", sy.CONFIGS["tiny"]),
    ("mx-ragged", sy.CONFIGS["mxfp4_32k"].with_shape(H=2, N=600, M=600)),
    ("causal-700", sy.CONFIGS["prefill32k"].with_shape(H=2, N=700, M=700)),
    ("smoothv-d64", sy.CONFIGS["video17k"].with_shape(B=2, H=1, N=333, M=333)),
    ("one-token", sy.Config("one", 1, 1, 1, 1, 64, "bf16", False, sy.Dist(), 79)),
    ("few-tokens", sy.Config("few", 1, 3, 5, 3, 128, "fp16", False, sy.Dist(k_off_std=1.0), 80)),
    ("causal-br-N<M", sy.CONFIGS["mxfp4_32k"].with_shape(H=2, N=300, M=1000, causal=2)),
]
FLAGS = oracle.MXFP4 | oracle.MX_P_TWO_LEVEL


def run(cfg, q, k, v, two=True):
    return gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, mxfp4=True,
                  mx_p_two_level=two).cpu().numpy()


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_two_level_parity_small(name, cfg):
    q, k, v = sy.make_qkv(cfg)
    say(f"mx two-level forward {name} B={cfg.B} H={cfg.H} N={cfg.N} M={cfg.M} d={cfg.d} causal={cfg.causal}")
    out = run(cfg, q, k, v)
    s = 1 / math.sqrt(cfg.d)
    fl = FLAGS | (oracle.SMOOTH_V if cfg.smooth_v else 0)
    err, bnd = [], []
    for bh in range(cfg.B * cfg.H):
        b, h = bh // cfg.H, bh % cfg.H
        ref, _, bd = oracle.forward_head_ties(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, s, fl)
        err.append(np.abs(out[b, h].astype(np.float64) - ref))
        bnd.append(bd)
    err, bnd = np.stack(err), np.stack(bnd)
    rmax = err.max(axis=-1)
    say(f"  max abs {err.max():.3g} mean abs {err.mean():.3g}; {(bnd > 0).sum()} rows with near-boundary "
        f"decisions (bound up to {bnd.max():.3g}); max abs beyond the bound {(rmax - bnd).max():.3g}")
    assert np.isfinite(out).all()
    assert err.mean() <= MEAN_ABS
    assert (rmax <= MAX_ABS + bnd).all()


@pytest.mark.parametrize("N,M,d,causal", [(256, 256, 64, False), (256, 256, 64, True), (192, 512, 128, False)])
def test_two_level_lossless_construction(N, M, d, causal):
    Q, K, V = two_level_case(50 + N + d, N, M, d)
    q, k, v = (f16(x)[None, None] for x in (Q, K, V))
    sm = math.log(1.5)
    say(f"mx two-level lossless N={N} M={M} d={d} causal={causal}")
    ex = textbook(Q, K, V, sm, causal)
    two = gu.fwd(q, k, v, True, causal, sm, mxfp4=True, mx_p_two_level=True).cpu().numpy()[0, 0]
    direct = gu.fwd(q, k, v, True, causal, sm, mxfp4=True).cpu().numpy()[0, 0]
    say(f"  two-level {np.abs(two - ex).max():.3g}  direct {np.abs(direct - ex).max():.3g}")
    assert np.abs(two - ex).max() < 1e-5
    assert np.abs(direct - ex).max() > 1e-3


def test_two_level_full_size_sampled():
    cfg = sy.CONFIGS["mxfp4_32k"]
    q, k, v = sy.make_qkv(cfg)
    say(f"mx two-level full-size forward B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d}")
    out = gu.fwd(q, k, v, cfg.fp16, cfg.causal, None, cfg.smooth_v, mxfp4=True, mx_p_two_level=True)
    BH = cfg.B * cfg.H
    s = 1 / math.sqrt(cfg.d)
    rng = np.random.default_rng(6)
    for bh in sorted({0, BH - 1}):
        b, h = bh // cfg.H, bh % cfg.H
        rows = np.array(sorted(set([0, 1, 127, 128, cfg.N // 2, cfg.N - 1] + list(rng.integers(0, cfg.N, 12)))))
        got = out[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        ref, _, bd = oracle.forward_head_ties(q[b, h], k[b, h], v[b, h], cfg.fp16, cfg.causal, s, FLAGS, rows=rows)
        err = np.abs(got - ref)
        say(f"  head {bh}: max abs {err.max():.3g}, {(bd > 0).sum()} rows with near-boundary decisions "
            f"(bound up to {bd.max():.3g})")
        assert err.mean() <= MEAN_ABS
        assert (err.max(axis=-1) <= MAX_ABS + bd).all()


@pytest.mark.parametrize("causal", [False, True])
def test_two_level_large_score_gaps(causal):
    """Tiles whose row maximum lies far below the running maximum (76 and 185 octaves here, and a
    later tile 4 octaves below): the level-one rescale of O must stay finite.  All query rows equal
    (Q^ = 0, S = Delta S sm_scale); K channel 0 = 1024 on key 0, 600 on every key of tile 1, 0 on
    tile 2, 1000 on one key of tile 3.  The oracle (FP64) gives the reference; every path of the MX
    variant, and the INT8/FP8 path, must stay within the usual bars."""
    N = M = 256
    d = 64
    rng = np.random.default_rng(31)
    Q = np.zeros((N, d)); Q[:, 0] = 1.0
    K = np.zeros((M, d)); K[0, 0] = 1024.0; K[64:128, 0] = 600.0; K[200, 0] = 1000.0
    V = rng.choice([0.0, 0.5, 1.0, 1.5, 2.0, 3.0], (M, d)) * rng.choice([-1.0, 1.0], (M, d))
    q, k, v = (f16(x) for x in (Q, K, V))
    sm = 0.125
    for flags, kw in ((FLAGS, dict(mxfp4=True, mx_p_two_level=True)), (oracle.MXFP4, dict(mxfp4=True)), (0, {})):
        say(f"large score gaps, causal={causal}, {kw or 'int8/fp8'}")
        got = gu.fwd(q[None, None], k[None, None], v[None, None], True, causal, sm, **kw).cpu().numpy()[0, 0]
        ref, _, bd = oracle.forward_head_ties(q, k, v, True, causal, sm, flags)
        err = np.abs(got.astype(np.float64) - ref)
        say(f"  max abs {err.max():.3g} mean abs {err.mean():.3g}")
        assert np.isfinite(got).all()
        assert err.mean() <= MEAN_ABS
        assert (err.max(axis=-1) <= MAX_ABS + bd).all()
