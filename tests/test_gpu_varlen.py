"""GPU checks of variable-length batches (sage_attn_varlen_fwd; needs an MI355X).

Source: "Handling Varying Sequence Lengths with VarLen Kernels" (a ragged batch packed along
the token axis with cumulative offsets).  The header defines each sequence's result as the
dense forward of that sequence alone, so:
  * every sequence of a packed batch equals, bit for bit, sage_attn on that sequence (its
    own means, scales, query blocks, Delta S and causal alignment), for the INT8/FP8 path,
    the E4M3 QK knob and the MXFP4 variant, with grouped heads, both causal alignments,
    ragged lengths, a one-token sequence and lengths that are not tile multiples;
  * one sequence per batch is also checked against the oracle (max |err| <= 1e-2, mean <=
    1e-3, FP32 output);
  * rows that see no key are 0: a sequence without keys, and causal = 2 with 128 more
    queries than keys, whose other rows equal the dense forward of the last queries.
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


import quantized_attention_amd as qa  # noqa: E402
from tests import gpu_util as gu  # noqa: E402


def make_batch(base, lens, seed0):
    """Per-sequence seeded inputs: lists of [H, N_b, d] / [Hkv, M_b, d] uint16 bits."""
    qs, ks, vs = [], [], []
    for b, (n, m) in enumerate(lens):
        cfg = base.with_shape(B=1, N=max(n, 1), M=max(m, 1), seed=seed0 + b)
        q, k, v = sy.make_qkv(cfg)
        qs.append(q[0, :, :n])
        ks.append(k[0, :, :m])
        vs.append(v[0, :, :m])
    return qs, ks, vs


def pack(parts):
    """[H, T_b, d] per sequence -> [total, H, d] and the int32 offsets."""
    cu = np.concatenate([[0], np.cumsum([p.shape[1] for p in parts])]).astype(np.int32)
    packed = np.concatenate([p.transpose(1, 0, 2) for p in parts], axis=0)
    return np.ascontiguousarray(packed), cu


def run_varlen(base, qs, ks, vs, causal, mxfp4=False, qk_fp8=False):
    qp, cuq = pack(qs)
    kp, cuk = pack(ks)
    vp, _ = pack(vs)
    tq, tk, tv = gu.to_dev(qp, base.fp16), gu.to_dev(kp, base.fp16), gu.to_dev(vp, base.fp16)
    out = torch.full((qp.shape[0], qp.shape[1], qp.shape[2]), float("nan"), dtype=torch.float32, device="cuda")
    out = qa.sage_attn_varlen(tq, tk, tv, torch.from_numpy(cuq).cuda(), torch.from_numpy(cuk).cuda(),
                              int(np.diff(cuq).max()), int(max(np.diff(cuk).max(), 1)), causal=causal,
                              smooth_v=base.smooth_v, out_fp32=True, out=out, mxfp4=mxfp4, qk_fp8=qk_fp8)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    return [o[cuq[b]:cuq[b + 1]].transpose(1, 0, 2) for b in range(len(qs))]


def dense(base, q, k, v, causal, mxfp4=False, qk_fp8=False):
    return gu.fwd(q[None], k[None], v[None], base.fp16, causal, None, base.smooth_v, mxfp4=mxfp4,
                  qk_fp8=qk_fp8).cpu().numpy()[0]


LENS = [(300, 300), (1, 1), (129, 700), (64, 64), (700, 129), (5, 3)]
CASES = [
    # name, base config, lengths, causal, mxfp4, qk_fp8
    ("noncausal-d64-smoothv", sy.CONFIGS["video17k"].with_shape(H=2), LENS, 0, False, False),
    ("causal1-d128", sy.CONFIGS["prefill32k"].with_shape(H=2), LENS, 1, False, False),
    ("causal2-d128-N<=M", sy.CONFIGS["prefill32k"].with_shape(H=2),
     [(300, 300), (1, 1), (129, 700), (64, 64), (5, 130)], 2, False, False),
    ("gqa-causal1", sy.CONFIGS["prefill32k_gqa"].with_shape(H=8, Hkv=2), LENS, 1, False, False),
    ("mxfp4-noncausal", sy.CONFIGS["mxfp4_32k"].with_shape(H=2), LENS, 0, True, False),
    ("qkfp8-causal1", sy.CONFIGS["prefill32k"].with_shape(H=2), LENS, 1, False, True),
]


@pytest.mark.parametrize("name,base,lens,causal,mx,f8", CASES, ids=[c[0] for c in CASES])
def test_varlen_equals_dense_per_sequence(name, base, lens, causal, mx, f8):
    qs, ks, vs = make_batch(base, lens, 2000)
    say(f"varlen {name}: lengths {lens}")
    outs = run_varlen(base, qs, ks, vs, causal, mx, f8)
    for b, (n, m) in enumerate(lens):
        ref = dense(base, qs[b], ks[b], vs[b], causal, mx, f8)
        assert np.array_equal(outs[b].view(np.uint32), ref.view(np.uint32)), f"sequence {b} (N={n}, M={m})"


def test_varlen_parity_vs_oracle():
    base = sy.CONFIGS["prefill32k_gqa"].with_shape(H=4, Hkv=2)
    lens = [(200, 333), (77, 77), (130, 64)]
    qs, ks, vs = make_batch(base, lens, 3000)
    say(f"varlen oracle parity: lengths {lens}")
    outs = run_varlen(base, qs, ks, vs, 1)
    s = 1 / math.sqrt(base.d)
    errs = []
    for b in range(len(lens)):
        for h in range(base.H):
            ref = oracle.forward_head(qs[b][h], ks[b][h // 2], vs[b][h // 2], base.fp16, 1, s, 0)
            errs.append(np.abs(outs[b][h].astype(np.float64) - ref).ravel())
    e = np.concatenate(errs)
    say(f"  max abs {e.max():.3g} mean abs {e.mean():.3g}")
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS


def test_varlen_rows_without_keys():
    base = sy.CONFIGS["prefill32k"].with_shape(H=2)
    # sequence 0: 128 more queries than keys under causal = 2; sequence 1: no keys at all
    lens = [(128 + 200, 200), (50, 0), (100, 300)]
    qs, ks, vs = make_batch(base, lens, 4000)
    say(f"varlen rows without keys: lengths {lens}")
    outs = run_varlen(base, qs, ks, vs, 2)
    assert not outs[0][:, :128].any() and not np.signbit(outs[0][:, :128]).any()
    assert not outs[1].any() and not np.signbit(outs[1]).any()
    # the rows after the first 128 see keys: the dense forward of the last 200 queries (their
    # 128-query blocks coincide with those of the whole sequence)
    ref = dense(base, np.ascontiguousarray(qs[0][:, 128:]), ks[0], vs[0], 2)
    assert np.array_equal(outs[0][:, 128:].view(np.uint32), ref.view(np.uint32))
    ref2 = dense(base, qs[2], ks[2], vs[2], 2)
    assert np.array_equal(outs[2].view(np.uint32), ref2.view(np.uint32))
