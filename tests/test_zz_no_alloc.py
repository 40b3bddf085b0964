"""The no-allocation entry point (sage_attn_fwd_noalloc) against the allocating one
(sage_attn_fwd_ex with a stream-ordered workspace), through the C ABI, on an MI355X.

Both run the same kernels on the same inputs, so their outputs must agree bit for bit (the
forward is deterministic); the bar of the parity tests (max |err| <= 1e-2, mean <= 1e-3) is
implied.  Two calls in a row, the second on a smaller problem, show that the shared scratch
array is reused correctly (no state of the first call leaks into the second); a third call
repeats the first shape after the smaller one.
"""
import sys

import numpy as np
import pytest
import torch

import quantized_attention_amd as qa
from quantized_attention_amd import synthetic as sy

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qa.load_library()


def _inputs(cfg):
    q, k, v = sy.make_qkv(cfg)
    dt = torch.float16 if cfg.fp16 else torch.bfloat16
    return [torch.from_numpy(x.view(np.int16)).view(dt).cuda() for x in (q, k, v)]


def _both(cfg, variant_extra=0):
    q, k, v = _inputs(cfg)
    var = (qa.SAGE_IN_FP16 if cfg.fp16 else qa.SAGE_IN_BF16) | qa.SAGE_OUT_FP32 | variant_extra
    if cfg.smooth_v:
        var |= qa.SAGE_SMOOTH_V
    shape = qa.SageAttnShape(cfg.B, cfg.H, cfg.hkv, cfg.N, cfg.M, cfg.d, int(cfg.causal), 0.0, var)
    assert qa.sage_attn_workspace_bytes_ex(shape) <= qa.SAGE_NOALLOC_MAX_BYTES
    stream = torch.cuda.current_stream().cuda_stream
    ref = torch.empty((cfg.B, cfg.H, cfg.N, cfg.d), dtype=torch.float32, device="cuda")
    got = torch.full_like(ref, float("nan"))
    rc = qa.sage_attn_fwd_ex(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), ref.data_ptr(), None, 0, stream)
    assert rc == qa.SAGE_OK
    rc = qa.sage_attn_fwd_noalloc(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), got.data_ptr(), stream)
    assert rc == qa.SAGE_OK
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


def test_noalloc_matches_allocating_entry_point():
    big = sy.CONFIGS["prefill32k"].with_shape(H=8, N=2048, M=2048)
    small = sy.CONFIGS["video17k"].with_shape(B=1, H=2, N=600, M=600)
    for name, cfg, extra in (("first", big, 0), ("second, smaller", small, 0), ("third, first shape again", big, 0),
                             ("mxfp4, smaller still", small.with_shape(N=333, M=333), qa.SAGE_PATH_MXFP4)):
        say(f"noalloc {name}: B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} causal={cfg.causal} variant+={extra:#x}")
        got, ref = _both(cfg, extra)
        err = np.abs(got.astype(np.float64) - ref)
        say(f"  max abs {err.max():.3g}")
        assert np.isfinite(got).all()
        assert err.max() <= 1e-2 and err.mean() <= 1e-3
        assert np.array_equal(got, ref)


def test_noalloc_rejects_oversized_problem():
    cfg = sy.CONFIGS["prefill32k"]
    shape = qa.SageAttnShape(cfg.B, cfg.H, cfg.H, cfg.N, cfg.M, cfg.d, 1, 0.0, qa.SAGE_IN_BF16)
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    p = x.data_ptr()
    assert qa.sage_attn_fwd_noalloc(shape, p, p, p, p, None) == qa.SAGE_ERR_NO_MEMORY
