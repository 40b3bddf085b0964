"""The forward under HIP graph capture (needs an MI355X).

A forward call with a caller workspace (sage_attn_fwd_ex) or with none (sage_attn_fwd_noalloc)
only enqueues kernels on its stream: no allocation, memset, event record or host
synchronization, so it can be captured into a graph and replayed.  The captured call is
replayed several times, with eager work and synchronizations between the replays and the inputs
rewritten in place before some of them; every replay must equal, bit for bit, the eager call on
the same inputs (the kernels are deterministic).
"""
import sys

import numpy as np
import pytest
import torch

from quantized_attention_amd import synthetic as sy

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_attention_amd
    quantized_attention_amd.load_library()


from tests import gpu_util as gu  # noqa: E402

CASES = [
    ("int8-causal-d128", sy.CONFIGS["prefill32k"].with_shape(H=2, N=700, M=700), 0),
    ("mxfp4-d64-smoothv", sy.CONFIGS["video17k"].with_shape(B=2, H=1, N=333, M=333), 1),
]


@pytest.mark.parametrize("entry", ["fwd_ex", "noalloc"])
@pytest.mark.parametrize("name,cfg,mx", CASES, ids=[c[0] for c in CASES])
def test_captured_forward_replays_match_eager(name, cfg, mx, entry):
    import quantized_attention_amd as qa
    q, k, v = sy.make_qkv(cfg)
    tq, tk, tv = (gu.to_dev(x, cfg.fp16) for x in (q, k, v))
    B, H, N, d = tq.shape
    var = qa._variant_for(tq, cfg.smooth_v, True, mxfp4=bool(mx))
    shape = qa.SageAttnShape(B, H, tk.shape[1], N, tk.shape[2], d, int(cfg.causal), 0.0, var)
    out = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(qa.sage_attn_workspace_bytes_ex(shape) + 256, dtype=torch.uint8, device="cuda")
    ws_ptr = (ws.data_ptr() + 255) // 256 * 256
    ws_bytes = qa.sage_attn_workspace_bytes_ex(shape)

    def call(stream):
        if entry == "fwd_ex":
            rc = qa.sage_attn_fwd_ex(shape, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), ws_ptr,
                                     ws_bytes, stream)
        else:
            rc = qa.sage_attn_fwd_noalloc(shape, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), stream)
        assert rc == qa.SAGE_OK, qa.sage_attn_status_string(rc)

    def eager():
        call(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        return out.cpu().numpy().copy()

    ref0 = eager()
    # a second input set, written into the same buffers before some replays
    q2, k2, v2 = (x[..., ::-1, :].copy() for x in (q, k, v))
    tq2, tk2, tv2 = (gu.to_dev(x, cfg.fp16) for x in (q2, k2, v2))
    saved = (tq.clone(), tk.clone(), tv.clone())
    tq.copy_(tq2), tk.copy_(tk2), tv.copy_(tv2)
    ref1 = eager()
    tq.copy_(saved[0]), tk.copy_(saved[1]), tv.copy_(saved[2])
    torch.cuda.synchronize()

    say(f"capture {name} via {entry}")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()  # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(s.cuda_stream)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        call(s.cuda_stream)
    torch.cuda.synchronize()
    for r, which in enumerate([0, 0, 1, 0, 1]):
        src = (tq2, tk2, tv2) if which else saved
        tq.copy_(src[0]), tk.copy_(src[1]), tv.copy_(src[2])
        out.fill_(float("nan"))
        _ = (tq.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, ref1 if which else ref0), f"replay {r} differs from the eager call"
