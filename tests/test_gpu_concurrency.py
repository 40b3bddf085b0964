"""Concurrent use of the library (needs an MI355X).

The forward entry points keep no state between calls beyond a per-device capability cache:
each call takes its workspace from the caller or from stream-ordered allocation on its own
stream.  So calls issued at the same time from several host threads, each on its own stream,
must return exactly what each call returns alone (the kernels are deterministic: same inputs,
same bits).  Checked on four problems of different paths and shapes, each repeated while the
others run, through sage_attn (stream-ordered workspace) and sage_attn_fwd_ex with a caller
workspace (one per thread).  The no-allocation entry point shares one scratch array per device and
is documented to race under overlapping calls, so it is not part of this test.
"""
import sys
import threading

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

PROBLEMS = [
    ("int8-causal-d128", sy.CONFIGS["prefill32k"].with_shape(H=2, N=700, M=700), {}),
    ("int8-d64-smoothv", sy.CONFIGS["video17k"].with_shape(B=2, H=1, N=333, M=333), {}),
    ("mxfp4-d128", sy.CONFIGS["mxfp4_32k"].with_shape(H=2, N=256, M=400), {"mxfp4": True}),
    ("qkfp8-gqa", sy.CONFIGS["prefill32k_gqa"].with_shape(H=4, Hkv=2, N=300, M=500, causal=2), {"qk_fp8": True}),
]
REPEATS = 4


def _inputs(cfg):
    q, k, v = sy.make_qkv(cfg)
    return tuple(gu.to_dev(x, cfg.fp16) for x in (q, k, v))


def _call(qa, tq, tk, tv, cfg, kw, ws=None):
    if ws is None:
        return qa.sage_attn(tq, tk, tv, causal=cfg.causal, smooth_v=cfg.smooth_v, out_fp32=True, **kw)
    B, H, N, d = tq.shape
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=tq.device)
    var = qa._variant_for(tq, cfg.smooth_v, True, mxfp4=kw.get("mxfp4", False), qk_fp8=kw.get("qk_fp8", False))
    shape = qa.SageAttnShape(B, H, tk.shape[1], N, tk.shape[2], d, int(cfg.causal), 0.0, var)
    rc = qa.sage_attn_fwd_ex(shape, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), ws.data_ptr(),
                             ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == qa.SAGE_OK, qa.sage_attn_status_string(rc)
    return out


@pytest.mark.parametrize("own_workspace", [False, True], ids=["stream_ordered", "caller_workspace"])
def test_concurrent_calls_match_single_calls(own_workspace):
    import quantized_attention_amd as qa
    inputs = [_inputs(cfg) for _, cfg, _ in PROBLEMS]
    wss = []
    for (name, cfg, kw), (tq, tk, tv) in zip(PROBLEMS, inputs):
        var = qa._variant_for(tq, cfg.smooth_v, True, mxfp4=kw.get("mxfp4", False), qk_fp8=kw.get("qk_fp8", False))
        B, H, N, d = tq.shape
        shape = qa.SageAttnShape(B, H, tk.shape[1], N, tk.shape[2], d, int(cfg.causal), 0.0, var)
        n = qa.sage_attn_workspace_bytes_ex(shape)
        wss.append(torch.empty(n, dtype=torch.uint8, device="cuda") if own_workspace else None)
    ref = []
    for (name, cfg, kw), (tq, tk, tv), ws in zip(PROBLEMS, inputs, wss):
        say(f"single call {name}")
        ref.append(_call(qa, tq, tk, tv, cfg, kw, ws).cpu().numpy())
    torch.cuda.synchronize()

    results = [[None] * REPEATS for _ in PROBLEMS]
    errors = []
    start = threading.Barrier(len(PROBLEMS))

    def worker(i):
        try:
            name, cfg, kw = PROBLEMS[i]
            tq, tk, tv = inputs[i]
            s = torch.cuda.Stream()  # default priority
            start.wait()
            with torch.cuda.stream(s):
                outs = [_call(qa, tq, tk, tv, cfg, kw, wss[i]) for _ in range(REPEATS)]
            s.synchronize()
            results[i] = [o.cpu().numpy() for o in outs]
        except Exception as e:  # reported on the main thread
            errors.append((i, repr(e)))

    say(f"{len(PROBLEMS)} threads x {REPEATS} calls, own workspace: {own_workspace}")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(PROBLEMS))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (name, _, _) in enumerate(PROBLEMS):
        for r in range(REPEATS):
            assert np.array_equal(results[i][r], ref[i]), f"{name}: call {r} differs from the single call"
