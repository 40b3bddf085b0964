"""The C-ABI library loads, exports every symbol include/sage_attn.h declares, and rejects
bad arguments before touching a device (CPU-only; no compute calls)."""
import ctypes
import os
import re

import pytest

import quantized_attention_amd as qa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sage_attn.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\**\s*(sage_attn_[a-z_]+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["sage_attn_fwd", "sage_attn_fwd_ws", "sage_attn_workspace_bytes",
                            "sage_attn_quantize", "sage_attn_set_profile_events",
                            "sage_attn_status_string", "sage_attn_version", "sage_attn_fwd_ex",
                            "sage_attn_workspace_bytes_ex", "sage_attn_quantize_ex",
                            "sage_attn_varlen_workspace_bytes", "sage_attn_varlen_fwd",
                            "sage_attn_train_workspace_bytes", "sage_attn_train_fwd", "sage_attn_train_bwd",
                            "sage_attn_fwd_noalloc"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(qa.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert hasattr(qa, name), name  # the binding keeps the same names


def test_status_strings_and_version():
    assert qa.sage_attn_version() >= 100
    for s in (qa.SAGE_OK, qa.SAGE_ERR_INVALID_ARG, qa.SAGE_ERR_UNSUPPORTED, qa.SAGE_ERR_NO_MEMORY,
              qa.SAGE_ERR_LAUNCH, qa.SAGE_ERR_DEVICE):
        assert qa.sage_attn_status_string(s)
    assert qa.sage_attn_status_string(123) == "unknown status"


def test_argument_errors_are_reported_before_any_device_work():
    f = qa.sage_attn_fwd
    A = 256  # a 16-byte aligned stand-in address; never dereferenced on these paths
    assert f(0, A, A, A, 1, 1, 64, 64, 64, 0, 0.0, 0, 0) == qa.SAGE_ERR_INVALID_ARG   # null q
    assert f(A + 2, A, A, A, 1, 1, 64, 64, 64, 0, 0.0, 0, 0) == qa.SAGE_ERR_INVALID_ARG  # misaligned
    assert f(A, A, A, A, 0, 1, 64, 64, 64, 0, 0.0, 0, 0) == qa.SAGE_ERR_INVALID_ARG   # B = 0
    assert f(A, A, A, A, 1, 1, 0, 64, 64, 0, 0.0, 0, 0) == qa.SAGE_ERR_INVALID_ARG   # N = 0
    assert f(A, A, A, A, 1, 1, 64, 64, 96, 0, 0.0, 0, 0) == qa.SAGE_ERR_UNSUPPORTED  # d = 96
    assert f(A, A, A, A, 1, 1, 65, 64, 64, 2, 0.0, 0, 0) == qa.SAGE_ERR_UNSUPPORTED  # bottom-right, N > M
    assert f(A, A, A, A, 1, 1, 64, 64, 64, 3, 0.0, 0, 0) == qa.SAGE_ERR_INVALID_ARG  # causal mode 3
    assert f(A, A, A, A, 1, 1, 64, 64, 64, -1, 0.0, 0, 0) == qa.SAGE_ERR_INVALID_ARG
    assert f(A, A, A, A, 1, 1, 64, 64, 64, 0, 0.0, 0x8, 0) == qa.SAGE_ERR_INVALID_ARG  # unknown bit
    both = qa.SAGE_PATH_MXFP4 | qa.SAGE_QK_FP8  # two Q K^T formats at once
    assert f(A, A, A, A, 1, 1, 64, 64, 64, 0, 0.0, both, 0) == qa.SAGE_ERR_INVALID_ARG
    assert qa.sage_attn_workspace_bytes(1, 1, 64, 64, 64, 0, both) == 0
    # two-level P needs the MX path and accumulates through the MFMA C operand
    for bad in (qa.SAGE_MX_P_TWO_LEVEL, qa.SAGE_MX_P_TWO_LEVEL | qa.SAGE_PATH_MXFP4 | qa.SAGE_ACC_VALU):
        assert f(A, A, A, A, 1, 1, 64, 64, 64, 0, 0.0, bad, 0) == qa.SAGE_ERR_INVALID_ARG
    assert qa.sage_attn_workspace_bytes(1, 1, 64, 64, 64, 0, qa.SAGE_MX_P_TWO_LEVEL | qa.SAGE_PATH_MXFP4) == \
        qa.sage_attn_workspace_bytes(1, 1, 64, 64, 64, 0, qa.SAGE_PATH_MXFP4)
    # E4M3 Q^ / K^ take the INT8 layouts: the same workspace
    assert qa.sage_attn_workspace_bytes(1, 4, 300, 500, 128, 1, qa.SAGE_QK_FP8) == \
        qa.sage_attn_workspace_bytes(1, 4, 300, 500, 128, 1, 0)
    ws = qa.sage_attn_workspace_bytes(1, 1, 64, 64, 64, 0, 0)
    assert ws > 0
    assert qa.sage_attn_fwd_ws(A, A, A, A, 1, 1, 64, 64, 64, 0, 0.0, 0, A, ws - 1, 0) == qa.SAGE_ERR_NO_MEMORY
    assert qa.sage_attn_fwd_ws(A, A, A, A, 1, 1, 64, 64, 64, 0, 0.0, 0, A + 16, ws, 0) == qa.SAGE_ERR_INVALID_ARG
    assert qa.sage_attn_workspace_bytes(1, 1, 64, 64, 80, 0, 0) == 0
    assert qa.sage_attn_quantize(0, A, A, 1, 1, 64, 64, 64, 0, 0, qa.QuantViews(), 0) == qa.SAGE_ERR_INVALID_ARG


def test_causal_modes_accept_uneven_lengths():
    # causal = 1 (first query aligned with the first key) takes any N, M; causal = 2 (last with
    # last) takes N <= M: both size a workspace, N != M included
    for causal, N, M in [(1, 64, 200), (1, 200, 64), (2, 64, 200), (2, 200, 200)]:
        assert qa.sage_attn_workspace_bytes(1, 1, N, M, 64, causal, 0) > 0
    assert qa.sage_attn_workspace_bytes(1, 1, 200, 64, 64, 2, 0) == 0
    # grid bounds: B*H <= 65535, and B*H times the query blocks / key tiles below 2^24
    assert qa.sage_attn_workspace_bytes(1, 65536, 64, 64, 64, 0, 0) == 0
    assert qa.sage_attn_workspace_bytes(1, 65535, 128, 64, 64, 0, 0) > 0
    assert qa.sage_attn_workspace_bytes(1, 65535, 256 * 128, 256 * 64, 64, 0, 0) > 0
    assert qa.sage_attn_workspace_bytes(1, 65535, 128, 257 * 64, 64, 0, 0) == 0
    assert qa.sage_attn_workspace_bytes(1, 65535, 257 * 128, 64, 64, 0, 0) == 0


def test_extended_shape_checks():
    S = qa.SageAttnShape
    A = 256
    assert qa.sage_attn_workspace_bytes_ex(None) == 0
    assert qa.sage_attn_fwd_ex(None, A, A, A, A, None, 0, None) == qa.SAGE_ERR_INVALID_ARG
    assert qa.sage_attn_fwd_ex(S(1, 8, 3, 64, 64, 64, 0, 0.0, 0), A, A, A, A, None, 0, None) == qa.SAGE_ERR_INVALID_ARG
    assert qa.sage_attn_fwd_ex(S(1, 8, 0, 64, 64, 64, 0, 0.0, 0), A, A, A, A, None, 0, None) == qa.SAGE_ERR_INVALID_ARG
    assert qa.sage_attn_workspace_bytes_ex(S(1, 8, 3, 64, 64, 64, 0, 0.0, 0)) == 0
    # same shape, Hkv = Hq: the plain entry point's size; grouped heads shrink the K/V side only
    full = qa.sage_attn_workspace_bytes_ex(S(1, 8, 8, 4096, 4096, 128, 0, 0.0, 0))
    assert full == qa.sage_attn_workspace_bytes(1, 8, 4096, 4096, 128, 0, 0)
    grouped = qa.sage_attn_workspace_bytes_ex(S(1, 8, 2, 4096, 4096, 128, 0, 0.0, 0))
    assert 0 < grouped < full
    ws = qa.sage_attn_workspace_bytes_ex(S(1, 8, 2, 64, 64, 64, 0, 0.0, 0))
    assert qa.sage_attn_fwd_ex(S(1, 8, 2, 64, 64, 64, 0, 0.0, 0), A, A, A, A, A, ws - 1, None) == qa.SAGE_ERR_NO_MEMORY
    assert qa.sage_attn_fwd_ex(S(1, 8, 2, 64, 64, 64, 0, 0.0, 0), A, A, A, A, A + 16, ws, None) == qa.SAGE_ERR_INVALID_ARG


def test_workspace_grows_with_problem():
    a = qa.sage_attn_workspace_bytes(1, 32, 4096, 4096, 128, 0, 0)
    b = qa.sage_attn_workspace_bytes(1, 32, 32768, 32768, 128, 1, 0)
    assert 0 < a < b
    # dominated by Delta S (nqb * Mp floats per head) and the three quantized tensors
    assert b < 2 * 1024 ** 3


def test_varlen_shape_checks():
    V = qa.SageAttnVarlenShape
    A = 256  # stand-in device addresses, never dereferenced on these paths

    def shape(**kw):
        f = dict(batch=3, Hq=4, Hkv=2, d=64, total_q=500, total_k=700, max_seqlen_q=300, max_seqlen_k=400,
                 cu_seqlens_q=A, cu_seqlens_k=A + 64, causal=1, sm_scale=0.0, variant=0)
        f.update(kw)
        return V(**f)

    # the workspace is the dense layout of `batch` sequences of the bound lengths
    assert qa.sage_attn_varlen_workspace_bytes(shape()) == qa.sage_attn_workspace_bytes_ex(
        qa.SageAttnShape(3, 4, 2, 300, 400, 64, 1, 0.0, 0))
    # causal = 2 with a longer query bound is allowed (rows without keys are written as 0)
    assert qa.sage_attn_varlen_workspace_bytes(shape(causal=2, max_seqlen_q=500, max_seqlen_k=100)) > 0
    bad = [shape(batch=0), shape(total_q=0), shape(total_k=0), shape(max_seqlen_q=0), shape(Hkv=3),
           shape(cu_seqlens_q=None), shape(cu_seqlens_k=None), shape(cu_seqlens_q=A + 2), shape(causal=3),
           shape(variant=qa.SAGE_PATH_MXFP4 | qa.SAGE_QK_FP8)]
    for s in bad:
        assert qa.sage_attn_varlen_workspace_bytes(s) == 0
        assert qa.sage_attn_varlen_fwd(s, A, A, A, A, None, 0, None) == qa.SAGE_ERR_INVALID_ARG
    assert qa.sage_attn_varlen_workspace_bytes(shape(d=96)) == 0
    assert qa.sage_attn_varlen_fwd(shape(d=96), A, A, A, A, None, 0, None) == qa.SAGE_ERR_UNSUPPORTED
    assert qa.sage_attn_varlen_workspace_bytes(None) == 0
    ws = qa.sage_attn_varlen_workspace_bytes(shape())
    assert qa.sage_attn_varlen_fwd(shape(), A, A, A, A, A, ws - 1, None) == qa.SAGE_ERR_NO_MEMORY
    assert qa.sage_attn_varlen_fwd(shape(), A + 8, A, A, A, None, 0, None) == qa.SAGE_ERR_INVALID_ARG



def test_train_binding_rejects_mismatched_tensors():
    """The SageBwd wrappers check every tensor's shape and dtype against q before the library
    sees a pointer (CPU tensors: the shape checks come before the device check)."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros(1, 4, 64, 64, dtype=bf)
    k = torch.zeros(1, 4, 96, 64, dtype=bf)
    grouped = torch.zeros(1, 2, 96, 64, dtype=bf)
    bad_forward = [(q, grouped, grouped), (q, k, torch.zeros(1, 4, 80, 64, dtype=bf)),
                   (q, torch.zeros(1, 4, 96, 128, dtype=bf), torch.zeros(1, 4, 96, 128, dtype=bf))]
    for a, b, c in bad_forward:
        with pytest.raises(ValueError):
            qa.sage_attn_train_forward(a, b, c)
    with pytest.raises(ValueError):  # right shapes, host tensors
        qa.sage_attn_train_forward(q, k, k)
    out = torch.zeros_like(q)
    lse = torch.zeros(1, 4, 64, dtype=torch.float32)
    bad_backward = [
        dict(k=grouped, v=grouped),
        dict(dout=torch.zeros(1, 4, 63, 64, dtype=bf)),
        dict(out=torch.zeros(1, 4, 64, 128, dtype=bf)),
        dict(lse=torch.zeros(1, 4, 65, dtype=torch.float32)),
        dict(lse=torch.zeros(1, 4, 64, dtype=torch.float64)),
        dict(out=torch.zeros(1, 4, 64, 64, dtype=torch.float16)),
    ]
    for change in bad_backward:
        args = dict(q=q, k=k, v=k, out=out, dout=q, lse=lse)
        args.update(change)
        with pytest.raises((ValueError, TypeError)):
            qa.sage_attn_train_backward(**args)


def test_train_workspace_holds_the_pair_buffer_up_to_its_limit():
    """The backward keeps every (128-query, 64-key) block pair's dS^ in its workspace (one 2192-byte
    record per wave of the query block: 2048 code bytes, 32 row sums, the pair's multiplier,
    padding) unless SAGE_TRAIN_RECOMPUTE_DS asks for the recomputing dQ kernel, or the buffer
    would pass 16 GiB; the training variant bits outside the known ones are rejected."""
    def ws(B, H, N, M, d, causal, var):
        return qa.sage_attn_train_workspace_bytes(qa.SageAttnShape(B, H, H, N, M, d, causal, 0.0, var))
    pair = 4 * 2192
    for B, H, N, M, d in ((1, 32, 8192, 8192, 128), (2, 3, 333, 700, 64)):
        pairs = B * H * -(-N // 128) * -(-M // 64)
        stored, recomputed = ws(B, H, N, M, d, 1, 0), ws(B, H, N, M, d, 1, qa.SAGE_TRAIN_RECOMPUTE_DS)
        assert stored > 0 and recomputed > 0
        assert pairs * pair <= stored - recomputed < pairs * pair + 256
    # 32 heads of 32768 tokens: 4 Mi pairs, 36 GB of pair buffer -> the recomputing form
    big = (1, 32, 32768, 32768, 128, 1)
    assert ws(*big, 0) == ws(*big, qa.SAGE_TRAIN_RECOMPUTE_DS) > 0
    assert ws(1, 2, 128, 128, 64, 0, 0x20000) == 0  # unknown bit
    assert ws(1, 2, 128, 128, 64, 0, qa.SAGE_TRAIN_KEEP_QUANT) == ws(1, 2, 128, 128, 64, 0, 0) > 0


def test_kept_quantization_needs_a_caller_workspace():
    """SAGE_TRAIN_KEEP_QUANT passes the forward's INT8 inputs to the backward through the caller's
    workspace: either call without one is an invalid argument, rejected before any device work."""
    A = 256
    sh = qa.SageAttnShape(1, 2, 2, 128, 128, 64, 0, 0.0, qa.SAGE_IN_BF16 | qa.SAGE_TRAIN_KEEP_QUANT)
    assert qa.sage_attn_train_fwd(sh, A, A, A, A, A, None, 0, None) == qa.SAGE_ERR_INVALID_ARG
    assert qa.sage_attn_train_bwd(sh, A, A, A, A, A, A, A, A, A, None, 0, None) == qa.SAGE_ERR_INVALID_ARG


def test_noalloc_rejects_problems_beyond_its_scratch():
    """The no-allocation entry point checks the problem's workspace against its fixed scratch
    before touching a device."""
    S = qa.SageAttnShape
    A = 256
    big = S(1, 32, 32, 32768, 32768, 128, 1, 0.0, 0)
    assert qa.sage_attn_workspace_bytes_ex(big) > qa.SAGE_NOALLOC_MAX_BYTES
    assert qa.sage_attn_fwd_noalloc(big, A, A, A, A, None) == qa.SAGE_ERR_NO_MEMORY
    assert qa.sage_attn_fwd_noalloc(None, A, A, A, A, None) == qa.SAGE_ERR_INVALID_ARG
    small = S(1, 2, 2, 256, 256, 64, 0, 0.0, 0)
    assert qa.sage_attn_fwd_noalloc(small, 0, A, A, A, None) == qa.SAGE_ERR_INVALID_ARG


def test_forward_bindings_check_a_caller_output_buffer():
    """A caller's out must have the shape and dtype the library writes; the check comes before
    the device checks, so host tensors show it."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros(1, 4, 64, 64, dtype=bf)
    kv = torch.zeros(1, 2, 96, 64, dtype=bf)
    for bad in (torch.zeros(1, 4, 64, 32, dtype=bf), torch.zeros(1, 4, 65, 64, dtype=bf),
                torch.zeros(1, 4, 64, 64, dtype=torch.float16), torch.zeros(1, 4, 64, 64, dtype=torch.float32)):
        with pytest.raises(ValueError):
            qa.sage_attn(q, kv, kv, out=bad)
    with pytest.raises(ValueError):  # fp32 requested, bf16 given
        qa.sage_attn(q, kv, kv, out_fp32=True, out=torch.zeros(1, 4, 64, 64, dtype=bf))
    qv = torch.zeros(100, 4, 64, dtype=bf)
    kvv = torch.zeros(120, 2, 64, dtype=bf)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32)
    cuk = torch.tensor([0, 50, 120], dtype=torch.int32)
    with pytest.raises(ValueError):
        qa.sage_attn_varlen(qv, kvv, kvv, cu, cuk, 60, 70, out=torch.zeros(99, 4, 64, dtype=bf))
    with pytest.raises(ValueError):  # right shapes, host tensors
        qa.sage_attn_varlen(qv, kvv, kvv, cu, cuk, 60, 70)
    with pytest.raises(ValueError):
        qa.sage_attn(q, kv, kv)
