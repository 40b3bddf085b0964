"""Helpers of the GPU parity tests: move seeded inputs to the device, call the C ABI
through the binding, and bring results back in the oracle's natural layouts.

The only layout knowledge here is what include/sage_attn.h documents for the quantize
views (padding, the per-tile transposed V^ with its key order); nothing is imported from
the HIP sources or the oracle."""
import numpy as np
import torch

import quantized_attention_amd as qa

BQ, BK_ = qa.SAGE_BQ, qa.SAGE_BK


def to_dev(bits: np.ndarray, fp16: bool) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if fp16 else torch.bfloat16).cuda()


def doc_kperm(h: int, b: int) -> int:
    """Key order of the transposed V^ tile, as the header documents it."""
    return 32 * (b // 16) + 8 * ((b % 16) // 4) + 4 * h + b % 4


INV_PERM = np.array([doc_kperm(p // 32, p % 32) for p in range(64)])


def doc_vperm_mx(h: int, j: int) -> int:
    """Key order of the transposed MX V^ tile, as the header documents it."""
    return 32 * h + 8 * ((j % 16) // 4) + 4 * (j // 16) + j % 4


INV_PERM_MX = np.array([doc_vperm_mx(p // 32, p % 32) for p in range(64)])


def fwd(q, k, v, fp16, causal, sm_scale, smooth_v=False, out_fp32=True, acc_valu=False, mxfp4=False,
        qk_fp8=False, mx_p_two_level=False):
    """q, k, v: uint16 bits [B, H, T, d] on the host; returns the output as a device tensor."""
    B, H, N, d = q.shape
    M = k.shape[2]
    tq, tk, tv = to_dev(q, fp16), to_dev(k, fp16), to_dev(v, fp16)
    out = qa.sage_attn(tq, tk, tv, causal=causal, sm_scale=sm_scale, smooth_v=smooth_v, out_fp32=out_fp32,
                       acc_valu=acc_valu, mxfp4=mxfp4, qk_fp8=qk_fp8, mx_p_two_level=mx_p_two_level)
    torch.cuda.synchronize()
    return out


def quantize(q, k, v, fp16, causal, smooth_v=False, qk_fp8=False):
    """Preprocessing through sage_attn_quantize_ex, returned per head in natural layouts
    (K/V-side tensors for the key/value heads, Q-side ones for the query heads)."""
    B, H, N, d = q.shape
    Hkv, M = k.shape[1], k.shape[2]
    BH, BK = B * H, B * Hkv
    nqb, nkt = -(-N // BQ), -(-M // BK_)
    Np, Mp = nqb * BQ, nkt * BK_
    dev = torch.device("cuda")
    bufs = dict(
        q_hat=torch.empty((BH, Np, d), dtype=torch.int8, device=dev),
        k_hat=torch.empty((BK, Mp, d), dtype=torch.int8, device=dev),
        v_hat=torch.empty((BK, nkt, d, 64), dtype=torch.uint8, device=dev),
        dq=torch.empty((BH, Np), dtype=torch.float32, device=dev),
        dk=torch.empty((BK, nkt, 4), dtype=torch.float32, device=dev),
        dv=torch.empty((BK, d), dtype=torch.float32, device=dev),
        k_mean=torch.empty((BK, d), dtype=torch.float32, device=dev),
        v_mean=torch.empty((BK, d), dtype=torch.float32, device=dev),
        q_mean=torch.empty((BH, nqb, d), dtype=torch.float32, device=dev),
        delta_s=torch.full((BH, nqb, Mp), float("nan"), dtype=torch.float32, device=dev),
    )
    views = qa.QuantViews(**{n: t.data_ptr() for n, t in bufs.items()})
    tq, tk, tv = to_dev(q, fp16), to_dev(k, fp16), to_dev(v, fp16)
    var = (qa.SAGE_IN_FP16 if fp16 else qa.SAGE_IN_BF16) | (qa.SAGE_SMOOTH_V if smooth_v else 0)
    var |= qa.SAGE_QK_FP8 if qk_fp8 else 0
    shape = qa.SageAttnShape(B, H, Hkv, N, M, d, int(causal), 0.0, var)
    rc = qa.sage_attn_quantize_ex(shape, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), views,
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == qa.SAGE_OK, qa.sage_attn_status_string(rc)
    torch.cuda.synchronize()
    h = {n: t.cpu().numpy() for n, t in bufs.items()}
    # V^: [BK][nkt][d][64] (permuted keys) -> [BK][Mp][d]
    vt = h["v_hat"]
    vnat = np.zeros((BK, Mp, d), np.uint8)
    for u in range(nkt):
        vnat[:, u * 64 + INV_PERM, :] = vt[:, u].transpose(0, 2, 1)
    h["v_nat"] = vnat
    return h


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] E2M1 codes, the lower-indexed element in the low nibble."""
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def quantize_mx(q, k, v, fp16, causal, smooth_v=False):
    """MX preprocessing through sage_attn_quantize; returns the raw views and, per head, the
    codes and unbiased exponents in the oracle's natural layouts."""
    B, H, N, d = q.shape
    M = k.shape[2]
    BH = B * H
    nqb, nkt = -(-N // BQ), -(-M // BK_)
    Np, Mp = nqb * BQ, nkt * BK_
    dev = torch.device("cuda")
    fill = dict(dtype=torch.uint8, device=dev)
    bufs = dict(
        q_hat=torch.full((BH, Np, d // 2), 0xAB, **fill),
        k_hat=torch.full((BH, Mp, d // 2), 0xAB, **fill),
        v_hat=torch.full((BH, nkt, d, 32), 0xAB, **fill),
        k_mean=torch.empty((BH, d), dtype=torch.float32, device=dev),
        v_mean=torch.empty((BH, d), dtype=torch.float32, device=dev),
        q_mean=torch.empty((BH, nqb, d), dtype=torch.float32, device=dev),
        delta_s=torch.full((BH, nqb, Mp), float("nan"), dtype=torch.float32, device=dev),
        mx_scales_q=torch.full((BH, Np, d // 32), 0xAB, **fill),
        mx_scales_k=torch.full((BH, nkt, 64, 4), 0xAB, **fill),
        mx_scales_v=torch.full((BH, nkt, 64, 4), 0xAB, **fill),
    )
    views = qa.QuantViews(**{n: t.data_ptr() for n, t in bufs.items()})
    tq, tk, tv = to_dev(q, fp16), to_dev(k, fp16), to_dev(v, fp16)
    var = (qa.SAGE_IN_FP16 if fp16 else qa.SAGE_IN_BF16) | (qa.SAGE_SMOOTH_V if smooth_v else 0) | qa.SAGE_PATH_MXFP4
    rc = qa.sage_attn_quantize(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), B, H, N, M, d, causal, var,
                               views, torch.cuda.current_stream().cuda_stream)
    assert rc == qa.SAGE_OK, qa.sage_attn_status_string(rc)
    torch.cuda.synchronize()
    h = {n: t.cpu().numpy() for n, t in bufs.items()}
    h["qcode"] = unpack_nibbles(h["q_hat"])                      # [BH][Np][d]
    h["kcode"] = unpack_nibbles(h["k_hat"])                      # [BH][Mp][d]
    h["qexp"] = h["mx_scales_q"].astype(np.int32) - 127          # [BH][Np][d/32]
    # K scales: byte 4l + 2T + c -> key 64u + 32T + l%32, channel block 2c + l/32
    ks = h["mx_scales_k"]
    kexp = np.zeros((BH, Mp, d // 32), np.int32)
    for u in range(nkt):
        for l in range(64):
            for T in range(2):
                for c in range(d // 64):
                    kexp[:, 64 * u + 32 * T + l % 32, 2 * c + l // 32] = ks[:, u, l, 2 * T + c].astype(np.int32) - 127
    h["kexp"] = kexp
    # V^: [BH][nkt][d][32 bytes] -> codes [BH][Mp][d]; V scales byte 4l + g -> channel 32g + l%32,
    # token block 2u + l/32
    vn = unpack_nibbles(h["v_hat"])                              # [BH][nkt][d][64] nibbles
    vcode = np.zeros((BH, Mp, d), np.uint8)
    for u in range(nkt):
        vcode[:, u * 64 + INV_PERM_MX, :] = vn[:, u].transpose(0, 2, 1)
    h["vcode"] = vcode
    vs = h["mx_scales_v"]
    vexp = np.zeros((BH, 2 * nkt, d), np.int32)
    for u in range(nkt):
        for l in range(64):
            for g in range(d // 32):
                vexp[:, 2 * u + l // 32, 32 * g + l % 32] = vs[:, u, l, g].astype(np.int32) - 127
    h["vexp"] = vexp
    return h
