"""ctypes wrapper around the C oracle (``sage_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The oracle is the slow CPU reference that the GPU path is
checked against; only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import it.  The product package never does.

Arrays cross the boundary as numpy arrays; 16-bit inputs are passed as their raw bit
patterns (``uint16``) with a flag that says whether they are fp16 or bf16.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sage_oracle.c")
SOURCES = [SRC, os.path.join(HERE, "sagebwd_oracle.c"), os.path.join(HERE, "sage_oracle.h")]
LIB = os.path.join(HERE, "liboracle.so")

BQ, BK = 128, 64
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]

SMOOTH_V = 0x0001
NO_SMOOTH_K = 0x0002
NO_SMOOTH_Q = 0x0004
QK_IDENTITY = 0x0010
QK_PER_BLOCK = 0x0020
QK_PER_TOKEN = 0x0040
QK_PER_TENSOR = 0x0080
PV_IDENTITY = 0x0100
PV_E5M2 = 0x0200
PV_INT8 = 0x0400
MXFP4 = 0x1000
MX_P_TWO_LEVEL = 0x4000  # MX knob: P~ row-scaled by rowmax / 6 before the E2M1 quantizer
QK_E4M3 = 0x2000  # Q^, K^ in E4M3 (scale amax / 448, same groups); khat, qhat then hold E4M3 codes


def _stale() -> bool:
    return not os.path.exists(LIB) or any(os.path.getmtime(LIB) < os.path.getmtime(f) for f in SOURCES)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, no fast-math, no FP contraction)."""
    if force or _stale():
        tmp = LIB + ".tmp"
        cmd = ["gcc", *_CFLAGS, *[f for f in SOURCES if f.endswith(".c")], "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


_lib = None


def _configure(L):
    """Declare the argument and result types of the library's entry points."""
    P = ctypes.c_void_p
    i, u, dbl = ctypes.c_int, ctypes.c_uint, ctypes.c_double
    L.orc_preprocess_head.argtypes = [P, P, P, i, i, i, i, u] + [P] * 10
    L.orc_preprocess_head.restype = i
    L.orc_preprocess_mx_head.argtypes = [P, P, P, i, i, i, i, u, P, P, P, P, P, P]
    L.orc_preprocess_mx_head.restype = i
    L.orc_forward_head.argtypes = [P, P, P, i, i, i, i, i, dbl, u, P, i, P]
    L.orc_forward_head.restype = i
    L.orc_forward_head_ties.argtypes = [P, P, P, i, i, i, i, i, dbl, u, P, i, P, dbl, dbl, P, P]
    L.orc_forward_head_ties.restype = i
    L.orc_exact_head.argtypes = [P, P, P, i, i, i, i, i, dbl, P, i, P]
    L.orc_exact_head.restype = i
    L.orc_exact_f64.argtypes = [P, P, P, i, i, i, i, dbl, P]
    L.orc_exact_f64.restype = i
    L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_decode.restype = dbl
    L.orc_e4m3_encode.argtypes = [dbl]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_e4m3_encode_f32_array.argtypes = [P, P, ctypes.c_size_t]
    L.orc_e4m3_encode_f32_array.restype = None
    L.orc_e5m2_decode.argtypes = [ctypes.c_uint8]
    L.orc_e5m2_decode.restype = dbl
    L.orc_e5m2_encode.argtypes = [dbl]
    L.orc_e5m2_encode.restype = ctypes.c_uint8
    L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
    L.orc_e2m1_decode.restype = dbl
    L.orc_e2m1_encode.argtypes = [dbl]
    L.orc_e2m1_encode.restype = ctypes.c_uint8
    L.orc_e8m0_exponent.argtypes = [dbl]
    L.orc_e8m0_exponent.restype = i
    L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_bf16_to_f32.restype = ctypes.c_float
    L.orc_fp16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_fp16_to_f32.restype = ctypes.c_float
    L.orc_k_group.argtypes = [i]
    L.orc_k_group.restype = i
    L.orc_sagebwd_forward.argtypes = [P, P, P, i, i, i, i, i, dbl, u, P, P]
    L.orc_sagebwd_forward.restype = i
    L.orc_sagebwd_backward.argtypes = [P, P, P, P, i, i, i, i, i, dbl, u, P, P, P, P, P]
    L.orc_sagebwd_backward.restype = i
    L.orc_sagebwd_quantize.argtypes = [P, P, P, P, i, i, i, i, u] + [P] * 9
    L.orc_sagebwd_quantize.restype = i
    L.orc_num_threads.argtypes = []
    L.orc_num_threads.restype = i
    return L


def lib():
    global _lib
    if _lib is None:
        if _stale():
            build(force=True)
        _lib = _configure(ctypes.CDLL(LIB))
    return _lib


@contextlib.contextmanager
def planted_mistake(*edits):
    """Temporarily replace the oracle by a copy compiled with deliberate mistakes, for tests
    that show a pin catches them.  edits: (file name, text, replacement) triples; each text
    must occur exactly once in that source file.  The mutant is built in a temporary
    directory with the same compiler flags; the real library is restored on exit."""
    global _lib
    with tempfile.TemporaryDirectory() as tmp:
        srcs = []
        for f in SOURCES:
            with open(f) as fh:
                text = fh.read()
            for name, old, new in edits:
                if name == os.path.basename(f):
                    if text.count(old) != 1:
                        raise ValueError(f"planted_mistake: {old!r} occurs {text.count(old)} times in {name}")
                    text = text.replace(old, new)
            dst = os.path.join(tmp, os.path.basename(f))
            with open(dst, "w") as fh:
                fh.write(text)
            srcs.append(dst)
        so = os.path.join(tmp, "liboracle_mutant.so")
        subprocess.run(["gcc", *_CFLAGS, *[f for f in srcs if f.endswith(".c")], "-o", so, "-lm"], check=True)
        saved = lib()
        _lib = _configure(ctypes.CDLL(so))
        try:
            yield
        finally:
            _lib = saved


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _u16(x):
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, x.dtype
    return x


def preprocess_head(q, k, v, fp16: bool, flags: int = 0) -> dict:
    """Quantized tensors and scales of one head, in natural layouts (see sage_oracle.h)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    N, d = q.shape
    M = k.shape[0]
    nqb, nkt = -(-N // BQ), -(-M // BK)
    o = dict(kmean=np.zeros(d, np.float32), vmean=np.zeros(d, np.float32),
             khat=np.zeros((M, d), np.int8), dk=np.zeros((nkt, 4), np.float32),
             vhat=np.zeros((M, d), np.uint8), dv=np.zeros(d, np.float32),
             qhat=np.zeros((N, d), np.int8), dq=np.zeros(N, np.float32),
             qmean=np.zeros((nqb, d), np.float32), ds=np.zeros((nqb, M), np.float64))
    rc = lib().orc_preprocess_head(_ptr(q), _ptr(k), _ptr(v), int(fp16), N, M, d, flags,
                                   *[_ptr(o[n]) for n in ("kmean", "vmean", "khat", "dk", "vhat",
                                                          "dv", "qhat", "dq", "qmean", "ds")])
    if rc != 0:
        raise ValueError("orc_preprocess_head rejected its arguments")
    if flags & QK_E4M3:
        o["qhat"], o["khat"] = o["qhat"].view(np.uint8), o["khat"].view(np.uint8)
    return o


def preprocess_mx_head(q, k, v, fp16: bool, flags: int = 0) -> dict:
    """MX-variant codes and exponents of one head (natural layouts, see sage_oracle.h)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    N, d = q.shape
    M = k.shape[0]
    o = dict(qcode=np.zeros((N, d), np.uint8), qexp=np.zeros((N, d // 32), np.int32),
             kcode=np.zeros((M, d), np.uint8), kexp=np.zeros((M, d // 32), np.int32),
             vcode=np.zeros((M, d), np.uint8), vexp=np.zeros((-(-M // 32), d), np.int32))
    rc = lib().orc_preprocess_mx_head(_ptr(q), _ptr(k), _ptr(v), int(fp16), N, M, d, flags & ~MXFP4,
                                      *[_ptr(o[n]) for n in ("qcode", "qexp", "kcode", "kexp", "vcode", "vexp")])
    if rc != 0:
        raise ValueError("orc_preprocess_mx_head rejected its arguments")
    return o


def forward_head(q, k, v, fp16: bool, causal: int, sm_scale: float, flags: int = 0, rows=None):
    """The quantized forward of one head in FP64: [len(rows) or N, d].  causal: 0 none, 1 key t
    visible to row r iff t <= r, 2 iff t <= r + M - N (needs N <= M)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    N, d = q.shape
    M = k.shape[0]
    if rows is None:
        nrows, rp = N, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        nrows, rp = len(rows), rows
    out = np.zeros((nrows, d), np.float64)
    rc = lib().orc_forward_head(_ptr(q), _ptr(k), _ptr(v), int(fp16), N, M, d, int(causal),
                                float(sm_scale), flags, _ptr(rp), nrows, _ptr(out))
    if rc != 0:
        raise ValueError("orc_forward_head rejected its arguments")
    return out


def forward_head_ties(q, k, v, fp16: bool, causal: int, sm_scale: float, flags: int = 0, rows=None,
                      tie_eps: float = 2.0 ** -16, qk_step_err: float = 0.0):
    """forward_head, and per row the count of its P rounding decisions whose input lies within
    relative distance tie_eps of a rounding boundary (where an FP32 kernel may round the other
    way) and a bound on the output change if all of them do: (out, ties, bound).  qk_step_err
    (with QK_E4M3): widen each decision's margin by the score error of a matrix core that sums
    every 64-channel step of Q^ K^ to within qk_step_err of the step's largest code product."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    N, d = q.shape
    M = k.shape[0]
    if rows is None:
        nrows, rp = N, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        nrows, rp = len(rows), rows
    out = np.zeros((nrows, d), np.float64)
    ties = np.zeros(nrows, np.int32)
    bound = np.zeros(nrows, np.float64)
    rc = lib().orc_forward_head_ties(_ptr(q), _ptr(k), _ptr(v), int(fp16), N, M, d, int(causal),
                                     float(sm_scale), flags, _ptr(rp), nrows, _ptr(out), float(tie_eps),
                                     float(qk_step_err), _ptr(ties), _ptr(bound))
    if rc != 0:
        raise ValueError("orc_forward_head_ties rejected its arguments")
    return out, ties, bound


def exact_head(q, k, v, fp16: bool, causal: int, sm_scale: float, rows=None):
    """softmax(Q K^T * sm_scale) V in FP64 on the widened inputs."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    N, d = q.shape
    M = k.shape[0]
    if rows is None:
        nrows, rp = N, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        nrows, rp = len(rows), rows
    out = np.zeros((nrows, d), np.float64)
    rc = lib().orc_exact_head(_ptr(q), _ptr(k), _ptr(v), int(fp16), N, M, d, int(causal),
                              float(sm_scale), _ptr(rp), nrows, _ptr(out))
    if rc != 0:
        raise ValueError("orc_exact_head rejected its arguments")
    return out


def exact_f64(q, k, v, causal: int, sm_scale: float):
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    N, d = q.shape
    M = k.shape[0]
    out = np.zeros((N, v.shape[1]), np.float64)
    assert v.shape[1] == d
    rc = lib().orc_exact_f64(_ptr(q), _ptr(k), _ptr(v), N, M, d, int(causal), float(sm_scale), _ptr(out))
    if rc != 0:
        raise ValueError("orc_exact_f64 rejected its arguments")
    return out


SB_IDENTITY = 0x1     # SageBwd: no quantizer anywhere
SB_NO_SMOOTH_K = 0x2  # SageBwd ablation: skip K - mean(K)
SB_DP_INT8 = 0x4      # SageBwd ablation: dP = dO V^T from per-block INT8 dO and V


def sagebwd_forward(q, k, v, fp16: bool, causal: int, sm_scale: float, flags: int = 0):
    """SageBwd forward of one head: (out [N][d], lse [N]) in FP64."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    N, d = q.shape
    M = k.shape[0]
    out, lse = np.zeros((N, d)), np.zeros(N)
    rc = lib().orc_sagebwd_forward(_ptr(q), _ptr(k), _ptr(v), int(fp16), N, M, d, int(causal), float(sm_scale),
                                   flags, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("orc_sagebwd_forward rejected its arguments")
    return out, lse


def sagebwd_backward(q, k, v, dout, fp16: bool, causal: int, sm_scale: float, flags: int = 0) -> dict:
    """SageBwd forward and backward of one head: out, lse, dq, dk, dv in FP64."""
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    N, d = q.shape
    M = k.shape[0]
    o = dict(out=np.zeros((N, d)), lse=np.zeros(N), dq=np.zeros((N, d)), dk=np.zeros((M, d)), dv=np.zeros((M, d)))
    rc = lib().orc_sagebwd_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), int(fp16), N, M, d, int(causal),
                                    float(sm_scale), flags, *[_ptr(o[n]) for n in ("out", "lse", "dq", "dk", "dv")])
    if rc != 0:
        raise ValueError("orc_sagebwd_backward rejected its arguments")
    return o


def sagebwd_quantize(q, k, v, dout, fp16: bool, flags: int = 0) -> dict:
    """SageBwd's INT8 codes and block scales of one head (dout may be None)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    dout = _u16(dout) if dout is not None else None
    N, d = q.shape
    M = k.shape[0]
    nqb, nkt = -(-N // BQ), -(-M // BK)
    o = dict(qcode=np.zeros((N, d), np.int8), sq=np.zeros(nqb, np.float32), kcode=np.zeros((M, d), np.int8),
             sk=np.zeros(nkt, np.float32), vcode=np.zeros((M, d), np.int8), sv=np.zeros(nkt, np.float32),
             docode=np.zeros((N, d), np.int8), sdo=np.zeros(nqb, np.float32), kmean=np.zeros(d, np.float32))
    rc = lib().orc_sagebwd_quantize(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), int(fp16), N, M, d, flags,
                                    *[_ptr(o[n]) for n in ("qcode", "sq", "kcode", "sk", "vcode", "sv", "docode",
                                                           "sdo", "kmean")])
    if rc != 0:
        raise ValueError("orc_sagebwd_quantize rejected its arguments")
    if dout is None:
        del o["docode"], o["sdo"]
    return o


def e4m3_encode_f32(x) -> np.ndarray:
    """E4M3 codes (round to nearest even, saturated) of an FP32 array, elementwise."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_encode_f32_array(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_decode_table() -> np.ndarray:
    return np.array([lib().orc_e4m3_decode(c) for c in range(256)])


def num_threads() -> int:
    return lib().orc_num_threads()
