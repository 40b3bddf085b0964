// sagebwd.hpp -- host entry points of SageBwd, the trainable INT8 attention (sagebwd.hip).
#pragma once

#include "sage_common.hpp"

namespace sage {

// Workspace bytes (offsets of its slices into `offsets` when given), the preprocessing of Q,
// K, V (K smoothed when smooth_k), the forward (out, lse), the backward's preprocessing (dO^,
// D, L) and the backward (dq, dk, dv in FP32).
size_t sb_layout(const Problem& p, bool bwd, size_t* offsets);
// Whether the backward keeps every (query block, key block) pair's dS^ (the dK/dV kernel writes
// it, the dQ kernel contracts it) or the dQ kernel recomputes dS: the latter with
// SAGE_TRAIN_RECOMPUTE_DS, or when the pair buffer would exceed kSbPairLimit bytes.
constexpr size_t kSbPairLimit = (size_t)16 << 30;
// The pair buffer holds one record per (pair, wave of the pair's query block): the wave's dS^
// codes in the dQ product's B-operand order (two halves of 64 lanes x 16 bytes), the FP32 sums of
// dS over the pair's keys for the wave's 32 queries, the pair's dQ multiplier
// (max|dS| / 127) s_K sm_scale, and padding to 2192 bytes (a multiple of 16, for the 16-byte
// DMAs).  In the dQ kernel's LDS ring a record takes kSbRecLds bytes: its tail's DMA writes
// 64 lanes x 4 bytes from offset 2048.
constexpr int kSbRec = 2192;
constexpr int kSbRecLds = 2048 + 64 * 4;
bool sb_store_ds(const Problem& p);
// The chunk reduction to K's mean alone, after launch_stats with v null (SageBwd takes no V
// statistics); defined with the other preprocessing launchers.
hipError_t launch_kv_finalize_k_only(const Problem& p, const Workspace& w, hipStream_t s);
hipError_t sb_prep_fwd(const Problem& p, const void* q, const void* k, const void* v, char* ws, bool bwd,
                       bool smooth_k, hipStream_t st);
hipError_t sb_forward(const Problem& p, char* ws, bool bwd, void* out, float* lse, hipStream_t st);
hipError_t sb_prep_bwd(const Problem& p, const void* out, const void* dout, const float* lse, char* ws,
                       hipStream_t st);
hipError_t sb_backward(const Problem& p, char* ws, bool smooth_k, const void* v, const void* dout, float* dq,
                       float* dk, float* dv, hipStream_t st);

}  // namespace sage
