// Helpers shared by the two budgeted streaming executors (rectangular blocks
// and cyclic quorums).  Internal to libattn.so.
#pragma once

#include <stdint.h>

#include "common.h"

namespace attn {
namespace streamx {

constexpr int64_t kAlign = 256;
constexpr int64_t kAllocSlack = 2ll << 20;  // device allocation granularity kept free inside the budget
inline int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t elem_size(attn_dtype dt) { return dt == ATTN_F32 ? 4 : 2; }

// Budget in bytes usable by block buffers (the budget less the allocation slack).
inline int64_t usable_budget(size_t budget) {
  const int64_t raw = budget > (size_t)INT64_MAX ? INT64_MAX : (int64_t)budget;
  return raw - kAllocSlack;
}

// Argument checks common to every streaming call (dtype, head dim, sizes).
attn_status check_stream_sizes(attn_dtype dt, int B, int Hq, int Hkv, int64_t S, int64_t T, int D);

// Every non-empty host buffer of a streaming call must be pinned host memory.
attn_status check_pinned(attn_dtype dt, const void* q, const void* k, const void* v, const float* o,
                         const float* lse, int B, int Hq, int Hkv, int64_t S, int64_t T, int D);

// Prefill arguments for n_q query rows held in device buffers q/o ([n_q, Hq, D])
// and lse ([Hq, n_q]) against n_k keys in k/v ([n_k, Hkv, D]); the rows sit at
// absolute positions q_abs0.., the keys at k_abs0...
PrefillArgs block_args(const void* q, const void* k, const void* v, float* o, float* lse, int Hq, int Hkv, int D,
                       int64_t n_q, int64_t n_k, int64_t q_abs0, int64_t k_abs0, int causal, int accumulate,
                       float scale_log2);

}  // namespace streamx
}  // namespace attn
