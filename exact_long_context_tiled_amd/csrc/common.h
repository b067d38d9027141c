// Internal declarations of libattn.so (not installed; the public ABI is include/attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <string>

#include "attn.h"

namespace attn {

// ---------------------------------------------------------------- vector types
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- errors
attn_status set_error(attn_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
attn_status check_launch(const char* what);

// Compute units of the current device (cached per device).
int device_cu_count();

// Raise `kernel`'s dynamic LDS limit on the current device to at least
// `bytes`; `raised` holds the limit already set per device (thread-safe).
constexpr int kMaxDevices = 64;
attn_status raise_lds_limit(const void* kernel, size_t bytes, std::atomic<size_t>* raised);

// ---------------------------------------------------------------- prefill
// One launch computes a block of n_q queries against a block of n_k keys for
// every (sequence, KV head).  Local query i sits at absolute position
// q_abs0 + i, local key j at k_abs0 + j; under `causal` key j is visible to
// query i iff k_abs0 + j <= q_abs0 + i.  With `accumulate`, the block's
// (O, lse) is merged by log-sum-exp into the (O, lse) already in memory.
// Element strides: q/o [b, s, h, d] with head stride D; k/v [b, t, hk, d];
// lse [b, h, s] with position stride 1.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;  // may be null unless accumulate
  int64_t q_sb, q_ss;
  int64_t k_sb, k_ss;
  int64_t o_sb, o_ss;
  int64_t l_sb, l_sh;
  int64_t n_q, n_k;
  int64_t q_abs0, k_abs0;
  int B, Hq, Hkv, G;
  int causal;
  int accumulate;
  float scale_log2;  // scale * log2(e)
  // e4m3 operands only: per-head scales, q [Hq], k and v [Hkv] (fp32, > 0)
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
};

// Launchers: validate nothing (the ABI layer did), launch on `stream`.
attn_status launch_prefill_bf16(const PrefillArgs& a, int D, hipStream_t stream);
attn_status launch_prefill_f32(const PrefillArgs& a, int D, hipStream_t stream);
attn_status launch_prefill_fp8(const PrefillArgs& a, int D, hipStream_t stream);

// ---------------------------------------------------------------- decode
// The KV of the whole batch is one run of 16-token groups, segment by
// segment ((sequence, KV head) in order, ceil(len / 16) groups each); work
// unit i of N takes groups [floor(i*W/N), floor((i+1)*W/N)).  A unit yields
// one partial record per segment it touches (record index i + segment); a
// segment covered by one unit alone is written straight to the output.
struct DecodeArgs {
  const void* q;  // [B, Hq, D] bf16
  const void* k;  // cache
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* page_table;  // null: contiguous
  int max_pages;
  int num_pages;   // physical pages of a paged cache: entries outside [0, num_pages) are not
                   // dereferenced (page 0 is read instead and the segment's rows come out NaN)
  int page_size;
  int page_shift;  // log2(page_size) when paged
  const int32_t* kv_lens;
  int max_kv_len;  // lengths are clamped to [0, max_kv_len]
  int B, Hq, Hkv;
  int G;        // Hq / Hkv
  int n_q;      // query tokens per sequence (rows of the segment: n_q * G)
  int n_units;  // N
  int piece_groups;  // groups each non-empty segment is charged in the split (matrix-core kernel; else 0)
  float scale_log2;
  float* part;       // records [N + B*Hkv - 1][R*D + pad16(R)], R = n_q*G: O rows, then lse (log2)
  int32_t* seg_info; // [B*Hkv][2]: vector-ALU split: first record, record count (written by the
                     // segment's first unit); matrix-core split: one 64-bit arrival counter
                     // per segment (tag << 16 | count) for its fused merge
  uint64_t tag;      // per-call tag of the arrival counters (48 bits, nonzero)
  float* o;          // [B, n_q, Hq, D]
  float* lse;        // [B, Hq, n_q] or null
};

constexpr int kDecodeGroup = 16;          // tokens per group (>= tokens per wave load step)
constexpr int kDecodeMaxAutoUnits = 2048; // upper bound of the automatic unit count
constexpr int kDecodeMaxUnits = 65535;
constexpr int kDecodeMaxPieceGroups = 4096;  // bound of DecodeArgs::piece_groups

// Floats of one partial record of `rows` query rows: O rows, then the rows' lse
// padded to a multiple of 16.
__host__ __device__ inline int decode_record_floats(int rows, int D) { return rows * D + (rows + 15) / 16 * 16; }
size_t decode_workspace_bytes(int B, int Hkv, int rows, int D, int n_units_bound);
// K + V cache bytes of one token of one KV head, scales included.
inline int64_t decode_token_bytes(attn_dtype kv_dt, int D) {
  switch (kv_dt) {
    case ATTN_BF16: return 4 * (int64_t)D;
    case ATTN_INT8: return 2 * (int64_t)D + 8;                      // + per-token fp32 scales
    case ATTN_INT4: return (int64_t)D + 2 * (int64_t)(D / 32) * 4;  // nibbles + group scales
    default: return 2 * (int64_t)D;                                 // e4m3 (per-head scales)
  }
}
// Process-wide decode tuning (attn_decode_set_tuning); results stay exact.
struct DecodeTuning {
  int path;             // 0: matrix cores where supported, 1: vector ALUs
  int units;            // automatic unit count (0: one per compute unit)
  int64_t piece_bytes;  // charge per non-empty segment in the matrix-core split (< 0: default)
};
constexpr int64_t kDecodePieceBytes = 192 << 10;
DecodeTuning decode_tuning();
// n_units == 0 picks one work-group per compute unit (at most
// kDecodeMaxAutoUnits).  The split runs on the matrix cores for bf16 / e4m3 /
// int8 caches and D = 128 int4 caches (unless the tuning selects the vector
// ALUs), on the vector ALUs otherwise.  The matrix-core split merges its own
// segments in the same launch; the vector-ALU split is followed by the merge
// kernel.
attn_status launch_decode(attn_dtype kv_dt, const DecodeArgs& a, int D, int G, hipStream_t stream);
bool decode_mfma_supported(attn_dtype kv_dt, int D);
attn_status launch_decode_split_mfma(attn_dtype kv_dt, const DecodeArgs& a, int D, hipStream_t stream);

// ---------------------------------------------------------------- merge
attn_status launch_merge(int n, const float* o_parts, const float* lse_parts, int64_t R, int D, float* o,
                         float* lse, hipStream_t stream);

}  // namespace attn
