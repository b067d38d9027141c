// Device helpers shared by the split-KV decode kernels (vector-ALU and
// matrix-core).  Internal to libattn.so.
#pragma once

#include "common.h"

namespace attn {
namespace dec {

// {a, b} = {x of this lane, x of lane ^ OFF} in a lane-fixed order (the
// combine below is symmetric in the two): one permlane swap for OFF = 32 or
// 16, a row rotation for OFF = 8, an LDS-free bpermute otherwise.
template <int OFF>
__device__ __forceinline__ void lane_pair(float x, float& a, float& b) {
  if constexpr (OFF == 32 || OFF == 16) {
    const uint32_t u = __float_as_uint(x);
    const auto r = OFF == 32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                             : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else if constexpr (OFF == 8) {
    a = x;
    b = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  } else {
    a = x;
    b = __shfl_xor(x, OFF);
  }
}

__device__ __forceinline__ int clamp_len(int t, int max_len) { return min(max(t, 0), max_len); }

// Groups one segment of a sequence of length t occupies in the split: its
// 16-token groups plus `charge` more when it is not empty.
__device__ __forceinline__ int64_t seg_slots(int t, int charge) {
  const int g = (t + kDecodeGroup - 1) / kDecodeGroup;
  return g > 0 ? (int64_t)g + charge : 0;
}

// pre[b] = slots of all segments of sequences < b (per KV head), pre[B] =
// total; computed by the whole work-group into LDS, with the clamped lengths
// in len_out[b] when it is not null.
template <int THREADS>
__device__ void group_prefix(const int32_t* __restrict__ lens, int B, int max_len, int charge, int64_t* pre,
                             int64_t* wsum, int* len_out = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (B + THREADS - 1) / THREADS;
  const int b0 = tid * per;
  int64_t s = 0;
  for (int k = 0; k < per; ++k)
    if (b0 + k < B) s += seg_slots(clamp_len(lens[b0 + k], max_len), charge);
  int64_t x = s;  // inclusive scan over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int64_t base = 0;
  for (int ww = 0; ww < w; ++ww) base += wsum[ww];
  int64_t run = base + x - s;
  for (int k = 0; k < per; ++k) {
    if (b0 + k < B) {
      const int t = clamp_len(lens[b0 + k], max_len);
      pre[b0 + k] = run;
      if (len_out) len_out[b0 + k] = t;
      run += seg_slots(t, charge);
    }
  }
  if (tid == THREADS - 1) pre[B] = base + x;
  __syncthreads();
}

// Loads and stores of partial records.  Records that another work-group
// merges in the same launch (the matrix-core split's fused merge) are written
// and read at device scope: the stores go through to the memory every XCD
// sees, the loads bypass a possibly stale copy in this XCD's L2.
template <bool COHERENT>
__device__ __forceinline__ float rec_load(const float* p) {
  if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COHERENT>
__device__ __forceinline__ void rec_store(float* p, float v) {
  if constexpr (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// Log-sum-exp merge of one output row over the n records rec0, rec0 + REC, ...
// (each: RT normalised rows of D floats, then RT log2-domain lse values); the
// row is r_rec of every record.  One wave, D / 64 columns per lane; writes
// orow and, when lse_out is not null, the natural-log lse.  A record of a row
// that saw no key there has lse = -inf and weight 0; a NaN record (a
// page-table entry outside the cache) makes the row NaN.
template <int D, bool COHERENT>
__device__ void merge_row(const float* rec0, int REC, int RT, int r_rec, int n, int lane, float* orow,
                          float* lse_out) {
  constexpr int CPL = D / 64;  // columns per lane
  float mx = -INFINITY, den = 0.f, acc[CPL];
  bool nan_seen = false;
#pragma unroll
  for (int k = 0; k < CPL; ++k) acc[k] = 0.f;
  // eight records at a time, all their loads issued before the first use;
  // an online log-sum-exp update folds each batch in
  for (int c0 = 0; c0 < n; c0 += 8) {
    float lv[8], x[8][CPL];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float* rec = rec0 + (int64_t)min(c0 + r, n - 1) * REC;  // past the end: a valid record, weighted 0
      lv[r] = rec_load<COHERENT>(rec + (int64_t)RT * D + r_rec);
#pragma unroll
      for (int k = 0; k < CPL; ++k) x[r][k] = rec_load<COHERENT>(rec + (int64_t)r_rec * D + lane + 64 * k);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (c0 + r >= n) lv[r] = -INFINITY;
      nan_seen |= lv[r] != lv[r];
      bm = fmaxf(bm, lv[r]);
    }
    const float M = fmaxf(mx, bm);
    if (M == -INFINITY) continue;  // nothing seen yet
    const float f = __builtin_amdgcn_exp2f(mx - M);
    den *= f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) acc[k] *= f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float w = __builtin_amdgcn_exp2f(lv[r] - M);
      den += w;
#pragma unroll
      for (int k = 0; k < CPL; ++k) acc[k] = fmaf(w, x[r][k], acc[k]);
    }
    mx = M;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int k = 0; k < CPL; ++k) orow[lane + 64 * k] = nan_seen ? qnan : acc[k] * inv;
  if (lane == 0 && lse_out) *lse_out = nan_seen ? qnan : den > 0.f ? (mx + __log2f(den)) * kLn2 : -INFINITY;
}

}  // namespace dec
}  // namespace attn
