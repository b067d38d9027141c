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

}  // namespace dec
}  // namespace attn
