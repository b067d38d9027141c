// Exact log-sum-exp merge of normalised partial attention results (the reduce
// phase of flash decoding: ONNX Runtime PR #28695 analysis, section 2; the
// exact recombination of independent sub-results: Stream-CQSA summary,
// "Methodology" item 2).
//
#include <math.h>

#include "common.h"

namespace attn {
namespace {

__device__ __forceinline__ float block_max(float x, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// One work-group per output row.  The partials' weights are formed once per
// chunk of 256 partials in LDS; the columns are then accumulated by
// 256 / D thread groups in parallel (each over a strided subset of the
// partials) and the groups are summed at the end.
__global__ void __launch_bounds__(256) merge_kernel(int n, const float* __restrict__ op,
                                                    const float* __restrict__ lp, int64_t R, int D,
                                                    float* __restrict__ o, float* __restrict__ lse) {
  __shared__ float wts[256];
  __shared__ float red[4];
  __shared__ float part[256];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  float mx = -INFINITY;
  for (int c = tid; c < n; c += 256) mx = fmaxf(mx, lp[(int64_t)c * R + row]);
  mx = block_max(mx, red);
  float* orow = o + row * D;
  if (mx == -INFINITY) {  // no partial holds a key
    for (int d = tid; d < D; d += 256) orow[d] = 0.f;
    if (tid == 0 && lse) lse[row] = -INFINITY;
    return;
  }
  // Column groups working on disjoint partials: ng groups of D threads when
  // D <= 128, else one group in which thread tid owns columns tid + 256k
  // (for 128 < D < 256 the threads tid >= D own no column and stay idle).
  const int ng = D > 128 ? 1 : 256 / D;
  const int grp = D > 128 ? 0 : tid / D;
  const int dl = D > 128 ? tid : tid % D;
  const bool active = grp < ng && dl < D;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};  // D <= 1024 -> at most 4 columns per thread
  float den = 0.f;
  for (int c0 = 0; c0 < n; c0 += 256) {
    __syncthreads();
    float wv = 0.f;
    if (c0 + tid < n) {
      const float lc = lp[(int64_t)(c0 + tid) * R + row];
      wv = lc == -INFINITY ? 0.f : expf(lc - mx);  // an empty partial's O is never read
    }
    wts[tid] = wv;
    den += wv;
    __syncthreads();
    const int cend = min(256, n - c0);
    if (active) {
      for (int c = grp; c < cend; c += ng) {
        const float wc = wts[c];
        if (wc == 0.f) continue;
        const float* src = op + ((int64_t)(c0 + c) * R + row) * D;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int d = dl + 256 * k;
          if (d < D) acc[k] = fmaf(wc, src[d], acc[k]);
        }
      }
    }
  }
  den = block_sum(den, red);
  const float inv = 1.f / den;
  if (ng > 1) {
    part[tid] = acc[0];
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
      for (int g = 0; g < ng; ++g) s += part[g * D + tid];
      orow[tid] = s * inv;
    }
  } else if (active) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = dl + 256 * k;
      if (d < D) orow[d] = acc[k] * inv;
    }
  }
  if (tid == 0 && lse) lse[row] = mx + logf(den);
}

}  // namespace

attn_status launch_merge(int n, const float* o_parts, const float* lse_parts, int64_t R, int D, float* o,
                         float* lse, hipStream_t stream) {
  if (R == 0) return ATTN_OK;
  if (R > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "merge: too many rows");
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)R), dim3(256), 0, stream, n, o_parts, lse_parts, R, D, o, lse);
  return check_launch("merge");
}

}  // namespace attn
