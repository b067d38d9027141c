// Exact log-sum-exp merge of normalised partial attention results (the reduce
// phase of flash decoding: ONNX Runtime PR #28695 analysis, section 2; the
// exact recombination of independent sub-results: Stream-CQSA summary,
// "Methodology" item 2).
//
// One wave per output row: every lane reads the n partial lse values (the same
// addresses, served as one broadcast), forms the weights, then streams its
// share of the D columns of every non-empty partial.
#include <math.h>

#include "common.h"

namespace attn {
namespace {

__global__ void __launch_bounds__(256) merge_kernel(int n, const float* __restrict__ op,
                                                    const float* __restrict__ lp, int64_t R, int D,
                                                    float* __restrict__ o, float* __restrict__ lse) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= R) return;
  float M = -INFINITY;
  for (int c = 0; c < n; ++c) M = fmaxf(M, lp[(int64_t)c * R + row]);
  float* orow = o + row * D;
  if (M == -INFINITY) {
    for (int d = lane; d < D; d += 64) orow[d] = 0.f;
    if (lane == 0 && lse) lse[row] = -INFINITY;
    return;
  }
  float den = 0.f;
  for (int c = 0; c < n; ++c) den += expf(lp[(int64_t)c * R + row] - M);
  const float inv = 1.f / den;
  for (int d = lane; d < D; d += 64) {
    float acc = 0.f;
    for (int c = 0; c < n; ++c) {
      const float lc = lp[(int64_t)c * R + row];
      if (lc == -INFINITY) continue;  // empty partial: its O is never read
      acc = fmaf(expf(lc - M), op[((int64_t)c * R + row) * D + d], acc);
    }
    orow[d] = acc * inv;
  }
  if (lane == 0 && lse) lse[row] = M + logf(den);
}

}  // namespace

attn_status launch_merge(int n, const float* o_parts, const float* lse_parts, int64_t R, int D, float* o,
                         float* lse, hipStream_t stream) {
  if (R == 0) return ATTN_OK;
  const int64_t blocks = (R + 3) / 4;
  if (blocks > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "merge: too many rows");
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, n, o_parts, lse_parts, R, D, o,
                     lse);
  return check_launch("merge");
}

}  // namespace attn
