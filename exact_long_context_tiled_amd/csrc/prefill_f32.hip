// Tiled exact attention prefill for fp32 operands (fp32 FMA arithmetic
// throughout, so results stay within fp32 rounding of the exact value).
//
// Same scheme as the bf16 kernel -- one pass over key tiles with an online
// softmax (ONNX Runtime PR #28695 analysis, section 1), work-groups serving
// one KV head and a tile of packed (position, head-in-group) rows so K/V tiles
// in LDS are shared by the whole query-head group -- but the dot products run
// on the vector ALUs: each packed row is owned by D/64 adjacent lanes holding
// 64 components of q and of the output accumulator.
#include <math.h>

#include "common.h"

namespace attn {
namespace {

constexpr int kBKf = 32;  // keys per LDS tile

template <int D>
__global__ void __launch_bounds__(256) prefill_f32_kernel(PrefillArgs a, int n_row_tiles) {
  constexpr int LPR = D / 64;         // lanes per packed row
  constexpr int RPW = 64 / LPR;       // packed rows per wave
  constexpr int RPB = 4 * RPW;        // packed rows per work-group
  constexpr int NV4 = kBKf * D / 4;   // float4 per K (or V) tile
  __shared__ __attribute__((aligned(16))) float Ks[kBKf * D];
  __shared__ __attribute__((aligned(16))) float Vs[kBKf * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int part = lane % LPR;
  const int d0 = part * 64;
  const int tile = n_row_tiles - 1 - (int)blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.G;

  const int64_t rows_total = a.n_q * G;
  const int64_t r0 = (int64_t)tile * RPB;
  const int64_t r = r0 + w * RPW + lane / LPR;
  const bool row_ok = r < rows_total;
  int64_t pos = 0;
  int h = 0;
  if (row_ok) {
    pos = r / G;
    h = hk * G + (int)(r - pos * G);
  }
  int64_t lim = -1;
  if (row_ok) {
    lim = a.n_k - 1;
    if (a.causal) lim = min(lim, a.q_abs0 + pos - a.k_abs0);
  }
  const int64_t pos_hi = min(r0 + RPB - 1, rows_total - 1) / G;
  int64_t kend = a.n_k;
  if (a.causal) kend = min(a.n_k, max((int64_t)0, a.q_abs0 + pos_hi - a.k_abs0 + 1));

  float q[64], acc[64];
  const float* qrow = (const float*)a.q + b * a.q_sb + pos * a.q_ss + (int64_t)h * D + d0;
#pragma unroll
  for (int d = 0; d < 64; d += 4) {
    float4 t = row_ok ? *(const float4*)(qrow + d) : float4{0.f, 0.f, 0.f, 0.f};
    q[d] = t.x;
    q[d + 1] = t.y;
    q[d + 2] = t.z;
    q[d + 3] = t.w;
    acc[d] = acc[d + 1] = acc[d + 2] = acc[d + 3] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float* kbase = (const float*)a.k + b * a.k_sb + (int64_t)hk * D;
  const float* vbase = (const float*)a.v + b * a.k_sb + (int64_t)hk * D;

  for (int64_t k0 = 0; k0 < kend; k0 += kBKf) {
    __syncthreads();
    for (int c = tid; c < NV4; c += 256) {
      const int key = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      const int64_t j = k0 + key;
      float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (j < a.n_k) {
        kv = *(const float4*)(kbase + j * a.k_ss + col);
        vv = *(const float4*)(vbase + j * a.k_ss + col);
      }
      *(float4*)(Ks + key * D + col) = kv;
      *(float4*)(Vs + key * D + col) = vv;
    }
    __syncthreads();

    float x[kBKf];
    float tmax = -INFINITY;
#pragma unroll 4
    for (int j = 0; j < kBKf; ++j) {
      const float* kr = Ks + j * D + d0;
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < 64; d += 4) {
        const float4 kv = *(const float4*)(kr + d);
        dot = fmaf(q[d], kv.x, dot);
        dot = fmaf(q[d + 1], kv.y, dot);
        dot = fmaf(q[d + 2], kv.z, dot);
        dot = fmaf(q[d + 3], kv.w, dot);
      }
      if (LPR == 2) dot += __shfl_xor(dot, 1);
      float xs = dot * a.scale_log2;
      if (k0 + j > lim) xs = -INFINITY;
      x[j] = xs;
      tmax = fmaxf(tmax, xs);
    }
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < 64; ++d) acc[d] *= alpha;
#pragma unroll 4
    for (int j = 0; j < kBKf; ++j) {
      const float p = exp2f(x[j] - m_use);
      l += p;
      const float* vr = Vs + j * D + d0;
#pragma unroll
      for (int d = 0; d < 64; d += 4) {
        const float4 vv = *(const float4*)(vr + d);
        acc[d] = fmaf(p, vv.x, acc[d]);
        acc[d + 1] = fmaf(p, vv.y, acc[d + 1]);
        acc[d + 2] = fmaf(p, vv.z, acc[d + 2]);
        acc[d + 3] = fmaf(p, vv.w, acc[d + 3]);
      }
    }
    m = m_new;
  }

  if (!row_ok) return;
  float lse_v = -INFINITY, inv = 0.f;
  if (l > 0.f) {
    inv = 1.f / l;
    lse_v = (m + log2f(l)) * kLn2;
  }
  float* orow = a.o + b * a.o_sb + pos * a.o_ss + (int64_t)h * D + d0;
  float* lse_p = a.lse ? a.lse + b * a.l_sb + (int64_t)h * a.l_sh + pos : nullptr;
  float w_old = 0.f, w_new = inv, lse_out = lse_v;
  bool have_old = false;
  if (a.accumulate) {
    const float old = *lse_p;
    have_old = old != -INFINITY;
    const float M = fmaxf(old, lse_v);
    w_new = 0.f;
    lse_out = -INFINITY;
    if (M != -INFINITY) {
      w_old = expf(old - M);
      const float wn = expf(lse_v - M);
      const float den = w_old + wn;
      w_old /= den;
      w_new = wn * inv / den;
      lse_out = M + logf(den);
    }
  }
#pragma unroll
  for (int d = 0; d < 64; d += 4) {
    float4 ov = {0.f, 0.f, 0.f, 0.f};
    if (have_old) ov = *(const float4*)(orow + d);
    float4 nv;
    nv.x = w_old * ov.x + w_new * acc[d];
    nv.y = w_old * ov.y + w_new * acc[d + 1];
    nv.z = w_old * ov.z + w_new * acc[d + 2];
    nv.w = w_old * ov.w + w_new * acc[d + 3];
    *(float4*)(orow + d) = nv;
  }
  if (part == 0 && lse_p) *lse_p = lse_out;
}

}  // namespace

attn_status launch_prefill_f32(const PrefillArgs& a, int D, hipStream_t stream) {
  const int rpb = 4 * (64 / (D / 64));
  const int64_t rows = a.n_q * a.G;
  const int64_t tiles = (rows + rpb - 1) / rpb;
  if (tiles == 0 || a.B == 0) return ATTN_OK;
  if (tiles > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "prefill: too many query rows per launch");
  dim3 grid((unsigned)tiles, a.Hkv, a.B);
  if (D == 128)
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(256), 0, stream, a, (int)tiles);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(256), 0, stream, a, (int)tiles);
  return check_launch("prefill_f32");
}

}  // namespace attn
