// Tiled exact attention prefill, bf16 operands on gfx950 matrix cores.
//
// One pass over key tiles with an online softmax (running row max m and row
// sum l, rescaling the fp32 output accumulator by exp(m_old - m_new)), the
// P.V product accumulated in fp32: the tiled flash-attention scheme of the
// ONNX Runtime PR #28695 analysis (section 1), laid out for CDNA4 waves.
//
// Work decomposition
//   grid = (row tiles, Hkv, B).  A work-group serves ONE KV head and a tile of
//   128 "packed" query rows r = position * G + g (g = query head within the
//   group), so every K/V tile staged in LDS is shared by all G query heads of
//   the group (GQA reuse: LLM-CoOpt, "Methodology" item 2).  Row tiles are
//   issued heaviest first (the causal ones that see the most keys).
//   4 waves x 32 packed rows each.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16)
//   S^T = K Q^T   : A = K tile rows (from LDS), B = Q rows (registers), so a
//                   lane's accumulator column is ONE query row and the row max /
//                   sum need only a swap with the other half-wave.
//   O^T += V^T P^T: A = V^T (from a transposed LDS tile), B = P^T taken straight
//                   from the S^T accumulator.  To make that possible the K rows
//                   are fed to the first product in a permuted order (bits 2 and
//                   3 of the row index swapped), which makes accumulator
//                   registers 0-7 / 8-15 of a lane hold 8 consecutive keys.
#include <math.h>

#include "common.h"

namespace attn {
namespace {

constexpr int kRowsPerWG = 128;
constexpr int kBK = 64;  // keys per tile

__device__ __forceinline__ int perm_row(int m) {
  // swap bits 2 and 3
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
__global__ void __launch_bounds__(256) prefill_bf16_kernel(PrefillArgs a, int n_row_tiles) {
  constexpr int KP = D + 8;    // K tile row pitch (bf16 elements)
  constexpr int VP = kBK + 8;  // V^T tile row pitch
  constexpr int NKK = D / 16;  // 16-wide chunks of D for S = Q K^T
  constexpr int NDB = D / 32;  // 32-row blocks of D for O^T
  constexpr int CPR = D / 8;   // 16-byte chunks per K/V row
  constexpr int NCH = kBK * CPR / 256;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBK * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int tile = n_row_tiles - 1 - (int)blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.G;

  const int64_t rows_total = a.n_q * G;
  const int64_t r0 = (int64_t)tile * kRowsPerWG;
  const int64_t r = r0 + 32 * w + n;
  const bool row_ok = r < rows_total;
  int64_t pos = 0;
  int h = 0;
  if (row_ok) {
    pos = r / G;
    h = hk * G + (int)(r - pos * G);
  }
  // last visible local key of this row
  int64_t lim = -1;
  if (row_ok) {
    lim = a.n_k - 1;
    if (a.causal) lim = min(lim, a.q_abs0 + pos - a.k_abs0);
  }
  // keys this work-group visits, and the prefix visible to all of its rows
  const int64_t pos_lo = r0 / G;
  const int64_t pos_hi = min(r0 + kRowsPerWG - 1, rows_total - 1) / G;
  int64_t kend = a.n_k, kfull = a.n_k;
  if (a.causal) {
    kend = min(a.n_k, max((int64_t)0, a.q_abs0 + pos_hi - a.k_abs0 + 1));
    kfull = min(a.n_k, max((int64_t)0, a.q_abs0 + pos_lo - a.k_abs0 + 1));
  }

  const uint16_t* qrow = (const uint16_t*)a.q + b * a.q_sb + pos * a.q_ss + (int64_t)h * D;
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    if (row_ok)
      qf[kk] = *(const bf16x8*)(qrow + 16 * kk + 8 * hh);
    else
      qf[kk] = bf16x8{};
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const uint16_t* kbase = (const uint16_t*)a.k + b * a.k_sb + (int64_t)hk * D;
  const uint16_t* vbase = (const uint16_t*)a.v + b * a.k_sb + (int64_t)hk * D;
  const int krow = perm_row(n);

  for (int64_t k0 = 0; k0 < kend; k0 += kBK) {
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + 256 * i;
      const int key = c / CPR;
      const int col = (c % CPR) * 8;
      const int64_t j = k0 + key;
      uint4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (j < a.n_k) {
        kv = *(const uint4*)(kbase + j * a.k_ss + col);
        vv = *(const uint4*)(vbase + j * a.k_ss + col);
      }
      *(uint4*)(Ks + key * KP + col) = kv;
      const uint16_t* ve = (const uint16_t*)&vv;
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(col + e) * VP + key] = ve[e];
    }
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16{};
      const uint16_t* kr = Ks + (32 * mb + krow) * KP + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) s[mb] = mfma32(*(const bf16x8*)(kr + 16 * kk), qf[kk], s[mb]);
    }

    const bool need_mask = k0 + kBK > kfull;
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[mb][i] * a.scale_log2;
        if (need_mask) {
          const int64_t key = k0 + 32 * mb + 16 * (i >> 3) + 8 * hh + (i & 7);
          if (key > lim) x = -INFINITY;
        }
        s[mb][i] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    float psum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[mb][i] - m_use);
        psum += p;
        pf[2 * mb + (i >> 3)][i & 7] = (__bf16)p;
      }
    }
    l = l * alpha + psum;
    m = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint16_t* vr = Vt + (32 * db + n) * VP + 8 * hh;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[db] = mfma32(*(const bf16x8*)(vr + 16 * c), pf[c], acc[db]);
    }
  }

  const float lt = l + __shfl_xor(l, 32);
  if (!row_ok) return;
  float lse_v = -INFINITY;
  float inv = 0.f;
  if (lt > 0.f) {
    inv = 1.f / lt;
    lse_v = (m + __log2f(lt)) * kLn2;
  }
  float* orow = a.o + b * a.o_sb + pos * a.o_ss + (int64_t)h * D;
  float* lse_p = a.lse ? a.lse + b * a.l_sb + (int64_t)h * a.l_sh + pos : nullptr;
  if (a.accumulate) {
    const float old = *lse_p;
    const float M = fmaxf(old, lse_v);
    float w_old = 0.f, w_new = 0.f, lse_out = -INFINITY;
    if (M != -INFINITY) {
      w_old = expf(old - M);
      w_new = expf(lse_v - M);
      const float den = w_old + w_new;
      w_old /= den;
      w_new = w_new * inv / den;
      lse_out = M + logf(den);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        float4* dst = (float4*)(orow + 32 * db + 8 * ig + 4 * hh);
        float4 ov = *dst;
        if (old == -INFINITY) ov = float4{0.f, 0.f, 0.f, 0.f};  // nothing merged yet
        float4 nv;
        nv.x = w_old * ov.x + w_new * acc[db][4 * ig + 0];
        nv.y = w_old * ov.y + w_new * acc[db][4 * ig + 1];
        nv.z = w_old * ov.z + w_new * acc[db][4 * ig + 2];
        nv.w = w_old * ov.w + w_new * acc[db][4 * ig + 3];
        *dst = nv;
      }
    }
    if (hh == 0) *lse_p = lse_out;
  } else {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        float4 nv;
        nv.x = acc[db][4 * ig + 0] * inv;
        nv.y = acc[db][4 * ig + 1] * inv;
        nv.z = acc[db][4 * ig + 2] * inv;
        nv.w = acc[db][4 * ig + 3] * inv;
        *(float4*)(orow + 32 * db + 8 * ig + 4 * hh) = nv;
      }
    }
    if (hh == 0 && lse_p) *lse_p = lse_v;
  }
}

}  // namespace

attn_status launch_prefill_bf16(const PrefillArgs& a, int D, hipStream_t stream) {
  const int64_t rows = a.n_q * a.G;
  const int64_t tiles = (rows + kRowsPerWG - 1) / kRowsPerWG;
  if (tiles == 0 || a.B == 0) return ATTN_OK;
  if (tiles > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "prefill: too many query rows per launch");
  dim3 grid((unsigned)tiles, a.Hkv, a.B);
  if (D == 128)
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, dim3(256), 0, stream, a, (int)tiles);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, dim3(256), 0, stream, a, (int)tiles);
  return check_launch("prefill_bf16");
}

}  // namespace attn
