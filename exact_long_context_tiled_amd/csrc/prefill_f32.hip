// Tiled exact attention prefill for fp32 operands (fp32 FMA arithmetic
// throughout, so results stay within fp32 rounding of the exact value).
//
// Same scheme as the bf16 kernel -- one pass over key tiles with an online
// softmax (ONNX Runtime PR #28695 analysis, section 1), work-groups serving
// one KV head and a tile of packed (position, head-in-group) rows so K/V tiles
// in LDS are shared by the whole query-head group -- but the dot products run
// on the vector ALUs.  Two kernels share the arithmetic:
//
// * the row-tile kernel: each packed row is owned by D/64 adjacent lanes
//   holding 64 components of q and of the output accumulator, 256 (D = 64)
//   or 128 (D = 128) rows per work-group;
// * the key-split kernel, for launches whose row tiles would leave compute
//   units idle (a short sequence makes a handful of row tiles): a work-group
//   serves 64 / LPR packed rows (LPR = D / 8 lanes per row, 8 components
//   each), all four waves hold the same rows, and the keys of each tile are
//   dealt among the waves, each running its own online softmax.  The waves'
//   (m, l, acc) are merged by the log-sum-exp rule of the split-KV reduce
//   phase (same page, section 2) at the end.
#include <math.h>

#include "common.h"

namespace attn {
namespace {

constexpr int kBKf = 32;  // keys per LDS tile of the row-tile kernel

struct RowRange {
  bool ok;       // the packed row exists
  int64_t pos;   // its query position
  int h;         // its query head
  int64_t lim;   // last visible local key (-1: none)
};

// Packed row r of KV head hk: position r / G, query head hk*G + r mod G.
__device__ inline RowRange packed_row(const PrefillArgs& a, int hk, int64_t r) {
  RowRange x{r < a.n_q * a.G, 0, 0, -1};
  if (x.ok) {
    x.pos = r / a.G;
    x.h = hk * a.G + (int)(r - x.pos * a.G);
    x.lim = a.n_k - 1;
    if (a.causal) x.lim = min(x.lim, a.q_abs0 + x.pos - a.k_abs0);
  }
  return x;
}

// Keys [0, kend) hold every key visible to packed rows up to r_last.
__device__ inline int64_t keys_seen(const PrefillArgs& a, int64_t r_last) {
  const int64_t pos_hi = min(r_last, a.n_q * a.G - 1) / a.G;
  if (!a.causal) return a.n_k;
  return min(a.n_k, max((int64_t)0, a.q_abs0 + pos_hi - a.k_abs0 + 1));
}

// Epilogue of one lane: O = acc / l and lse = m + log2(l) (in ln units) for
// ND components starting at d0, or, with accumulate, the log-sum-exp merge of
// that result into the (O, lse) already stored.  A row with no visible key
// has l = 0: O = 0 and lse = -inf.
template <int ND>
__device__ inline void store_row(const PrefillArgs& a, int b, const RowRange& x, int D, int d0, bool lse_lane,
                                 const float* acc, float m, float l) {
  float lse_v = -INFINITY, inv = 0.f;
  if (l > 0.f) {
    inv = 1.f / l;
    lse_v = (m + log2f(l)) * kLn2;
  }
  float* orow = a.o + b * a.o_sb + x.pos * a.o_ss + (int64_t)x.h * D + d0;
  float* lse_p = a.lse ? a.lse + b * a.l_sb + (int64_t)x.h * a.l_sh + x.pos : nullptr;
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
  for (int d = 0; d < ND; d += 4) {
    float4 ov = {0.f, 0.f, 0.f, 0.f};
    if (have_old) ov = *(const float4*)(orow + d);
    float4 nv;
    nv.x = w_old * ov.x + w_new * acc[d];
    nv.y = w_old * ov.y + w_new * acc[d + 1];
    nv.z = w_old * ov.z + w_new * acc[d + 2];
    nv.w = w_old * ov.w + w_new * acc[d + 3];
    *(float4*)(orow + d) = nv;
  }
  if (lse_lane && lse_p) *lse_p = lse_out;
}

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

  const int64_t r0 = (int64_t)tile * RPB;
  const RowRange x = packed_row(a, hk, r0 + w * RPW + lane / LPR);
  const int64_t kend = keys_seen(a, r0 + RPB - 1);

  float q[64], acc[64];
  const float* qrow = (const float*)a.q + b * a.q_sb + x.pos * a.q_ss + (int64_t)x.h * D + d0;
#pragma unroll
  for (int d = 0; d < 64; d += 4) {
    float4 t = x.ok ? *(const float4*)(qrow + d) : float4{0.f, 0.f, 0.f, 0.f};
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

    float s[kBKf];
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
      if (k0 + j > x.lim) xs = -INFINITY;
      s[j] = xs;
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
      const float p = exp2f(s[j] - m_use);
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

  if (!x.ok) return;
  store_row<64>(a, b, x, D, d0, part == 0, acc, m, l);
}

// Sum over the LPR adjacent lanes of a row (row-local DPP moves).
template <int LPR>
__device__ inline float row_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xf, 0xf, false));  // xor 1
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xf, 0xf, false));  // xor 2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false));  // mirror in 8
  if constexpr (LPR == 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xf, 0xf, false));  // mirror in 16
  return v;
}

constexpr int kSplitWaves = 4;

template <int D>
__global__ void __launch_bounds__(256) prefill_f32_split_kernel(PrefillArgs a, int n_row_tiles) {
  constexpr int LPR = D / 8;           // lanes per packed row (8 components each)
  constexpr int RPB = 64 / LPR;        // packed rows per work-group (shared by its waves)
  constexpr int kBKs = 4096 / D;      // keys per LDS tile (a 16 KB K tile)
  constexpr int KPW = kBKs / kSplitWaves;  // keys of a tile per wave
  constexpr int NV4 = kBKs * D / 4;    // float4 per K (or V) tile
  constexpr int PER = NV4 / 256;       // ... per thread
  static_assert(LPR == 8 || LPR == 16, "D = 64 or 128");
  // two stages: tile t+1 is read from global memory while tile t is used
  __shared__ __attribute__((aligned(16))) float Ks[2][kBKs * D];
  __shared__ __attribute__((aligned(16))) float Vs[2][kBKs * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int part = lane % LPR;
  const int d0 = 8 * part;
  const int tile = n_row_tiles - 1 - (int)blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;

  const int64_t r0 = (int64_t)tile * RPB;
  const RowRange x = packed_row(a, hk, r0 + lane / LPR);
  const int64_t kend = keys_seen(a, r0 + RPB - 1);
  const int ntiles = (int)((kend + kBKs - 1) / kBKs);

  float q[8], acc[8];
  {
    const float* qrow = (const float*)a.q + b * a.q_sb + x.pos * a.q_ss + (int64_t)x.h * D + d0;
    const float4 q0 = x.ok ? *(const float4*)qrow : float4{0.f, 0.f, 0.f, 0.f};
    const float4 q1 = x.ok ? *(const float4*)(qrow + 4) : float4{0.f, 0.f, 0.f, 0.f};
    q[0] = q0.x, q[1] = q0.y, q[2] = q0.z, q[3] = q0.w;
    q[4] = q1.x, q[5] = q1.y, q[6] = q1.z, q[7] = q1.w;
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float* kbase = (const float*)a.k + b * a.k_sb + (int64_t)hk * D;
  const float* vbase = (const float*)a.v + b * a.k_sb + (int64_t)hk * D;

  // this thread's share of a tile: float4 number tid + 256c (keys past the
  // block read as zeros, and are masked)
  float4 kr[PER], vr[PER];
  auto fetch = [&](int t) {
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int idx = tid + 256 * c;
      const int64_t j = (int64_t)t * kBKs + idx / (D / 4);
      const int col = (idx % (D / 4)) * 4;
      kr[c] = vr[c] = float4{0.f, 0.f, 0.f, 0.f};
      if (j < a.n_k) {
        kr[c] = *(const float4*)(kbase + j * a.k_ss + col);
        vr[c] = *(const float4*)(vbase + j * a.k_ss + col);
      }
    }
  };
  if (ntiles > 0) fetch(0);
  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    // Stage st was last read in tile t - 2, which every wave finished
    // before the previous barrier.
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int idx = tid + 256 * c;
      *(float4*)(Ks[st] + 4 * idx) = kr[c];
      *(float4*)(Vs[st] + 4 * idx) = vr[c];
    }
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);

    // keys 4i + w of the tile
    const int64_t k0 = (int64_t)t * kBKs;
    float s[KPW];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int j = kSplitWaves * i + w;
      const float4 k_lo = *(const float4*)(Ks[st] + j * D + d0);
      const float4 k_hi = *(const float4*)(Ks[st] + j * D + d0 + 4);
      float dot = q[0] * k_lo.x;
      dot = fmaf(q[1], k_lo.y, dot);
      dot = fmaf(q[2], k_lo.z, dot);
      dot = fmaf(q[3], k_lo.w, dot);
      dot = fmaf(q[4], k_hi.x, dot);
      dot = fmaf(q[5], k_hi.y, dot);
      dot = fmaf(q[6], k_hi.z, dot);
      dot = fmaf(q[7], k_hi.w, dot);
      float xs = row_sum<LPR>(dot) * a.scale_log2;
      if (k0 + j > x.lim) xs = -INFINITY;
      s[i] = xs;
      tmax = fmaxf(tmax, xs);
    }
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] *= alpha;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int j = kSplitWaves * i + w;
      const float p = exp2f(s[i] - m_use);
      l += p;
      const float4 v_lo = *(const float4*)(Vs[st] + j * D + d0);
      const float4 v_hi = *(const float4*)(Vs[st] + j * D + d0 + 4);
      acc[0] = fmaf(p, v_lo.x, acc[0]);
      acc[1] = fmaf(p, v_lo.y, acc[1]);
      acc[2] = fmaf(p, v_lo.z, acc[2]);
      acc[3] = fmaf(p, v_lo.w, acc[3]);
      acc[4] = fmaf(p, v_hi.x, acc[4]);
      acc[5] = fmaf(p, v_hi.y, acc[5]);
      acc[6] = fmaf(p, v_hi.z, acc[6]);
      acc[7] = fmaf(p, v_hi.w, acc[7]);
    }
    m = m_new;
  }

  // Merge the waves' partial softmax states: M = max m_w, l = sum l_w 2^(m_w - M),
  // acc = sum acc_w 2^(m_w - M).  Waves 1..3 leave theirs in LDS (stage 0 of
  // Ks, free once every wave is past its last tile), wave 0 merges and stores.
  __syncthreads();
  float* red = Ks[0];  // [waves - 1][64 lanes][8 acc + m + l]
  if (w > 0) {
    float* p = red + ((w - 1) * 64 + lane) * 10;
#pragma unroll
    for (int d = 0; d < 8; ++d) p[d] = acc[d];
    p[8] = m;
    p[9] = l;
  }
  __syncthreads();
  if (w != 0) return;
  float M = m;
#pragma unroll
  for (int u = 1; u < kSplitWaves; ++u) M = fmaxf(M, red[((u - 1) * 64 + lane) * 10 + 8]);
  const float M_use = M == -INFINITY ? 0.f : M;
  const float w0 = exp2f(m - M_use);
  l *= w0;
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] *= w0;
#pragma unroll
  for (int u = 1; u < kSplitWaves; ++u) {
    const float* p = red + ((u - 1) * 64 + lane) * 10;
    const float wu = exp2f(p[8] - M_use);
    l = fmaf(p[9], wu, l);
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = fmaf(p[d], wu, acc[d]);
  }
  if (!x.ok) return;
  store_row<8>(a, b, x, D, d0, part == 0, acc, M, l);
}

template <int D>
attn_status launch_f32(const PrefillArgs& a, hipStream_t stream) {
  const int64_t rows = a.n_q * a.G;
  constexpr int kRowTile = 4 * (64 / (D / 64));  // rows of the row-tile kernel's work-group
  constexpr int kSplitRows = 64 / (D / 8);       // rows of the key-split kernel's work-group
  const int64_t tiles = (rows + kRowTile - 1) / kRowTile;
  if (tiles * a.Hkv * a.B < device_cu_count()) {
    const int64_t st = (rows + kSplitRows - 1) / kSplitRows;
    if (st > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "prefill: too many query rows per launch");
    hipLaunchKernelGGL(prefill_f32_split_kernel<D>, dim3((unsigned)st, a.Hkv, a.B), dim3(256), 0, stream, a, (int)st);
  } else {
    if (tiles > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "prefill: too many query rows per launch");
    hipLaunchKernelGGL(prefill_f32_kernel<D>, dim3((unsigned)tiles, a.Hkv, a.B), dim3(256), 0, stream, a,
                       (int)tiles);
  }
  return check_launch("prefill_f32");
}

}  // namespace

attn_status launch_prefill_f32(const PrefillArgs& a, int D, hipStream_t stream) {
  if (a.n_q * a.G == 0 || a.B == 0) return ATTN_OK;
  return D == 128 ? launch_f32<128>(a, stream) : launch_f32<64>(a, stream);
}

}  // namespace attn
