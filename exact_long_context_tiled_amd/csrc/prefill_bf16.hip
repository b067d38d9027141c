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

constexpr int kWaves = 8;                  // 2 per SIMD: one wave's softmax overlaps the other's MFMAs
constexpr int kRowsPerWG = 32 * kWaves;    // 32 packed rows per wave
constexpr int kBK = 64;                    // keys per tile
constexpr int kThreads = 64 * kWaves;

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ int perm_row(int m) {
  // swap bits 2 and 3
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value of lane (l ^ 32): v_permlane32_swap returns {x[l], x[l^32]} in some order.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct Tile {
  static constexpr int KP = D + 8;   // K row pitch (bf16): consecutive rows shift by 4 banks
  static constexpr int VP = D + 32;  // V row pitch: transposed reads of 4 rows hit disjoint banks
  static constexpr int K_ELEMS = kBK * KP;
  static constexpr int V_ELEMS = kBK * VP;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr int BYTES = 2 * BUF * 2;  // double buffered
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int NCH = kBK * CPR / kThreads;  // chunks of K (and of V) per thread
};

template <int D>
__global__ void __launch_bounds__(kThreads, 1) prefill_bf16_kernel(PrefillArgs a, int n_row_tiles) {
  using TL = Tile<D>;
  constexpr int NKK = D / 16;  // 16-wide chunks of D for S = Q K^T
  constexpr int NDB = D / 32;  // 32-row blocks of D for O^T
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int tile = n_row_tiles - 1 - (int)blockIdx.x;  // heaviest (causal) tiles first
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
  int64_t lim = -1;  // last visible local key of this row
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
  const int ntiles = (int)((kend + kBK - 1) / kBK);

  // Q rows as the B operand of S^T = K Q^T (8 consecutive d per lane)
  const uint16_t* qrow = (const uint16_t*)a.q + b * a.q_sb + pos * a.q_ss + (int64_t)h * D;
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = row_ok ? *(const bf16x8*)(qrow + 16 * kk + 8 * hh) : bf16x8{};

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m = -INFINITY;  // running max of the scaled scores (log2 domain)
  float l = 0.f;        // this lane's half of the running sum

  const uint16_t* kbase = (const uint16_t*)a.k + b * a.k_sb + (int64_t)hk * D;
  const uint16_t* vbase = (const uint16_t*)a.v + b * a.k_sb + (int64_t)hk * D;
  const int64_t nk1 = a.n_k - 1;

  // global -> registers for one K/V tile; keys past the block are clamped (and zeroed when stored)
  uint4 kpre[TL::NCH], vpre[TL::NCH];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < TL::NCH; ++i) {
      const int c = tid + kThreads * i;
      const int key = c / TL::CPR;
      const int col = (c % TL::CPR) * 8;
      const int64_t j = min((int64_t)t * kBK + key, nk1);
      kpre[i] = *(const uint4*)(kbase + j * a.k_ss + col);
      vpre[i] = *(const uint4*)(vbase + j * a.k_ss + col);
    }
  };
  auto store_tile = [&](int t, int buf) {
    uint16_t* Ks = lds + buf * TL::BUF;
    uint16_t* Vs = Ks + TL::K_ELEMS;
#pragma unroll
    for (int i = 0; i < TL::NCH; ++i) {
      const int c = tid + kThreads * i;
      const int key = c / TL::CPR;
      const int col = (c % TL::CPR) * 8;
      const bool in = (int64_t)t * kBK + key <= nk1;
      *(uint4*)(Ks + key * TL::KP + col) = in ? kpre[i] : uint4{0, 0, 0, 0};
      *(uint4*)(Vs + key * TL::VP + col) = in ? vpre[i] : uint4{0, 0, 0, 0};
    }
  };

  // per-lane LDS offsets of the matrix-core operands
  const int krow = perm_row(n);
  const int g16 = lane >> 4, r16 = lane & 15;
  // V^T operand by transposed reads: lane (a=r16/4, b=r16%4) of each 16-lane group
  // addresses key row 8*(g16/2) + a (+4), columns 16*(g16%2) + 4*b
  const int v_off = (8 * (g16 >> 1) + (r16 >> 2)) * TL::VP + 16 * (g16 & 1) + 4 * (r16 & 3);

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0, 0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* Ks = lds + cur * TL::BUF;
    const uint16_t* Vs = Ks + TL::K_ELEMS;
    const int64_t k0 = (int64_t)t * kBK;

    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16{};
      const uint16_t* kr = Ks + (32 * mb + krow) * TL::KP + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) s[mb] = mfma32(*(const bf16x8*)(kr + 16 * kk), qf[kk], s[mb]);
    }
    if (k0 + kBK > kfull) {  // tile reaches past the keys every row sees: mask per element
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t key = k0 + 32 * mb + 16 * (i >> 3) + 8 * hh + (i & 7);
          if (key > lim) s[mb][i] = -INFINITY;
        }
    }
    float tmax = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) tmax = fmaxf(tmax, fmaxf(s[0][i], s[0][i + 1]));
#pragma unroll
    for (int i = 0; i < 16; i += 2) tmax = fmaxf(tmax, fmaxf(s[1][i], s[1][i + 1]));
    tmax = half_swap_max(tmax);
    // scale > 0, so the max of the raw scores times scale*log2(e) is the scaled max
    const float m_new = fmaxf(m, tmax * a.scale_log2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    m = m_new;
    float psum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][i], a.scale_log2, -m_use));
        psum += p;
        pf[2 * mb + (i >> 3)][i & 7] = (__bf16)p;
      }
    }
    l = l * alpha + psum;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint16_t* vp = Vs + v_off + 16 * c * TL::VP + 32 * db;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)vp);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 4 * TL::VP));
        const i16x8 v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, v8);
        acc[db] = mfma32(vf, pf[c], acc[db]);
      }
    }
    if (t + 1 < ntiles) store_tile(t + 1, cur ^ 1);
    __syncthreads();
  }

  const float lt = half_swap_sum(l);
  if (!row_ok) return;
  float lse_v = -INFINITY;
  float inv = 0.f;
  if (lt > 0.f) {
    inv = 1.f / lt;
    lse_v = (m + __log2f(lt)) * kLn2;
  }
  float* orow = a.o + b * a.o_sb + pos * a.o_ss + (int64_t)h * D;
  float* lse_p = a.lse ? a.lse + b * a.l_sb + (int64_t)h * a.l_sh + pos : nullptr;
  float w_old = 0.f, w_new = inv, lse_out = lse_v;
  bool have_old = false;
  if (a.accumulate) {  // merge with the (O, lse) already in memory by log-sum-exp
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
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      float4* dst = (float4*)(orow + 32 * db + 8 * ig + 4 * hh);
      float4 ov = {0.f, 0.f, 0.f, 0.f};
      if (have_old) ov = *dst;
      float4 nv;
      nv.x = w_old * ov.x + w_new * acc[db][4 * ig + 0];
      nv.y = w_old * ov.y + w_new * acc[db][4 * ig + 1];
      nv.z = w_old * ov.z + w_new * acc[db][4 * ig + 2];
      nv.w = w_old * ov.w + w_new * acc[db][4 * ig + 3];
      *dst = nv;
    }
  }
  if (hh == 0 && lse_p) *lse_p = lse_out;
}

template <int D>
attn_status launch_d(const PrefillArgs& a, int tiles, hipStream_t stream) {
  static bool attr_set[64] = {false};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    const hipError_t e = hipFuncSetAttribute((const void*)prefill_bf16_kernel<D>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, Tile<D>::BYTES);
    if (e != hipSuccess) return set_error(ATTN_E_DEVICE, "prefill_bf16: LDS attribute: %s", hipGetErrorString(e));
    attr_set[dev] = true;
  }
  dim3 grid((unsigned)tiles, a.Hkv, a.B);
  hipLaunchKernelGGL(prefill_bf16_kernel<D>, grid, dim3(kThreads), Tile<D>::BYTES, stream, a, tiles);
  return check_launch("prefill_bf16");
}

}  // namespace

attn_status launch_prefill_bf16(const PrefillArgs& a, int D, hipStream_t stream) {
  const int64_t rows = a.n_q * a.G;
  const int64_t tiles = (rows + kRowsPerWG - 1) / kRowsPerWG;
  if (tiles == 0 || a.B == 0) return ATTN_OK;
  if (tiles > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "prefill: too many query rows per launch");
  return D == 128 ? launch_d<128>(a, (int)tiles, stream) : launch_d<64>(a, (int)tiles, stream);
}

}  // namespace attn
