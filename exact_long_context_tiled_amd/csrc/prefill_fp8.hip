// Tiled exact attention prefill with OCP e4m3fn (fp8) Q, K and V, per-head
// scales, on gfx950 matrix cores.
//
// Same scheme as the bf16 kernel (one pass over key tiles, online softmax,
// fp32 P.V accumulation: ONNX Runtime PR #28695 analysis, section 1; GQA
// reuse of each staged K/V tile by the G query heads of a KV head: LLM-CoOpt
// "Methodology" item 2; FP8 K/V halving the bytes per token: LLM-CoOpt
// "Methodology" item 1), with the operands kept in fp8 from HBM through LDS:
//
//   S^T = K Q^T  on v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit block
//                scales): a lane holds 32 consecutive bytes of its K row (A) and
//                of its Q row (B); D = 128 is two products per 32x32 block.
//                The raw scores are exact sums of products of e4m3 values; the
//                per-head scales q_scale[h] * k_scale[hk] join scale*log2(e) in
//                one per-lane multiplier (a lane's column is one query row).
//   O^T += V^T P^T on v_mfma_f32_32x32x16_bf16: P is rounded to bf16 (as in the
//                bf16 kernel: e4m3's 3-bit mantissa would cost several percent
//                per weight), and V^T comes from fp8 tiles by 8-bit transposing
//                LDS reads (ds_read_b64_tr_b8: 16 lanes turn an 8-key x 16-byte
//                block into one 8-key column each), converted exactly to bf16.
//                v_scale[hk] multiplies the output once, in the epilogue.
//
// K rows are fed in the permuted order of the bf16 kernel (bits 2 and 3 of
// the row swapped) so that the S^T accumulator registers of a lane hold runs
// of 8 consecutive keys, the B operand of the P.V product.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWG = 32 * kWaves;
constexpr int kBK = 64;  // keys per tile
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Asynchronous 16-byte copy from a buffer to LDS: lane i reads 16 bytes at
// byte offset voff of the buffer and writes them at LDS offset 16*i from the
// wave-uniform destination (the builtin exists in the device pass only).
constexpr int kBufDword3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format, no swizzle
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
#endif
}

__device__ __forceinline__ int perm_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0 = e4m3 for A and B; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Eight e4m3 bytes (keys in order) -> eight exact bf16 values.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(i32x2 raw) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// LDS tiles: kBK rows of D bytes, 16-byte chunks XOR-swizzled by the row: V
// by swz (chunk c of row r at c ^ (r mod chunks-per-row); 16 lanes read 8
// rows x 16 bytes), K by swz_k below (16 lanes read one chunk of 16 rows).
template <int D>
struct Tile8 {
  static constexpr int ROWB = D;                  // bytes per row
  static constexpr int CPR = D / 16;              // 16-byte chunks per row
  static constexpr int BYTES = kBK * ROWB;        // one K (or V) tile
  static constexpr int STAGE = 2 * BYTES;         // K + V
  static constexpr int ROWS_PER_COPY = 64 / CPR;  // rows one wave-wide copy covers
  static constexpr int COPIES = kBK / ROWS_PER_COPY / kWaves;
};
template <int D>
__device__ __forceinline__ int swz(int r) {
  return r & (D / 16 - 1);
}
// K tiles: chunk c of row r at c ^ ((r / (256 / row bytes)) mod chunks-per-row).
// 16 lanes read one chunk of 16 rows; rows of D bytes start 256 / D rows
// apart in bank order, so the swizzle must separate rows that agree mod
// 256 / D (r mod chunks-per-row alone gives rows r and r + 8 the same banks).
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return (r >> (D == 128 ? 1 : 2)) & (D / 16 - 1);
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) prefill_fp8_kernel(PrefillArgs a, int n_row_tiles) {
  using TL = Tile8<D>;
  constexpr int NKK = D / 64;  // 64-wide chunks of D for S = Q K^T
  constexpr int NDB = D / 32;  // 32-row blocks of D for O^T
  static_assert(TL::COPIES >= 1, "tile copy split");
  __shared__ __attribute__((aligned(1024))) char stage0[TL::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[TL::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;

  // XCD-aware work mapping, heaviest row tiles first (as in the bf16 kernel)
  const int total = n_row_tiles * a.Hkv * a.B;
  const int L = blockIdx.x;
  const int xcd = L % kXcds, kidx = L / kXcds;
  const int per = total / kXcds, rem = total % kXcds;
  const int W = xcd * per + min(xcd, rem) + kidx;
  const int pair = W / n_row_tiles;
  const int tile = n_row_tiles - 1 - (W - pair * n_row_tiles);
  const int hk = pair % a.Hkv;
  const int b = pair / a.Hkv;
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
  int64_t lim = -1;
  if (row_ok) {
    lim = a.n_k - 1;
    if (a.causal) lim = min(lim, a.q_abs0 + pos - a.k_abs0);
  }
  const int64_t pos_lo = r0 / G;
  const int64_t pos_hi = min(r0 + kRowsPerWG - 1, rows_total - 1) / G;
  int64_t kend = a.n_k, kfull = a.n_k;
  if (a.causal) {
    kend = min(a.n_k, max((int64_t)0, a.q_abs0 + pos_hi - a.k_abs0 + 1));
    kfull = min(a.n_k, max((int64_t)0, a.q_abs0 + pos_lo - a.k_abs0 + 1));
  }
  const int ntiles = (int)((kend + kBK - 1) / kBK);

  // score multiplier of this lane's query row: q and k head scales and scale*log2(e)
  const float qk_mul = a.q_scale[h] * a.k_scale[hk] * a.scale_log2;

  // Q row as the B operand of S^T = K Q^T: 32 consecutive bytes per lane half
  const uint8_t* qrow = (const uint8_t*)a.q + b * a.q_sb + pos * a.q_ss + (int64_t)h * D;
  i32x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = row_ok ? *(const i32x8*)(qrow + 64 * kk + 32 * hh) : i32x8{};

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m = -INFINITY;
  float l = 0.f;

  const uint8_t* kbase = (const uint8_t*)a.k + b * a.k_sb + (int64_t)hk * D;
  const uint8_t* vbase = (const uint8_t*)a.v + b * a.k_sb + (int64_t)hk * D;
  const int cp_row = lane / TL::CPR;
  const int cp_chunk = lane % TL::CPR;
  // Copies go through buffer resources whose base moves with the tile (scalar
  // registers); the per-lane byte offsets are loop-invariant.  The rows of
  // one lane's copies differ by multiples of the chunks per row, so V needs
  // one swizzled chunk offset and K (whose swizzle uses higher row bits) one
  // per copy.  Rows past the block are clamped onto the last key (finite
  // data, masked below): row offsets grow with the row, so the clamp is a min
  // on the offset.
  const int ksb = (int)a.k_ss;  // bytes between key rows (< 2^24)
  int rowb[TL::COPIES];
#pragma unroll
  for (int c = 0; c < TL::COPIES; ++c) rowb[c] = ((w * TL::COPIES + c) * TL::ROWS_PER_COPY + cp_row) * ksb;
  const int chb = 16 * (cp_chunk ^ swz<D>(w * TL::COPIES * TL::ROWS_PER_COPY + cp_row));  // V
  int chbk[TL::COPIES];                                                                    // K, per copy
#pragma unroll
  for (int c = 0; c < TL::COPIES; ++c) chbk[c] = 16 * (cp_chunk ^ swz_k<D>((w * TL::COPIES + c) * TL::ROWS_PER_COPY + cp_row));
  auto issue_tile = [&](int t, char* kst) {
    char* vst = kst + TL::BYTES;
    const int64_t k0 = (int64_t)t * kBK;
    const uint64_t remb = (uint64_t)(a.n_k - k0) * (uint64_t)ksb;
    const int nrec = (int)(uint32_t)min(remb, (uint64_t)0xFFFFFFFFu);
    const int lastb = (int)min((int64_t)(kBK - 1), a.n_k - 1 - k0) * ksb;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + k0 * a.k_ss), (short)0, nrec, kBufDword3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + k0 * a.k_ss), (short)0, nrec, kBufDword3);
#pragma unroll
    for (int c = 0; c < TL::COPIES; ++c) {
      const int q = w * TL::COPIES + c;
      const int rb = min(rowb[c], lastb);
      copy16_to_lds(rk, (lds_void*)(kst + q * 1024), (uint32_t)(rb + chbk[c]));
      copy16_to_lds(rv, (lds_void*)(vst + q * 1024), (uint32_t)(rb + chb));
    }
  };

  // V^T by 8-bit transposing reads: in each 16-lane group, lane i supplies
  // key row 8*(group/2) + i/2 (+16*c) and bytes 16*(group%2) + 8*(i%2) (+32*db)
  const int g16 = lane >> 4, i16 = lane & 15;
  const int v_row = 8 * (g16 >> 1) + (i16 >> 1);
  const int v_chunk = g16 & 1;  // + 2*db
  const int v_half = 8 * (i16 & 1);

  // S^T = K Q^T of the tile in Ks, then the keys past a row's last visible
  // key masked
  auto scores = [&](const char* Ks, int64_t k0, f32x16 (&s)[2]) {
    const int kr0 = perm_row(n);
    const int ksw = swz_k<D>(kr0);  // the same swizzle for both blocks (rows 32 apart)
    const char* krow = Ks + kr0 * TL::ROWB;
    auto kread = [&](int kk, int mb) {
      const char* base = krow + mb * 32 * TL::ROWB;
      const int c0 = 4 * kk + 2 * hh;
      const i32x4 lo = *(const lds_i32x4*)(base + 16 * (c0 ^ ksw));
      const i32x4 hi = *(const lds_i32x4*)(base + 16 * ((c0 + 1) ^ ksw));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const i32x8 k0v = kread(kk, 0), k1v = kread(kk, 1);
      s[0] = mfma_fp8(k0v, qf[kk], s[0]);
      s[1] = mfma_fp8(k1v, qf[kk], s[1]);
    }
  };
  auto mask = [&](int64_t k0, f32x16 (&s)[2]) {
    if (k0 + kBK > kfull) {  // mask per element past the keys every row sees
      const int rel = (int)max(min(lim - k0, (int64_t)kBK), (int64_t)-1) - 8 * hh;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * mb + 16 * (i >> 3) + (i & 7) > rel) s[mb][i] = -INFINITY;
    }
  };
  // moves the reference m to the tile's scaled max (qk_mul > 0: the max of
  // the raw scores times qk_mul) where that exceeds m for some row of the
  // wave, rescaling the accumulators
  auto rebase = [&](const f32x16 (&s)[2]) {
    float tmax = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[1][i]);
    tmax = half_swap_max(tmax);
    const float tx = tmax * qk_mul;
    if (__builtin_amdgcn_ballot_w64(tx > m) != 0) {
      const float m_new = fmaxf(m, tx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
  };
  auto weights = [&](const f32x16 (&s)[2], float mu, bf16x8 (&pf)[4]) {
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][i], qk_mul, -mu));
        ps[i & 3] += p;
        pf[2 * mb + (i >> 3)][i & 7] = (__bf16)p;
      }
    }
    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };

  // The first tile sets the reference m from its max.  Later tiles use the
  // reference as it stands and only check that the weights stayed finite (m
  // need not be the running max, only keep the weights in range): when a
  // lane's part of a tile sum leaves (0, 2^32] (or is not a number, as while
  // m is still -inf), the scores are computed again from the tile, still in
  // LDS, and m moves to their max.  Any reference gives the exact result;
  // the final lse uses the one actually applied.
  auto tile_step = [&](auto first, int t, const char* Ks, char* next) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile t have landed
    __syncthreads();
    const char* Vs = Ks + TL::BYTES;
    const int64_t k0 = (int64_t)t * kBK;
    f32x16 s[2];
    scores(Ks, k0, s);

    // raw V^T operands of the tile (key chunk c of 16, output rows 32*db ..),
    // read before the next tile's copies are issued
    i32x2 vraw[4][NDB];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int row = 16 * c + v_row;
        const char* p = Vs + row * TL::ROWB + 16 * ((2 * db + v_chunk) ^ swz<D>(row)) + v_half;
        vraw[c][db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
      }
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < ntiles) issue_tile(t + 1, next);

    mask(k0, s);
    bf16x8 pf[4];
    float lt;
    if constexpr (decltype(first)::value) {
      rebase(s);
      lt = weights(s, m == -INFINITY ? 0.f : m, pf);
    } else {
      lt = weights(s, m, pf);
      if (__builtin_amdgcn_ballot_w64(!(lt <= 0x1p32f)) != 0) {
        f32x16 s2[2];
        scores(Ks, k0, s2);
        mask(k0, s2);
        rebase(s2);
        lt = weights(s2, m == -INFINITY ? 0.f : m, pf);
      }
    }
    l += lt;
    // O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = mfma_bf16(fp8x8_to_bf16(vraw[c][db]), pf[c], acc[db]);
  };

  if (ntiles > 0) {
    issue_tile(0, stage0);
    tile_step(std::true_type{}, 0, stage0, stage1);
  }
  for (int t = 1; t < ntiles; t += 2) {
    tile_step(std::false_type{}, t, stage1, stage0);
    if (t + 1 < ntiles) tile_step(std::false_type{}, t + 1, stage0, stage1);
  }

  const float lt = half_swap_sum(l);
  if (!row_ok) return;
  float lse_v = -INFINITY;
  float inv = 0.f;
  if (lt > 0.f) {
    inv = a.v_scale[hk] / lt;
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
  const int64_t total = (int64_t)tiles * a.Hkv * a.B;
  if (total > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "prefill_fp8: too many work-groups per launch");
  hipLaunchKernelGGL(prefill_fp8_kernel<D>, dim3((unsigned)total), dim3(kThreads), 0, stream, a, tiles);
  return check_launch("prefill_fp8");
}

}  // namespace

attn_status launch_prefill_fp8(const PrefillArgs& a, int D, hipStream_t stream) {
  const int64_t rows = a.n_q * a.G;
  const int64_t tiles = (rows + kRowsPerWG - 1) / kRowsPerWG;
  if (tiles == 0 || a.B == 0) return ATTN_OK;
  if (tiles > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "prefill_fp8: too many query rows per launch");
  if (a.n_k > 0x7fffff00) return set_error(ATTN_E_UNSUPPORTED, "prefill_fp8: more than 2^31 - 256 keys per launch");
  return D == 128 ? launch_d<128>(a, (int)tiles, stream) : launch_d<64>(a, (int)tiles, stream);
}

}  // namespace attn
