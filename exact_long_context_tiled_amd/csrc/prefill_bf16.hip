// Tiled exact attention prefill, bf16 operands on gfx950 matrix cores.
//
// One pass over key tiles with an online softmax (a per-row reference m and
// row sum l, rescaling the fp32 output accumulator by exp(m_old - m_new) when
// m moves), the P.V product accumulated in fp32: the tiled flash-attention
// scheme of the ONNX Runtime PR #28695 analysis (section 1), laid out for
// CDNA4 waves.  m is the first tile's row max and moves only when a tile's
// weights would leave a safe range (below), not on every new maximum.
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

#include <type_traits>

#include "common.h"

namespace attn {
namespace {

constexpr int kWaves = 4;                  // 4 waves x 32 packed rows; two work-groups per CU
constexpr int kRowsPerWG = 32 * kWaves;
constexpr int kBK = 64;                    // keys per tile
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;                   // MI355X dispatches work-groups round-robin over 8 XCDs

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous 16-byte copy from a buffer to LDS: lane i reads 16 bytes at
// byte offset voff + soff of the buffer and writes them at LDS offset 16*i
// from the wave-uniform destination.  The builtin only exists in the device
// compilation pass; the host pass only needs the declaration.
constexpr int kBufDword3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format, no swizzle
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
#endif
}

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

// LDS tiles hold kBK rows of D bf16 without padding; the 16-byte chunks of a
// row are XOR-swizzled so that the matrix-core operand reads are free of
// bank conflicts:
//   K: chunk c of row r sits at c ^ (r mod chunks-per-row)
//      (16 lanes read 16 rows, one chunk each)
//   V: chunk c of row r sits at c ^ (D/32)*(r & 3)
//      (transposed reads: 4 rows x 2 chunks per 16-lane group, two groups
//      2 chunks apart)
// A tile is filled by direct global->LDS copies: lane i of a copy writes the
// 16 bytes at LDS offset 16*i, so it fetches the global chunk that belongs
// there.
template <int D>
struct Tile {
  static constexpr int ROWB = D * 2;                // bytes per row
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int BYTES = kBK * ROWB;          // one K (or V) tile
  static constexpr int STAGE = 2 * BYTES;           // K + V
  static constexpr int ROWS_PER_COPY = 64 / CPR;    // rows one wave-wide copy covers
  static constexpr int COPIES = kBK / ROWS_PER_COPY / kWaves;  // copies per wave per tile (K or V)
};

template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return r & (D / 8 - 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return (D / 32) * (r & 3);
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) prefill_bf16_kernel(PrefillArgs a, int n_row_tiles) {
  using TL = Tile<D>;
  constexpr int NKK = D / 16;  // 16-wide chunks of D for S = Q K^T
  constexpr int NDB = D / 32;  // 32-row blocks of D for O^T
  // The two stages of the K/V ring are separate arrays and the tile loop is
  // unrolled by two, so every access names its stage statically: the
  // compiler can then tell the next tile's direct-to-LDS copies from the
  // current tile's reads and does not wait for the copies before each read.
  __shared__ __attribute__((aligned(1024))) char stage0[TL::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[TL::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;

  // XCD-aware work mapping: work-group L runs on XCD L % 8; give each XCD a
  // contiguous range of (sequence, KV head, row tile) items so the K/V of one
  // (sequence, KV head) is reused from that XCD's L2.  Within a pair, the
  // row tiles that see the most keys go first.
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
  float m = -INFINITY;  // reference max of the scaled scores (log2 domain)
  float l = 0.f;        // this lane's half of the running sum

  // ---- direct global -> LDS copies of one K/V tile
  // Copy c of wave w fills rows R*(4c + w) .. +R-1 of the tile (R rows per
  // wave-wide copy).  Row r mod (chunks per row), which sets K's swizzle,
  // and r mod 4, which sets V's, do not depend on c, so each lane has one
  // byte offset for K and one for V, and the copies of a tile differ only by
  // a scalar offset.  The copies go through buffer resources whose base moves
  // with the tile (scalar registers), so the offsets are loop-invariant.
  // Rows past the block are clamped onto the last key (finite data, masked
  // below) on the one tile that reaches past it.
  const uint16_t* kbase = (const uint16_t*)a.k + b * a.k_sb + (int64_t)hk * D;
  const uint16_t* vbase = (const uint16_t*)a.v + b * a.k_sb + (int64_t)hk * D;
  const int cp_row = lane / TL::CPR;  // row within a copy
  const int cp_chunk = lane % TL::CPR;
  const int ksb = (int)a.k_ss * 2;  // bytes between key rows (< 2^26)
  const int r_w = w * TL::ROWS_PER_COPY + cp_row;  // this lane's row in copy 0
  const uint32_t koff = (uint32_t)(r_w * ksb + 16 * (cp_chunk ^ swz_k<D>(r_w)));
  const uint32_t voff = (uint32_t)(r_w * ksb + 16 * (cp_chunk ^ swz_v<D>(r_w)));
  auto issue_tile = [&](int t, char* kst) {
    char* vst = kst + TL::BYTES;
    const int64_t k0 = (int64_t)t * kBK;
    const uint64_t rem = (uint64_t)(a.n_k - k0) * (uint64_t)ksb;
    const int nrec = (int)(uint32_t)min(rem, (uint64_t)0xFFFFFFFFu);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + k0 * a.k_ss), (short)0, nrec, kBufDword3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + k0 * a.k_ss), (short)0, nrec, kBufDword3);
    // this wave's first copy within the stage; opaque, so each destination is
    // formed here by one scalar add instead of being held in a register
    int wo = w * 1024;
    asm volatile("" : "+s"(wo));
    if (k0 + kBK <= a.n_k) {
#pragma unroll
      for (int c = 0; c < TL::COPIES; ++c) {
        const int so = c * kWaves * TL::ROWS_PER_COPY * ksb;
        copy16_to_lds(rk, (lds_void*)(kst + wo + c * kWaves * 1024), koff, so);
        copy16_to_lds(rv, (lds_void*)(vst + wo + c * kWaves * 1024), voff, so);
      }
    } else {
      const int last = (int)(a.n_k - 1 - k0);
#pragma unroll
      for (int c = 0; c < TL::COPIES; ++c) {
        const int rr = (kWaves * c + w) * TL::ROWS_PER_COPY + cp_row;
        const int j = min(rr, last);
        copy16_to_lds(rk, (lds_void*)(kst + wo + c * kWaves * 1024), (uint32_t)(j * ksb + 16 * (cp_chunk ^ swz_k<D>(rr))), 0);
        copy16_to_lds(rv, (lds_void*)(vst + wo + c * kWaves * 1024), (uint32_t)(j * ksb + 16 * (cp_chunk ^ swz_v<D>(rr))), 0);
      }
    }
  };

  // V^T by transposed reads: lane (a=r16/4, b=r16%4) of each 16-lane group
  // addresses key row 8*(lane/32) + a (+4), columns 16*(g16%2) + 4*b
  // (+ 32*db).  Rows 16c + v_row (+4) share v_row's swizzle, so the byte
  // offset of block db from the stage is vofs[db] + 16c*ROWB (+ 4*ROWB).
  // The offsets are opaque, so the reads keep their stage's alias scope.
  const int g16 = lane >> 4, r16 = lane & 15;
  const int v_row = 8 * (g16 >> 1) + (r16 >> 2);
  const int v_col = 16 * (g16 & 1) + 4 * (r16 & 3);
  int vofs[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int col = 32 * db + v_col;
    vofs[db] = TL::BYTES + v_row * TL::ROWB + 16 * ((col >> 3) ^ swz_v<D>(v_row)) + 2 * (col & 7);
    asm volatile("" : "+v"(vofs[db]));
  }

  // S^T = K Q^T of the tile in Ks, operands software-pipelined: the K chunks
  // of step kk+1 are read from LDS while the two (independent) products of
  // step kk run; then the keys past a row's last visible key are masked
  auto scores = [&](const char* Ks, int64_t k0, f32x16 (&s)[2]) {
    const int kr0 = perm_row(n);  // K row of this lane in block mb: 32*mb + kr0
    const int ksw = swz_k<D>(kr0);  // the same swizzle for both blocks (32 = 0 mod 16)
    const char* krow = Ks + kr0 * TL::ROWB;
    auto kread = [&](int kk, int mb) {
      return *(const lds_bf16x8*)(krow + mb * 32 * TL::ROWB + 16 * ((2 * kk + hh) ^ ksw));
    };
    s[0] = f32x16{};
    s[1] = f32x16{};
    bf16x8 kc0 = kread(0, 0), kc1 = kread(0, 1);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 kn0, kn1;
      if (kk + 1 < NKK) {
        kn0 = kread(kk + 1, 0);
        kn1 = kread(kk + 1, 1);
      }
      // (keeps the next reads above these products: sunk below them, the
      // reads would share registers with the current operands and serialise)
      __builtin_amdgcn_sched_barrier(0);
      s[0] = mfma32(kc0, qf[kk], s[0]);
      s[1] = mfma32(kc1, qf[kk], s[1]);
      if (kk + 1 < NKK) {
        kc0 = kn0;
        kc1 = kn1;
      }
    }
  };
  auto mask = [&](int64_t k0, f32x16 (&s)[2]) {
    if (k0 + kBK > kfull) {  // tile reaches past the keys every row sees: mask per element
      // last visible key in the tile, relative to this lane's first key (8*hh)
      const int rel = (int)max(min(lim - k0, (int64_t)kBK), (int64_t)-1) - 8 * hh;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * mb + 16 * (i >> 3) + (i & 7) > rel) s[mb][i] = -INFINITY;
    }
  };
  // moves the reference m to the tile's scaled max when that exceeds m + thr
  // (log2 units) for some row of the wave, rescaling the accumulators
  auto rebase = [&](const f32x16 (&s)[2], float thr) {
    float tmax = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) tmax = fmaxf(fmaxf(tmax, s[0][i]), s[0][i + 1]);
    tmax = fmaxf(fmaxf(tmax, s[0][15]), s[1][0]);
#pragma unroll
    for (int i = 1; i < 15; i += 2) tmax = fmaxf(fmaxf(tmax, s[1][i]), s[1][i + 1]);
    tmax = fmaxf(tmax, s[1][15]);
    tmax = half_swap_max(tmax);
    const float tx = tmax * a.scale_log2;
    if (__builtin_amdgcn_ballot_w64(tx > m + thr) != 0) {
      const float m_new = fmaxf(m, tx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
  };
  // weights against the reference mu: bf16 copies and this lane's sum
  auto weights = [&](const f32x16 (&s)[2], float mu, bf16x8 (&pf)[4]) {
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][i], a.scale_log2, -mu));
        ps[i & 3] += p;
        pf[2 * mb + (i >> 3)][i & 7] = (__bf16)p;
      }
    }
    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };

  // FIRST: the first tile sets the reference from its max.  Later tiles use
  // the reference as it stands and only check that the weights stayed
  // finite: m need not be the running max, only keep the weights in range,
  // so it moves only when a lane's part of a tile sum leaves (0, 2^32] (or
  // is not a number: also when m is still -inf).  Then the scores are
  // computed again from the tile, still in LDS, and the reference moved to
  // their max.  Any reference gives the exact result; the final lse uses the
  // one actually applied.
  auto tile_step = [&](auto first, int t, const char* Ks, char* next) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile t have landed
    __syncthreads();                     // ... everyone's; and tile t-1 is fully consumed
    const int64_t k0 = (int64_t)t * kBK;
    f32x16 s[2];
    scores(Ks, k0, s);

    // V^T operand (key chunk c of 16, output rows 32*db ..) by two transposing reads
    auto vread = [&](int c, int db) {
      const int o0 = vofs[db] + 16 * c * TL::ROWB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Ks + o0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Ks + o0 + 4 * TL::ROWB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // all V^T operands of the tile, read before the next tile's copies are
    // issued: a transposing LDS read issued while direct-to-LDS copies are in
    // flight makes the compiler wait for those copies first
    bf16x8 vt[4][NDB];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) vt[c][db] = vread(c, db);
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < ntiles) issue_tile(t + 1, next);

    mask(k0, s);
    bf16x8 pf[4];
    float lt;
    if constexpr (decltype(first)::value) {
      rebase(s, 0.f);
      lt = weights(s, m == -INFINITY ? 0.f : m, pf);
    } else {
      lt = weights(s, m, pf);
      if (__builtin_amdgcn_ballot_w64(!(lt <= 0x1p32f)) != 0) {
        // (the V operands are read again afterwards, so they need no
        // registers while the scores are recomputed)
        f32x16 s2[2];
        scores(Ks, k0, s2);
        mask(k0, s2);
        rebase(s2, 0.f);
        lt = weights(s2, m == -INFINITY ? 0.f : m, pf);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int db = 0; db < NDB; ++db) vt[c][db] = vread(c, db);
      }
    }
    l += lt;
    // O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = mfma32(vt[c][db], pf[c], acc[db]);
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
  const int64_t total = (int64_t)tiles * a.Hkv * a.B;
  if (total > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "prefill: too many work-groups per launch");
  hipLaunchKernelGGL(prefill_bf16_kernel<D>, dim3((unsigned)total), dim3(kThreads), 0, stream, a, tiles);
  return check_launch("prefill_bf16");
}

}  // namespace

attn_status launch_prefill_bf16(const PrefillArgs& a, int D, hipStream_t stream) {
  const int64_t rows = a.n_q * a.G;
  const int64_t tiles = (rows + kRowsPerWG - 1) / kRowsPerWG;
  if (tiles == 0 || a.B == 0) return ATTN_OK;
  if (tiles > 0x7fffffff) return set_error(ATTN_E_UNSUPPORTED, "prefill: too many query rows per launch");
  if (a.n_k > 0x7fffff00) return set_error(ATTN_E_UNSUPPORTED, "prefill: more than 2^31 - 256 keys per launch");
  return D == 128 ? launch_d<128>(a, (int)tiles, stream) : launch_d<64>(a, (int)tiles, stream);
}

}  // namespace attn
