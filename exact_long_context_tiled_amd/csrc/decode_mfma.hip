// Split-KV decode on the matrix cores (bf16, e4m3, int8 and, for D = 128,
// int4 caches).
//
// The work split, the partial records and the log-sum-exp merge are those of
// the vector-ALU kernel in decode.hip (flash decoding: ONNX Runtime PR #28695
// analysis, section 2; pages: LLM-CoOpt "Methodology" item 3; quantised
// caches dequantised on the fly: LLM-CoOpt "Methodology" item 1 and the
// ONNX Runtime analysis, section 1).  Only the scan of a piece differs: the
// query rows of a KV head (n_q * G of them, up to 16 per pass) form the
// n = 16 side of v_mfma_f32_16x16x32_bf16 products, so the per-token work
// moves from the vector ALUs to the matrix cores:
//
//   S^T = K Q^T   (16 tokens x 16 rows per product).  K comes straight from
//                 HBM into the A operand: a lane quarter j holds D/4
//                 contiguous dims of a token row (one to four 16-byte loads),
//                 Q the same dims of its row.  The 16 tokens of sub-block sb
//                 of a 32-token block are taken in the order
//                 8*(i/4) + 4*sb + i%4 (i = A row), which makes the
//                 accumulator of lane quarter j hold tokens 8j .. 8j+7 of the
//                 block: the B operand of the next product as it stands.
//   O^T += V^T P^T (16 dims x 16 rows, 32 tokens per product).  V goes
//                 through LDS (direct global -> LDS copies into per-wave
//                 tiles, two or three stages) and comes back transposed: two
//                 16-bit transposing reads (4 tokens each) for bf16, one
//                 8-bit read (8 tokens) for e4m3 / int8 / int4.
//
// e4m3 and int8 codes become exact bf16 numbers; P is rounded to bf16 as in
// the prefill kernels.  int8 scales (per token) multiply the fp32 scores and
// the softmax weights; e4m3 scales (per KV head) join scale*log2(e) and the
// output factor.  int4 (32-element scale groups, D = 128) needs no
// arithmetic per element: each code enters as the exact bf16 n + 136 (bit
// masks), a transpose across lane quarters makes every k-step of S^T one
// scale group (so a token's score is the sum of its group scales times the
// group products), the V scales go into group-scaled copies of P, and
// products with a constant -136 operand remove the offset.
//
// int8 and int4 scales of a block go through LDS with the V tile: one
// wave-wide copy per block (4 bytes per lane for int8's per-token scales, 16
// for int4's group scales), read back by each lane quarter for its 8 tokens.
// Loaded per lane instead, every lane of a quarter would fetch the same
// scales (16 extra loads per block for int4) and hold them in registers for
// every pipeline stage.
//
// Each of the 4 waves of a work-group scans every 4th 32-token block of a
// piece with its own online softmax (a per-row reference m that moves only
// when a block's weights would leave a safe range, as in the prefill
// kernels); blocks load one (bf16) or two (smaller tiles) ahead of the one
// consumed.  The waves are then combined through LDS and the piece's record
// (or the final output) written.
#include <math.h>
#include <stdlib.h>

#include <algorithm>

#include "common.h"
#include "decode_common.h"

namespace attn {
namespace {

using dec::clamp_len;
using dec::group_prefix;
using dec::lane_pair;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlk = 32;   // tokens per wave iteration
constexpr int kRows = 16;  // query rows per pass (the products' n)

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

__device__ __forceinline__ void copy4_to_lds(const void* src, lds_void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
#endif
}
__device__ __forceinline__ void copy16_to_lds(const void* src, lds_void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
#endif
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bytes of a D-element row
template <int KV>
constexpr int row_bytes(int D) {
  return KV == ATTN_BF16 ? 2 * D : KV == ATTN_INT4 ? D / 2 : D;
}

// Eight 8-bit codes (two words, element order) -> eight exact bf16 values.
template <int KV>
__device__ __forceinline__ bf16x8 codes8_to_bf16(uint32_t w0, uint32_t w1) {
  if constexpr (KV == ATTN_FP8_E4M3) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    // int8 -> fp32 (exact), whose upper half is the exact bf16
    const uint32_t w[2] = {w0, w1};
    uint32_t pk[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t src = w[h >> 1];
      const int sh = 16 * (h & 1);
      const float f0 = (float)(int)(int8_t)(src >> sh);
      const float f1 = (float)(int)(int8_t)(src >> (sh + 8));
      pk[h] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    }
    return __builtin_bit_cast(bf16x8, uint4{pk[0], pk[1], pk[2], pk[3]});
  }
}

// int4 codes as exact bf16 integers without arithmetic per element: for a
// 4-bit two's-complement code n, v = code ^ 8 = n + 8 lies in [0, 15], and the
// bf16 bit pattern 0x4300 | v is the value 128 + v = n + 136 (exponent 2^7,
// v in the low mantissa bits).  The offset 136 is taken off afterwards by a
// product with the constant operand kNeg136 below.
constexpr uint16_t kBf16Neg136 = 0xC308u;

// Codes e and e + 4 of x >> sh (bits sh .. sh+3 and sh+16 .. sh+19) as the
// bf16 pair n + 136.  One three-input bit operation per word: where
// kNibBits is set the result is the code bit XOR kNibSet (which flips bit 3
// of each code: code ^ 8 = n + 8), elsewhere it is kNibSet (the 0x4300
// exponent pattern).  The truth table 0x6A is f(a, b, c) = b ? a ^ c : c
// evaluated on the operand masks a = 0xF0, b = 0xCC, c = 0xAA.
constexpr uint32_t kNibBits = 0x000F000Fu;
constexpr uint32_t kNibSet = 0x43084308u;
__device__ __forceinline__ uint32_t nib_pair(uint32_t x, int sh) {
  return __builtin_amdgcn_bitop3_b32(x >> sh, kNibBits, kNibSet, 0x6A);
}

// The 8 codes of w (code e at bits 4e .. 4e+3), as n + 136, in the element
// order 0, 4, 1, 5, 2, 6, 3, 7 (nib_pair of a shift takes codes e and e + 4).
__device__ __forceinline__ bf16x8 nib8_strided(uint32_t w) {
  return __builtin_bit_cast(bf16x8, uint4{nib_pair(w, 0), nib_pair(w, 4), nib_pair(w, 8), nib_pair(w, 12)});
}

// 4x4 transpose of dwords across the lane quarters: lane (j, i) holds d[c]
// of quarter j on entry and quarter c's d[j] on exit (permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second; permlane16_swap the odd 16-lane rows of the first with the even
// rows of the second).
__device__ __forceinline__ void quarter_transpose(uint32_t (&d)[4]) {
  {
    const auto r = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
    d[0] = r[0];
    d[2] = r[1];
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
    d[1] = r[0];
    d[3] = r[1];
  }
  {
    const auto r = __builtin_amdgcn_permlane16_swap(d[0], d[1], false, false);
    d[0] = r[0];
    d[1] = r[1];
  }
  {
    const auto r = __builtin_amdgcn_permlane16_swap(d[2], d[3], false, false);
    d[2] = r[0];
    d[3] = r[1];
  }
}

template <int KV, int D>
struct MTile {
  static constexpr int ROWB = row_bytes<KV>(D);       // bytes per token row
  static constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
  static constexpr int BYTES = kBlk * ROWB;           // one wave's V tile
  static constexpr int COPIES = BYTES / 1024;         // wave-wide 1 KiB copies per tile
  static constexpr int QD = D / 4;                    // dims per lane quarter (QK operands)
  static constexpr int QB = row_bytes<KV>(QD);        // K bytes per token per lane quarter
  static constexpr int KL = QB / 16;                  // 16-byte K loads per token per lane
  static constexpr int NKS = D / 32;                  // k-steps of the QK product
  static constexpr int NDB = D / 16;                  // 16-dim blocks of the PV product
  // V-tile stages per wave: with small tiles (8-bit and 4-bit caches) two
  // blocks' loads are kept in flight behind the one being consumed
  static constexpr int STAGES = BYTES <= 4096 ? 3 : 2;
  // vector-memory operations of one block's loads (the fewest of their forms:
  // K operands, scales, V copies)
  static constexpr int OPS = 2 * KL + COPIES + (KV == ATTN_INT8 || KV == ATTN_INT4 ? 1 : 0);
  // a wave's K and V scales of one block, staged in LDS after the V tiles of
  // the stage: int8 one per token (32 x 2 floats), int4 one per 32-element
  // group (32 x 4 x 2 floats)
  static constexpr int SCB = KV == ATTN_INT4 ? 1024 : KV == ATTN_INT8 ? 256 : 0;
  static constexpr int STAGE = kWaves * (BYTES + SCB);
  // wave partials of the combine (dynamic LDS, before the length prefix)
  static constexpr int RED = ((kWaves * kRows * D + 2 * kWaves * kRows) * 4 + 255) / 256 * 256;
};

// V tile swizzle (16-byte chunk c of row r sits at c ^ swz(r)), chosen so the
// transposing reads of a 16-lane group touch distinct banks.
template <int KV, int D>
__device__ __forceinline__ int swz_v(int r) {
  using TL = MTile<KV, D>;
  if constexpr (KV == ATTN_BF16) return (2 * (r & 3)) & (TL::CPR - 1);
  else return r & (TL::CPR - 1);
}

template <int KV, int D>
__global__ void __launch_bounds__(kThreads) decode_mfma_kernel(DecodeArgs a) {
  using TL = MTile<KV, D>;
  static_assert(KV != ATTN_INT4 || D == 128, "int4: one 32-element scale group per lane quarter");
  // V-tile stages, one array each (so the compiler tells copies into one
  // stage from reads of another), [waves][BYTES]
  __shared__ __attribute__((aligned(1024))) char vst0[TL::STAGE];
  __shared__ __attribute__((aligned(1024))) char vst1[TL::STAGE];
  __shared__ __attribute__((aligned(16))) char vst2[TL::STAGES == 3 ? TL::STAGE : 16];  // (unused with two stages)
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int64_t* pre = (int64_t*)(smem + TL::RED);               // [B + 1]
  int* lens_s = (int*)(pre + a.B + 1);                     // [B] clamped lengths
  __shared__ int64_t wsum[kWaves];
  __shared__ int red_bad[kWaves];  // per wave: a page-table entry outside the cache was met
  __shared__ int merge_first, merge_n;  // fused merge: first record and record count, or -1
  // wave partials for the combine
  float* red_acc = (float*)smem;                           // [waves][kRows][D]
  float* red_m = red_acc + kWaves * kRows * D;             // [waves][kRows]
  float* red_l = red_m + kWaves * kRows;                   // [waves][kRows]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane >> 4, i = lane & 15;  // lane quarter, lane in quarter
  const uint8_t* kb = (const uint8_t*)a.k;
  const uint8_t* vb = (const uint8_t*)a.v;
  // This lane's transposed V reads: byte offsets from a stage array, one per
  // read group (16-dim block, or 32-dim int4 group).  Made opaque to the
  // optimiser: every read address is then the stage array plus one register
  // plus an immediate, which keeps the array's alias scope on the read (a
  // deeper chain of address arithmetic loses it, and the wait counters would
  // then hold the read until every copy in flight had landed).
  constexpr int NVR = KV == ATTN_INT4 ? TL::CPR : TL::NDB;
  int vro[NVR];
#pragma unroll
  for (int x = 0; x < NVR; ++x) {
    if constexpr (KV == ATTN_BF16) {
      const int col = 32 * x + 8 * (i & 3);  // byte within the row
      const int r_lo = 8 * j + (i >> 2);
      vro[x] = w * TL::BYTES + r_lo * TL::ROWB + 16 * ((col >> 4) ^ swz_v<KV, D>(r_lo)) + (col & 15);
    } else {
      const int rrow = 8 * j + (i >> 1);
      vro[x] = w * TL::BYTES + rrow * TL::ROWB + 16 * (x ^ swz_v<KV, D>(rrow)) + 8 * (i & 1);
    }
    asm volatile("" : "+v"(vro[x]));
  }
  // this lane quarter's scales (tokens 8j .. 8j+7) in the wave's scale tile
  // of a stage (opaque, like the V offsets)
  int sro = kWaves * TL::BYTES + w * TL::SCB + TL::SCB / 8 * j;
  asm volatile("" : "+v"(sro));

  // The split: segment (b, hk) occupies piece_groups charged slots followed
  // by its 16-token groups; all segments laid end to end (W slots) are cut
  // into N equal runs [floor(u W / N), floor((u + 1) W / N)).
  group_prefix<kThreads>(a.kv_lens, a.B, a.max_kv_len, a.piece_groups, pre, wsum, lens_s);
  const int64_t W = pre[a.B] * a.Hkv;
  const int64_t N = a.n_units < W ? (int64_t)a.n_units : W;
  const int unit = blockIdx.x;
  // empty sequences: O = 0, lse = -inf (every launched work-group takes some)
  for (int bb = unit; bb < a.B; bb += (int)gridDim.x) {
    if (lens_s[bb] != 0) continue;
    const int per_b = a.n_q * a.Hq;
    for (int idx = tid; idx < per_b * D; idx += kThreads) a.o[(int64_t)bb * per_b * D + idx] = 0.f;
    if (a.lse)
      for (int idx = tid; idx < per_b; idx += kThreads) a.lse[(int64_t)bb * per_b + idx] = -INFINITY;
  }
  if (unit >= N) return;
  // W = qd N + rw, so floor(u W / N) = u qd + floor(u rw / N), the last term
  // in 32 bits (u, rw < N <= 65535)
  const int64_t qd = W / N;
  const uint32_t rw = (uint32_t)(W - qd * N);
  const int64_t x0 = (int64_t)unit * qd + (int64_t)((uint32_t)unit * rw / (uint32_t)N);
  const int64_t x1 = (int64_t)(unit + 1) * qd + (int64_t)((uint32_t)(unit + 1) * rw / (uint32_t)N);
  const int G = a.G;
  const int n_q = a.n_q;
  const int RT = n_q * G;
  const int REC = decode_record_floats(RT, D);
  // int8 scale arrays whose base is 16-byte aligned can be read 8 tokens at a time
  const bool scales16 = (((uintptr_t)a.k_scale | (uintptr_t)a.v_scale) & 15) == 0;

  for (int64_t pos = x0; pos < x1;) {
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] * a.Hkv <= pos) lo = mid;
      else hi = mid - 1;
    }
    const int b = __builtin_amdgcn_readfirstlane(lo);
    const int64_t sbase = pre[b] * a.Hkv;
    const int ns = (int)(pre[b + 1] - pre[b]);  // slots of one segment of b (> 0: b holds pos)
    const int64_t off = pos - sbase;
    const int hk = __builtin_amdgcn_readfirstlane(off <= 0x7fffffff ? (int)((uint32_t)off / (uint32_t)ns)
                                                                      : (int)(off / ns));
    const int64_t sstart = sbase + (int64_t)hk * ns;
    const int64_t seg_end = sstart + ns;
    const int64_t pend = seg_end < x1 ? seg_end : x1;
    const int64_t gstart = sstart + a.piece_groups;  // the segment's first group
    if (pend <= gstart) {  // the run holds only charged slots of this segment
      pos = pend;
      continue;
    }
    const int64_t pg = pos > gstart ? pos : gstart;
    const int j0 = (int)(pg - gstart);
    const int T = lens_s[b];
    const int t0 = __builtin_amdgcn_readfirstlane(j0 * kDecodeGroup);
    const int t1 = __builtin_amdgcn_readfirstlane(min(T, (j0 + (int)(pend - pg)) * kDecodeGroup));
    const int seg = b * a.Hkv + hk;
    const bool whole = j0 == 0 && pend == seg_end;
    float smul = a.scale_log2;
    if constexpr (KV == ATTN_FP8_E4M3) smul *= a.k_scale[hk];
    const int64_t hk_rows = (int64_t)hk * a.page_size;
    float* rec = a.part + (int64_t)(unit + seg) * REC;
    // A split segment's counter word is brought to this call's tag with a
    // count of zero as the launch starts, by each unit whose run begins in
    // the segment (every split segment has one: all its units but the
    // first).  A device-scope max leaves a word that already carries this
    // call's tag, and any count in it, as it is, and nothing waits for it;
    // the units finishing later then count themselves in with one add.  (A
    // unit's later pieces do not open their segment: under full load the
    // atomic's latency held up their first blocks.)
    if (!whole && pos == x0 && tid == 0)
      __hip_atomic_fetch_max((uint64_t*)a.seg_info + seg, a.tag << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    bool bad_page = false;  // a page-table entry of this piece lay outside the cache
    for (int r0 = 0; r0 < RT; r0 += kRows) {
      const int n_rows = min(kRows, RT - r0);
      // this lane's row (clamped onto the pass's last row when past it: computed, not written)
      const int r = r0 + min(i, n_rows - 1);
      const int sq = r / G, g = r - (r / G) * G;
      // query token sq sits at T - n_q + sq and sees the keys before T - (n_q - 1 - sq)
      const int lim = max(t0, min(t1, T - (n_q - 1 - sq)));
      const int tend = __builtin_amdgcn_readfirstlane(
          max(t0, min(t1, T - (n_q - 1 - (r0 + n_rows - 1) / G))));  // past the last key any row reads

      // Q operand: dims QD*j .. of the lane's row; for int4, step ks takes
      // dims 32ks + 8j .. 32ks + 8j + 7 (scale group ks) in the element order
      // of nib8_strided, and qoff[ks] = -136 x (the row's sum over group ks)
      bf16x8 qf[TL::NKS];
      f32x4 qoff[KV == ATTN_INT4 ? TL::NKS : 1];
      {
        const uint16_t* qrow = (const uint16_t*)a.q + (((int64_t)b * n_q + sq) * a.Hq + (int64_t)hk * G + g) * D;
        if constexpr (KV == ATTN_INT4) {
          const uint16_t c = kBf16Neg136;
          const bf16x8 neg136 = __builtin_bit_cast(bf16x8, uint4{c * 0x10001u, c * 0x10001u, c * 0x10001u, c * 0x10001u});
#pragma unroll
          for (int ks = 0; ks < TL::NKS; ++ks) {
            const bf16x8 raw = *(const bf16x8*)(qrow + 32 * ks + 8 * j);
            qf[ks] = __builtin_shufflevector(raw, raw, 0, 4, 1, 5, 2, 6, 3, 7);
            qoff[ks] = mfma16(neg136, qf[ks], f32x4{0.f, 0.f, 0.f, 0.f});
          }
        } else {
          const bf16x8* qp = (const bf16x8*)(qrow + TL::QD * j);
#pragma unroll
          for (int ks = 0; ks < TL::NKS; ++ks) qf[ks] = qp[ks];
        }
      }
      f32x4 acc[TL::NDB];
      // int4: the -136 offset's share of group c's output, the same for its
      // even and odd dims, added to both once the piece is scanned
      f32x4 corr[KV == ATTN_INT4 ? TL::CPR : 1];
#pragma unroll
      for (int c = 0; c < (KV == ATTN_INT4 ? TL::CPR : 1); ++c) corr[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < TL::NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      float m = -INFINITY, l = 0.f;

      // cache row (token row index) of token t < tend of this segment
      auto page_row = [&](int t16) {  // first row of the 16-token group holding token t16 (wave-uniform)
        if (a.page_table) {
          const auto* pt = (const __attribute__((address_space(4))) int32_t*)a.page_table;
          const int pe = pt[(int64_t)b * a.max_pages + (t16 >> a.page_shift)];
          // an entry outside the cache is never dereferenced: page 0 is read
          // instead and the rows of the piece are written as NaN
          const bool ok = (uint32_t)pe < (uint32_t)a.num_pages;
          bad_page |= !ok;
          const int pg = ok ? pe : 0;
          return (int64_t)pg * a.Hkv * a.page_size + hk_rows - (t16 & ~(a.page_size - 1));
        }
        return (int64_t)b * a.Hkv * a.page_size + hk_rows;
      };
      struct Kbuf {
        uint4 k[2][TL::KL];
      };
      // Block addresses.  A 32-token block starts on a 16-token group, so
      // each of its halves lies within one page: the block's two half bases
      // are wave-uniform (scalar), and each lane adds an offset of its own.
      // The K loads of lanes i >= 8 lie in the second half; V copy c lies in
      // half c / (COPIES / 2).  Tokens past the piece are clamped onto its
      // last token (cached, valid data, never weighed); on the last block a
      // clamped token of the second half lies in the first half's group, and
      // then both half bases are that group's.  The clamp is branch-free, so
      // every block issues the same instructions (a branch around the loads
      // would make the compiler drain the loads in flight at every step).
      const bool k_hi = i >= 8;
      int ktok[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) ktok[sb] = 8 * (i >> 2) + 4 * sb + (i & 3);
      constexpr int kRowsPerCopy = 1024 / TL::ROWB;
      const int v_rr0 = 16 * lane / TL::ROWB;
      const uint32_t vcol = (uint32_t)(16 * (((16 * lane) % TL::ROWB / 16) ^ swz_v<KV, D>(v_rr0)));
      // loads of the block starting at token g0: K operands to registers, V
      // tile (and int8 / int4 scales) to LDS
      auto issue = [&](int g0, Kbuf& kbf, char* st) {
        char* vt = st + w * TL::BYTES;
        const int tl = tend - 1;
        // A block wholly past the piece (issued ahead, never consumed) is
        // moved onto its last token, so every in-block offset stays >= 0.
        const int gb = min(g0, tl);
        const int lim = tl - gb;  // the last in-block token that is loaded as itself
        const int64_t row0 = page_row(__builtin_amdgcn_readfirstlane(gb)) + gb;
        const int64_t row1 = page_row(__builtin_amdgcn_readfirstlane(min(g0 + 16, tl))) + gb;
        const uint8_t* kp = k_hi ? kb + row1 * TL::ROWB : kb + row0 * TL::ROWB;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const uint4* src = (const uint4*)(kp + (uint32_t)(min(ktok[sb], lim) * TL::ROWB + TL::QB * j));
#pragma unroll
          for (int u = 0; u < TL::KL; ++u) kbf.k[sb][u] = src[u];
        }
        if constexpr (KV == ATTN_INT4) {
          // K and V scales [row][4 groups] of the block's 32 tokens into the
          // wave's scale tile: K scales of token t at 16 t, V scales at
          // 512 + 16 t.  One 16-byte copy per lane (lane L: token L % 32, K
          // for L < 32), or four 4-byte copies when the scale arrays are not
          // 16-byte aligned.
          char* sct = st + kWaves * TL::BYTES + w * TL::SCB;
          if (scales16) {
            const int ts = lane & 31;
            const float* arr = lane < 32 ? a.k_scale : a.v_scale;
            copy16_to_lds(arr + ((ts >= 16 ? row1 : row0) + min(ts, lim)) * 4, (lds_void*)sct);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int o = 256 * q + 4 * lane;  // byte of the scale tile
              const int ts = (o & 511) >> 4;
              const float* arr = o < 512 ? a.k_scale : a.v_scale;
              copy4_to_lds(arr + ((ts >= 16 ? row1 : row0) + min(ts, lim)) * 4 + ((o & 15) >> 2), (lds_void*)(sct + 256 * q));
            }
          }
        }
        if constexpr (KV == ATTN_INT8) {
          // K and V scales of the block's 32 tokens into the wave's scale
          // tile (K scale of token t at 4 t, V scale at 128 + 4 t): one
          // 4-byte copy per lane (lane L: token L % 32, K for L < 32)
          char* sct = st + kWaves * TL::BYTES + w * TL::SCB;
          const int ts = lane & 31;
          const float* arr = lane < 32 ? a.k_scale : a.v_scale;
          copy4_to_lds(arr + (ts >= 16 ? row1 : row0) + min(ts, lim), (lds_void*)sct);
        }
#pragma unroll
        for (int c = 0; c < TL::COPIES; ++c) {
          const uint8_t* vp = vb + (c < TL::COPIES / 2 ? row0 : row1) * TL::ROWB;
          const int rr = min(c * kRowsPerCopy + v_rr0, lim);
          copy16_to_lds(vp + (uint32_t)(rr * TL::ROWB + vcol), (lds_void*)(vt + c * 1024));
        }
      };
      // V^T operands of a block: lane (j, i) holds dim 16*db + i of tokens 8j .. 8j+7
      struct Vops {
        bf16x8 v[TL::NDB];
        i32x2 raw4[TL::CPR];  // int4: 8 tokens x byte i of each 16-byte chunk (= 32-dim group)
        f32x4 ks4[KV == ATTN_INT4 ? 8 : 1];  // int4: K scales of tokens 8j + e, all 4 groups
        f32x4 vs4[KV == ATTN_INT4 ? 8 : 1];  // int4: V scales of tokens 8j + e, all 4 groups
        f32x4 ks[2], vs[2];                  // int8: scales of tokens 8j .. 8j+7
      };
      auto vread = [&](char* st, Vops& vo) {
        bf16x8* vop = vo.v;
        if constexpr (KV == ATTN_INT4) {
#pragma unroll
          for (int c = 0; c < TL::CPR; ++c) vo.raw4[c] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(st + vro[c]));
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            vo.ks4[e] = *(const lds_f32x4*)(st + sro + 16 * e);
            vo.vs4[e] = *(const lds_f32x4*)(st + sro + 512 + 16 * e);
          }
        } else if constexpr (KV == ATTN_BF16) {
#pragma unroll
          for (int db = 0; db < TL::NDB; ++db) {
            const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + vro[db]));
            const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + vro[db] + 4 * TL::ROWB));
            vop[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        } else {
          if constexpr (KV == ATTN_INT8) {
            vo.ks[0] = *(const lds_f32x4*)(st + sro);
            vo.ks[1] = *(const lds_f32x4*)(st + sro + 16);
            vo.vs[0] = *(const lds_f32x4*)(st + sro + 128);
            vo.vs[1] = *(const lds_f32x4*)(st + sro + 144);
          }
          i32x2 raw[TL::NDB];
#pragma unroll
          for (int db = 0; db < TL::NDB; ++db) raw[db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(st + vro[db]));
#pragma unroll
          for (int db = 0; db < TL::NDB; ++db) vop[db] = codes8_to_bf16<KV>((uint32_t)raw[db][0], (uint32_t)raw[db][1]);
        }
      };
      auto consume = [&](int g0, const Kbuf& kbf, const Vops& vo) {
        const bf16x8* vop = vo.v;
        // S^T = K Q^T for the two 16-token sub-blocks
        // scores of tokens 8j + e of the block (e = 4*sb + register), this lane's row
        float sc[8];
        if constexpr (KV == ATTN_INT4) {
          // One product per scale group: after the transpose, dword ks of the
          // lane's 16 bytes holds dims 32ks + 8j .. of its token (group ks),
          // and the product starts from qoff[ks], which takes the 136 offset
          // of the codes off.  A token's score is then the sum over groups of
          // its group scale times the group's product.
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            const uint4 wv = kbf.k[sb][0];
            uint32_t d[4] = {wv.x, wv.y, wv.z, wv.w};
            quarter_transpose(d);
            f32x4 sg[TL::NKS];
#pragma unroll
            for (int ks = 0; ks < TL::NKS; ++ks) sg[ks] = mfma16(nib8_strided(d[ks]), qf[ks], qoff[ks]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const f32x4 k4 = vo.ks4[4 * sb + r];
              sc[4 * sb + r] = k4[0] * sg[0][r] + k4[1] * sg[1][r] + k4[2] * sg[2][r] + k4[3] * sg[3][r];
            }
          }
        } else {
          f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int ks = 0; ks < TL::NKS; ++ks) {
              bf16x8 kop;
              if constexpr (KV == ATTN_BF16) {
                kop = __builtin_bit_cast(bf16x8, kbf.k[sb][ks]);
              } else {
                const uint4 wv = kbf.k[sb][ks >> 1];
                kop = (ks & 1) ? codes8_to_bf16<KV>(wv.z, wv.w) : codes8_to_bf16<KV>(wv.x, wv.y);
              }
              s[sb] = mfma16(kop, qf[ks], s[sb]);
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[e] = s[e >> 2][e & 3];
        }
        float vsc[8];
        if constexpr (KV == ATTN_INT8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            sc[e] *= vo.ks[e >> 2][e & 3];
            vsc[e] = vo.vs[e >> 2][e & 3];
          }
        }
        if (g0 + kBlk > lim) {  // keys past this row's limit weigh nothing
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[e] = g0 + 8 * j + e < lim ? sc[e] : -INFINITY;
        }
        // The weights against the reference m as it stands.  Any m gives the
        // exact result while the weights stay finite (the lse uses the m
        // applied), so m moves only when a lane's weights would pass 2^32,
        // or while it is still -inf (the weights are then inf or NaN): then
        // it becomes the block's row max and the weights are taken again.
        float pv[8];
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], smul, -m));
          ls += pv[e];
        }
        if (__builtin_amdgcn_ballot_w64(!(ls <= 0x1p32f)) != 0) {
          float mx = sc[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
          {
            float u0, u1;
            lane_pair<16>(mx, u0, u1);
            mx = fmaxf(u0, u1);
            lane_pair<32>(mx, u0, u1);
            mx = fmaxf(u0, u1);
          }
          const float m_new = fmaxf(m, mx * smul);
          const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
          m = m_new;
          l *= alpha;
#pragma unroll
          for (int db = 0; db < TL::NDB; ++db) acc[db] *= alpha;
          if constexpr (KV == ATTN_INT4) {
#pragma unroll
            for (int c = 0; c < TL::CPR; ++c) corr[c] *= alpha;
          }
          const float m_use = m == -INFINITY ? 0.f : m;
          ls = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], smul, -m_use));
            ls += pv[e];
          }
        }
        // the weights as a bf16 pair hi + lo (lo = the rounding residue of
        // hi): two P.V products carry them to ~2^-17 relative, where bf16
        // alone would err by 2^-9 of each weight times |v|.  The scan is
        // bound by HBM, so the second product is free.
        bf16x8 pf, plo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float p = pv[e];
          if constexpr (KV == ATTN_INT8) p = sc[e] == -INFINITY ? 0.f : p * vsc[e];
          pf[e] = (__bf16)p;
          plo[e] = (__bf16)(p - (float)pf[e]);
        }
        l += ls;
        // O^T += V^T P^T
        if constexpr (KV == ATTN_INT4) {
          // Group c: even dims 32c + 2i (low nibbles) into acc[2c], odd dims
          // into acc[2c+1].  The codes enter as n + 136 (byte pairs 0, 2 and
          // 1, 3 of each dword: token order 0, 2, 1, 3, 4, 6, 5, 7 in both
          // operands), each token's V scale of group c goes into its weight,
          // and a product with the constant -136 (one per group: the even and
          // odd dims share it, added to both after the scan) takes the offset
          // off.
          const uint16_t cn = kBf16Neg136;
          const bf16x8 neg136 = __builtin_bit_cast(bf16x8, uint4{cn * 0x10001u, cn * 0x10001u, cn * 0x10001u, cn * 0x10001u});
#pragma unroll
          for (int c = 0; c < TL::CPR; ++c) {
            constexpr int tok[8] = {0, 2, 1, 3, 4, 6, 5, 7};
            bf16x8 pc;
#pragma unroll
            for (int k = 0; k < 8; ++k) pc[k] = (__bf16)(pv[tok[k]] * vo.vs4[tok[k]][c]);
            const uint32_t x0 = (uint32_t)vo.raw4[c][0], x1 = (uint32_t)vo.raw4[c][1];
            const bf16x8 lo8 = __builtin_bit_cast(bf16x8, uint4{nib_pair(x0, 0), nib_pair(x0, 8), nib_pair(x1, 0), nib_pair(x1, 8)});
            const bf16x8 hi8 = __builtin_bit_cast(bf16x8, uint4{nib_pair(x0, 4), nib_pair(x0, 12), nib_pair(x1, 4), nib_pair(x1, 12)});
            acc[2 * c] = mfma16(lo8, pc, acc[2 * c]);
            acc[2 * c + 1] = mfma16(hi8, pc, acc[2 * c + 1]);
            corr[c] = mfma16(neg136, pc, corr[c]);
          }
        } else {
#pragma unroll
          for (int db = 0; db < TL::NDB; ++db) acc[db] = mfma16(vop[db], pf, acc[db]);
#pragma unroll
          for (int db = 0; db < TL::NDB; ++db) acc[db] = mfma16(vop[db], plo, acc[db]);
        }
      };

      // pipeline over this wave's blocks (every 4th 32-token block of [t0, tend))
      const int nblk = tend > t0 ? (tend - t0 + kBlk - 1) / kBlk : 0;
      const int n_it = nblk > w ? (nblk - w + kWaves - 1) / kWaves : 0;
      constexpr int kStride = kWaves * kBlk;
      const int g0 = t0 + w * kBlk;
      // (the transposing V reads of a block come before the next block's
      // direct-to-LDS copies into the same stage array would be issued)
      if (n_it > 0) {
        Vops vo;
        if constexpr (TL::STAGES == 3) {
          // Blocks it + 1 and it + 2 load while block it is consumed.  Every
          // step issues one block, so every wait is the same count; blocks
          // past the last are issued too (clamped onto the piece's last
          // tokens: cached, valid data into stages nobody consumes).
          constexpr int kWait = 0x0F70 | (TL::OPS & 15) | ((TL::OPS >> 4) << 14);  // vmcnt(OPS): one block may still load
          static_assert(TL::OPS < 64, "wait count");
          Kbuf k0, k1, k2;
          issue(g0, k0, vst0);
          issue(g0 + kStride, k1, vst1);
          // full trips of three steps, no exit inside (an exit after a step
          // would let the compiler sink the next blocks' K loads past it,
          // behind later copies, and then wait for everything)
          int it = 0, gi = g0;
          for (; it + 3 <= n_it; it += 3, gi += 3 * kStride) {
            __builtin_amdgcn_s_waitcnt(kWait);
            vread(vst0, vo);
            __builtin_amdgcn_sched_barrier(0);
            issue(gi + 2 * kStride, k2, vst2);
            __builtin_amdgcn_sched_barrier(0);
            consume(gi, k0, vo);
            __builtin_amdgcn_s_waitcnt(kWait);
            vread(vst1, vo);
            __builtin_amdgcn_sched_barrier(0);
            issue(gi + 3 * kStride, k0, vst0);
            __builtin_amdgcn_sched_barrier(0);
            consume(gi + kStride, k1, vo);
            __builtin_amdgcn_s_waitcnt(kWait);
            vread(vst2, vo);
            __builtin_amdgcn_sched_barrier(0);
            issue(gi + 4 * kStride, k1, vst1);
            __builtin_amdgcn_sched_barrier(0);
            consume(gi + 2 * kStride, k2, vo);
          }
          // the last one or two blocks (already loading into stages 0 and 1)
          if (it < n_it) {
            __builtin_amdgcn_s_waitcnt(kWait);
            vread(vst0, vo);
            consume(gi, k0, vo);
            if (it + 1 < n_it) {
              __builtin_amdgcn_s_waitcnt(0x0F70);
              vread(vst1, vo);
              consume(gi + kStride, k1, vo);
            }
          }
        } else {
          // one block loads while the previous one is consumed (counted, with
          // a single loop exit)
          Kbuf k0, k1;
          issue(g0, k0, vst0);
          int it = 0, gi = g0;
          for (; it + 2 <= n_it; it += 2) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this block's loads have landed
            vread(vst0, vo);
            __builtin_amdgcn_sched_barrier(0);
            issue(gi + kStride, k1, vst1);
            __builtin_amdgcn_sched_barrier(0);
            consume(gi, k0, vo);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            vread(vst1, vo);
            __builtin_amdgcn_sched_barrier(0);
            if (it + 2 < n_it) issue(gi + 2 * kStride, k0, vst0);
            __builtin_amdgcn_sched_barrier(0);
            consume(gi + kStride, k1, vo);
            gi += 2 * kStride;
          }
          if (it < n_it) {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            vread(vst0, vo);
            consume(gi, k0, vo);
          }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy into a V tile is still in flight
      }

      if constexpr (KV == ATTN_INT4) {
#pragma unroll
        for (int c = 0; c < TL::CPR; ++c) {
          acc[2 * c] += corr[c];
          acc[2 * c + 1] += corr[c];
        }
      }
      // the row's sum over the lane quarters; then combine the waves through LDS
      {
        float u0, u1;
        lane_pair<16>(l, u0, u1);
        l = u0 + u1;
        lane_pair<32>(l, u0, u1);
        l = u0 + u1;
      }
#pragma unroll
      for (int db = 0; db < TL::NDB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // output dim of accumulator row 4j + q: 16*db + 4j + q, or for int4 the
          // interleaved dims 32*(db/2) + 2*(4j + q) + db%2
          const int d = KV == ATTN_INT4 ? 32 * (db >> 1) + 2 * (4 * j + q) + (db & 1) : 16 * db + 4 * j + q;
          red_acc[(w * kRows + i) * D + d] = acc[db][q];
        }
      if (j == 0) {
        red_m[w * kRows + i] = m;
        red_l[w * kRows + i] = l;
      }
      if (lane == 0) red_bad[w] = bad_page;
      __syncthreads();
      float vmul = 1.f;
      if constexpr (KV == ATTN_FP8_E4M3) vmul = a.v_scale[hk];
      bool poison = false;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) poison |= red_bad[ww] != 0;
      // four consecutive dims of one row per item: the row's wave weights
      // once, then one 16-byte LDS read per wave
      for (int idx = tid; idx < n_rows * (D / 4); idx += kThreads) {
        const int rr = idx / (D / 4), d0 = 4 * (idx - rr * (D / 4));
        float mw[kWaves];
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          mw[ww] = red_m[ww * kRows + rr];
          M = fmaxf(M, mw[ww]);
        }
        float den = 0.f;
        f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          const float f = mw[ww] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[ww] - M);
          den = fmaf(f, red_l[ww * kRows + rr], den);
          num += f * *(const f32x4*)(red_acc + (ww * kRows + rr) * D + d0);
        }
        const float sc = den > 0.f ? vmul / den : 0.f;
        const int rg = r0 + rr;
        const int64_t orow = ((int64_t)b * n_q + rg / G) * a.Hq + (int64_t)hk * G + rg % G;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float val = poison ? __builtin_nanf("") : num[e] * sc;
          if (whole) a.o[orow * D + d0 + e] = val;
          else dec::rec_store<true>(rec + (int64_t)rg * D + d0 + e, val);
        }
      }
      if (tid < n_rows) {
        float M = red_m[tid];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, red_m[ww * kRows + tid]);
        float den = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          const float mw = red_m[ww * kRows + tid];
          den = fmaf(mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M), red_l[ww * kRows + tid], den);
        }
        const float v = poison ? __builtin_nanf("") : den > 0.f ? M + __log2f(den) : -INFINITY;
        const int rg = r0 + tid;
        if (!whole) dec::rec_store<true>(rec + (int64_t)RT * D + rg, v);
        else if (a.lse) a.lse[((int64_t)b * a.Hq + (int64_t)hk * G + rg % G) * n_q + rg / G] = v * kLn2;
      }
      __syncthreads();  // the partials are read before the next pass writes its own
    }
    if (!whole) {
      // Fused merge: the segment's records come from the units holding its
      // groups, fu .. lu (records fu + seg .. lu + seg).  Each such unit
      // counts itself in at device scope once its record stores (device
      // scope too) have completed; the one that completes the count merges
      // the records into the output and clears the counter for the next call.
      // The counter word holds a 48-bit per-call tag above a 16-bit count, so
      // a word left from an earlier call or never written counts as zero.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) {
        uint64_t* ctr = (uint64_t*)a.seg_info + seg;
        // One device-scope add counts this unit in when the word carries
        // this call's tag (raised at the pieces' start).  A word with a later
        // tag (never written: any bits) is opened here for this call with a
        // count of one, unless another unit has opened it meanwhile; the add
        // has left its count meaningless.
        const uint64_t v = __hip_atomic_fetch_add(ctr, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int64_t fu = ((gstart + 1) * N - 1) / W;
        const int64_t lu = (seg_end * N - 1) / W;
        const uint64_t nrec = (uint64_t)(lu - fu + 1);
        uint64_t cnt;
        if ((v >> 16) == a.tag) {
          cnt = (v & 0xFFFF) + 1;
        } else {
          uint64_t old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          for (;;) {
            if ((old >> 16) == a.tag) {
              cnt = (__hip_atomic_fetch_add(ctr, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xFFFF) + 1;
              break;
            }
            if (__hip_atomic_compare_exchange_weak(ctr, &old, (a.tag << 16) | 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)) {
              cnt = 1;
              break;
            }
          }
        }
        const bool last = cnt == nrec;
        if (last) __hip_atomic_store(ctr, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        merge_first = last ? (int)(fu + seg) : -1;
        merge_n = (int)nrec;
      }
      __syncthreads();
      asm volatile("" ::: "memory");
      const int first = merge_first, n_rec = merge_n;
      if (first >= 0) {
        for (int rr = w; rr < RT; rr += kWaves) {
          const int sq = rr / G, g = rr - (rr / G) * G;
          const int h = hk * G + g;
          float* orow = a.o + (((int64_t)b * n_q + sq) * a.Hq + h) * D;
          float* lse_out = a.lse ? a.lse + ((int64_t)b * a.Hq + h) * n_q + sq : nullptr;
          dec::merge_row<D, true>(a.part + (int64_t)first * REC, REC, RT, rr, n_rec, lane, orow, lse_out);
        }
      }
    }
    pos = pend;
  }
}

template <int KV, int D>
size_t mfma_lds_bytes(int B) {
  return (size_t)MTile<KV, D>::RED + (size_t)(B + 1) * sizeof(int64_t) + (size_t)B * sizeof(int);
}

template <int KV, int D>
attn_status launch_kd(const DecodeArgs& a, hipStream_t stream) {
  auto kern = decode_mfma_kernel<KV, D>;
  const size_t lds = mfma_lds_bytes<KV, D>(a.B);
  static std::atomic<size_t> lds_set[kMaxDevices];  // the length prefix grows with B
  attn_status st = raise_lds_limit((const void*)kern, lds, lds_set);
  if (st != ATTN_OK) return st;
  hipLaunchKernelGGL(kern, dim3(a.n_units), dim3(kThreads), lds, stream, a);
  return check_launch("decode_mfma");
}

}  // namespace

bool decode_mfma_supported(attn_dtype kv_dt, int D) {
  return kv_dt == ATTN_BF16 || kv_dt == ATTN_FP8_E4M3 || kv_dt == ATTN_INT8 || (kv_dt == ATTN_INT4 && D == 128);
}

attn_status launch_decode_split_mfma(attn_dtype kv_dt, const DecodeArgs& a, int D, hipStream_t stream) {
  switch (kv_dt) {
    case ATTN_BF16: return D == 128 ? launch_kd<ATTN_BF16, 128>(a, stream) : launch_kd<ATTN_BF16, 64>(a, stream);
    case ATTN_FP8_E4M3:
      return D == 128 ? launch_kd<ATTN_FP8_E4M3, 128>(a, stream) : launch_kd<ATTN_FP8_E4M3, 64>(a, stream);
    case ATTN_INT8: return D == 128 ? launch_kd<ATTN_INT8, 128>(a, stream) : launch_kd<ATTN_INT8, 64>(a, stream);
    case ATTN_INT4:
      if (D == 128) return launch_kd<ATTN_INT4, 128>(a, stream);
      break;
    default: break;
  }
  return set_error(ATTN_E_UNSUPPORTED, "decode: no matrix-core path for KV dtype %d", (int)kv_dt);
}

}  // namespace attn
