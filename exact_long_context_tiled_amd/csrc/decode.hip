// Split-KV ("flash") decoding: one query token per sequence against a KV
// cache.  The KV sequence of each (sequence, KV head) is scanned in pieces by
// independent work-groups; each piece yields, for all G query heads sharing
// that KV head, a normalised partial output and its log-sum-exp, and the
// pieces are combined exactly by log-sum-exp (ONNX Runtime PR #28695
// analysis, section 2: parallel KV scan over idle workers + log-sum-exp
// reduce).
//
// Work split.  The batch's KV is laid end to end as one run of 16-token
// groups, segment by segment ((sequence, KV head) in order), and cut into N
// equal runs, one per work-group, N being the number of compute units (one
// work-group each, all resident at once).  Every work-group streams the same
// number of bytes whatever the length mix, so all finish together, and the
// partial results written (one per piece, about N + segments in all, instead
// of one per fixed-size chunk) stay few: stores mixed into a saturated read
// stream cost far more than their size.  A segment that one work-group
// covers whole is written straight to the output; the others are merged by
// decode_merge_kernel.

// The caches may be paged (fixed-size pages located through a page table:
// LLM-CoOpt, "Methodology" item 3) and quantised (int8 with a per-token,
// per-KV-head scale; OCP e4m3fn with a per-KV-head scale: LLM-CoOpt
// "Methodology" item 1, ONNX Runtime PR #28695 analysis, section 1; int4
// codes packed two per byte with one scale per 32-element group: the same
// analysis, introduction); bytes are dequantised in registers right after the
// loads.
//
// This is a bandwidth-bound scan, so the vector ALUs do the arithmetic.  The
// lanes of a wave form token slots, each lane owning one slice of a token's K
// and V rows (16 bytes; 8 bytes = 16 elements for int4); every iteration a wave loads the K
// and V slices of 4 tokens per slot (all loads in flight together), reduces
// the slice dot products across the slot with row-local DPP moves, and
// folds the tokens into a per-slot online softmax (running max, sum and
// output accumulator).  K slices of every type are turned into exact bf16
// pairs (e4m3 and int8 values are all bf16 numbers) and dotted with the exact
// bf16 query by the packed bf16 dot product; V slices are converted to fp32
// for the fp32 P.V accumulation.  At the end of a piece the slots of a wave,
// then the waves of the work-group, are combined by the same max/rescale
// rule.  Pieces start on 16-token group boundaries and pages hold
// a power-of-two number >= 16 of tokens, so the tokens of one wave load step
// never straddle a page and its page-table entry is one scalar read.
#include <math.h>
#include <stdlib.h>

#include <string.h>

#include <algorithm>

#include "common.h"
#include "decode_common.h"

namespace attn {
namespace {

using dec::clamp_len;
using dec::group_prefix;
using dec::lane_pair;

// A lane's slice of a token's K or V row: 16 bytes (8 bf16, 16 e4m3 or 16
// int8 elements) or, for int4, 8 bytes (16 packed elements, so that a lane
// holds as many elements, and accumulators, as for the 8-bit types).
template <int KV>
struct KvTraits;
template <>
struct KvTraits<ATTN_BF16> {
  using Slice = uint4;
  static constexpr int kEpl = 8;
  static constexpr int row_bytes(int D) { return 2 * D; }
};
template <>
struct KvTraits<ATTN_FP8_E4M3> {
  using Slice = uint4;
  static constexpr int kEpl = 16;
  static constexpr int row_bytes(int D) { return D; }
};
template <>
struct KvTraits<ATTN_INT8> {
  using Slice = uint4;
  static constexpr int kEpl = 16;
  static constexpr int row_bytes(int D) { return D; }
};
template <>
struct KvTraits<ATTN_INT4> {
  using Slice = uint2;
  static constexpr int kEpl = 16;
  static constexpr int row_bytes(int D) { return D / 2; }
};
constexpr int kInt4Group = 32;  // elements per int4 scale group

// The 4-bit two's-complement code at nibble e (element e of the word: bits
// 4e .. 4e+3, low nibble of a byte first) as an int.  (A shift pair, not the
// bitfield-extract builtin: this compiler can convert the builtin's result to
// float as an unsigned value.)
__device__ __forceinline__ int int4_code(uint32_t w, int e) { return ((int)(w << (28 - 4 * e))) >> 28; }

// Decode one slice into EPL floats (without scales).
template <int KV>
__device__ __forceinline__ void decode_slice(const typename KvTraits<KV>::Slice& raw, float* out) {
  if constexpr (KV == ATTN_INT4) {
    const uint32_t wd[2] = {raw.x, raw.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[8 * i + e] = (float)int4_code(wd[i], e);
    }
  } else {
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
    if constexpr (KV == ATTN_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(wd[i] << 16);
        out[2 * i + 1] = __uint_as_float(wd[i] & 0xffff0000u);
      }
    } else if constexpr (KV == ATTN_FP8_E4M3) {
      // gfx950 converts OCP e4m3fn in hardware, two bytes per instruction
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], true);
        out[4 * i] = lo[0];
        out[4 * i + 1] = lo[1];
        out[4 * i + 2] = hi[0];
        out[4 * i + 3] = hi[1];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[4 * i + k] = (float)(int)(int8_t)(wd[i] >> (8 * k));
      }
    }
  }
}

// Sum over the LPT lanes (1, 2, 4, 8 or 16 adjacent lanes) that hold one
// token's slices, with row-local DPP moves (no LDS round trip).
template <int LPT>
__device__ __forceinline__ float token_sum(float x) {
  if constexpr (LPT >= 2) x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, false));  // xor 1
  if constexpr (LPT >= 4) x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, false));  // xor 2
  if constexpr (LPT >= 8) x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false));  // mirror in 8
  if constexpr (LPT >= 16) x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xf, 0xf, false));  // mirror in 16
  return x;
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// One K slice as EPL/2 exact bf16 pairs, the operand of the packed bf16 dot
// product: every e4m3fn value and every int8 / int4 code is a bf16 number.
// e4m3fn goes through gfx950's scaled fp8 -> bf16 pair conversion (scale 1);
// int8 and int4 through fp32, whose upper half is then the exact bf16.
template <int KV>
__device__ __forceinline__ void k_pairs(const typename KvTraits<KV>::Slice& raw, bf16x2* out) {
  if constexpr (KV == ATTN_INT4) {
    const uint32_t wd[2] = {raw.x, raw.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float f0 = (float)int4_code(wd[i], e);
        const float f1 = (float)int4_code(wd[i], e + 1);
        out[4 * i + e / 2] = __builtin_bit_cast(
            bf16x2, __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u));
      }
    }
  } else {
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
    if constexpr (KV == ATTN_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = __builtin_bit_cast(bf16x2, wd[i]);
    } else if constexpr (KV == ATTN_FP8_E4M3) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)wd[i], 1.0f, false);
        out[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)wd[i], 1.0f, true);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const float f0 = (float)(int)(int8_t)(wd[i] >> (16 * hf));
          const float f1 = (float)(int)(int8_t)(wd[i] >> (16 * hf + 8));
          out[2 * i + hf] = __builtin_bit_cast(
              bf16x2, __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u));
        }
      }
    }
  }
}

// Merge the online-softmax states (m, l, acc) of lanes OFF apart.
template <int OFF, int G, int EPL>
__device__ __forceinline__ void combine_lanes(float (&m)[G], float (&l)[G], float (&acc)[G][EPL]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m0, m1, l0, l1;
    lane_pair<OFF>(m[g], m0, m1);
    lane_pair<OFF>(l[g], l0, l1);
    const float M = fmaxf(m0, m1);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float f0 = __builtin_amdgcn_exp2f(m0 - Mu), f1 = __builtin_amdgcn_exp2f(m1 - Mu);
    l[g] = l0 * f0 + l1 * f1;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float a0, a1;
      lane_pair<OFF>(acc[g][e], a0, a1);
      acc[g][e] = a0 * f0 + a1 * f1;
    }
    m[g] = M;
  }
}

constexpr int kDecodeWaves = 4;  // waves per work-group
constexpr int kDecodeThreads = 64 * kDecodeWaves;

// Rows of a segment: R = n_q * G query rows (query token s, head g) share the
// (sequence, KV head) KV.  They are processed TQ query tokens (TQ * G <= 8
// rows, what the registers hold) at a time; a piece's later row chunks re-read
// the piece's K/V right after the first, from the caches.
template <int KV, int D, int G, int TQ>
__global__ void __launch_bounds__(kDecodeThreads) decode_split_kernel(DecodeArgs a) {
  using Tr = KvTraits<KV>;
  using Slice = typename Tr::Slice;
  constexpr int EPL = Tr::kEpl;  // elements per lane slice
  constexpr int LPT = D / EPL;   // lanes per token
  constexpr int TPW = 64 / LPT;  // tokens per wave per load step (token slots)
  constexpr int U = 4;           // load steps per iteration
  constexpr int TPI = TPW * U;   // tokens per wave per iteration
  constexpr int RC = TQ * G;      // rows per chunk
  const int RT = a.n_q * G;      // rows per segment
  const int REC = decode_record_floats(RT, D);
  static_assert(kDecodeGroup % TPW == 0, "a load step must not straddle a group");
  extern __shared__ int64_t pre[];  // [B + 1]
  __shared__ float red_acc[kDecodeWaves][RC * D];
  __shared__ float red_m[kDecodeWaves][RC], red_l[kDecodeWaves][RC];
  __shared__ int64_t wsum[kDecodeWaves];
  __shared__ int red_bad[kDecodeWaves];  // per wave: a page-table entry outside the cache was met

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int slot = lane / LPT, part = lane % LPT;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // wave index as a scalar
  const uint8_t* kb = (const uint8_t*)a.k;
  const uint8_t* vb = (const uint8_t*)a.v;
  const int64_t lane_off = (int64_t)part * sizeof(Slice);
  constexpr int64_t RB = Tr::row_bytes(D);  // bytes of one token's K (or V) row
  constexpr int kStride = kDecodeWaves * TPI;  // tokens between a wave's consecutive iterations

  group_prefix<kDecodeThreads>(a.kv_lens, a.B, a.max_kv_len, 0, pre, wsum);
  const int64_t W = pre[a.B] * a.Hkv;
  // never more units than groups, so that every unit owns at least one group
  // and the records of a segment are the consecutive units that cover it
  const int64_t N = a.n_units < W ? (int64_t)a.n_units : W;
  const int unit = blockIdx.x;
  if (unit >= N) return;
  const int64_t x1 = (unit + 1) * W / N;

  for (int64_t pos = unit * W / N; pos < x1;) {
    // the segment holding group `pos`: the last sequence starting at or before it
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] * a.Hkv <= pos) lo = mid;
      else hi = mid - 1;
    }
    const int b = __builtin_amdgcn_readfirstlane(lo);
    const int64_t sbase = pre[b] * a.Hkv;
    const int ng = (int)(pre[b + 1] - pre[b]);
    const int hk = __builtin_amdgcn_readfirstlane((int)((pos - sbase) / ng));
    const int j0 = (int)(pos - sbase - (int64_t)hk * ng);
    const int64_t seg_end = sbase + (int64_t)(hk + 1) * ng;
    const int64_t pend = seg_end < x1 ? seg_end : x1;
    const int T = clamp_len(a.kv_lens[b], a.max_kv_len);
    const int t0 = __builtin_amdgcn_readfirstlane(j0 * kDecodeGroup);
    const int t1 = __builtin_amdgcn_readfirstlane(min(T, (j0 + (int)(pend - pos)) * kDecodeGroup));
    const int seg = b * a.Hkv + hk;
    const bool whole = j0 == 0 && pend == seg_end;
    const int n_q = a.n_q;
    float smul = a.scale_log2;  // scale*log2(e) (and the e4m3 per-head K scale)
    if constexpr (KV == ATTN_FP8_E4M3) smul *= a.k_scale[hk];
    const int64_t hk_rows = (int64_t)hk * a.page_size;
    float* rec = a.part + (int64_t)(unit + seg) * REC;
    bool bad_page = false;  // a page-table entry of this piece lay outside the cache
    for (int s0 = 0; s0 < n_q; s0 += TQ) {
    // query token s sits at position T - n_q + s and sees the keys before
    // T - (n_q - 1 - s); rows past the last query token repeat it (not written)
    const int tq_n = min(TQ, n_q - s0);
    int lim[TQ];
#pragma unroll
    for (int j = 0; j < TQ; ++j) lim[j] = max(t0, min(t1, T - (n_q - 1 - (s0 + min(j, tq_n - 1)))));
    const int tend = lim[TQ - 1];  // this chunk reads keys [t0, tend)

    // query slices as exact bf16 pairs for the packed dot product
    bf16x2 q2[RC][EPL / 2];
#pragma unroll
    for (int j = 0; j < TQ; ++j) {
      // q row (b, s, hk*G + g) of [B, n_q, Hq, D]
      const uint16_t* qb = (const uint16_t*)a.q +
                           (((int64_t)b * n_q + s0 + min(j, tq_n - 1)) * a.Hq + (int64_t)hk * G) * D + part * EPL;
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < EPL; e += 8) {
          const uint4 raw = *(const uint4*)(qb + (int64_t)g * D + e);
          const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) q2[j * G + g][e / 2 + i] = __builtin_bit_cast(bf16x2, wd[i]);
        }
      }
    }

    float m[RC], l[RC], acc[RC][EPL];
#pragma unroll
    for (int g = 0; g < RC; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }

    // Loads of one iteration (U steps of TPW tokens).  TPW consecutive tokens
    // from a TPW-aligned index never straddle a page and every step index is
    // wave-uniform, so the page-table entries are scalar loads issued first.
    struct Buf {
      Slice kr[U], vr[U];
      float ksc[U], vsc[U];
    };
    // Every call issues the same number of vector loads with no branch around
    // them (tokens past the piece are clamped onto its last token, a cache
    // hit), so the compiler's wait counters keep the next iteration's loads in
    // flight while the current one is consumed.
    auto issue = [&](int g0, Buf& bf) {
      int64_t step_row[U];  // cache row of token 0 of the step's page
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // first token of the step, wave-uniform and inside the piece;
        // readfirstlane keeps it (and the page-table read) on the scalar unit
        const int tc = __builtin_amdgcn_readfirstlane(min(g0 + u * TPW, tend - 1));
        if (a.page_table) {
          // read through the constant address space: a scalar (SMEM) load
          const auto* pt = (const __attribute__((address_space(4))) int32_t*)a.page_table;
          const int pe = pt[(int64_t)b * a.max_pages + (tc >> a.page_shift)];
          // an entry outside the cache is never dereferenced: page 0 is read
          // instead and the rows of the piece are written as NaN
          const bool ok = (uint32_t)pe < (uint32_t)a.num_pages;
          bad_page |= !ok;
          const int pg = ok ? pe : 0;
          step_row[u] = (int64_t)pg * a.Hkv * a.page_size + hk_rows - (tc & ~(a.page_size - 1));
        } else {
          step_row[u] = (int64_t)b * a.Hkv * a.page_size + hk_rows;
        }
      }
      // (all scalar work first, then the vector loads back to back; with the
      // lane's token clamped as a whole index the compiler's wait counters
      // keep the other buffer's loads in flight)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t row = step_row[u] + min(g0 + u * TPW + slot, tend - 1);
        bf.kr[u] = *(const Slice*)(kb + row * RB + lane_off);
        bf.vr[u] = *(const Slice*)(vb + row * RB + lane_off);
        if constexpr (KV == ATTN_INT8) {
          bf.ksc[u] = a.k_scale[row];  // q already carries scale*log2(e)
          bf.vsc[u] = a.v_scale[row];
        } else if constexpr (KV == ATTN_INT4) {
          // the scale of this lane's 32-element group (two lane slices per group)
          bf.ksc[u] = a.k_scale[row * (D / kInt4Group) + (part * EPL) / kInt4Group];
          bf.vsc[u] = a.v_scale[row * (D / kInt4Group) + (part * EPL) / kInt4Group];
        } else {
          bf.ksc[u] = bf.vsc[u] = 1.f;
        }
      }
    };
    auto consume = [&](int g0, const Buf& bf) {
      // raw scores of the U tokens of this lane's slot (int8: times the token's K scale)
      float s[U][RC];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bf16x2 kp[EPL / 2];
        k_pairs<KV>(bf.kr[u], kp);
#pragma unroll
        for (int g = 0; g < RC; ++g) {
          float d = 0.f;
#pragma unroll
          for (int i = 0; i < EPL / 2; ++i) d = __builtin_amdgcn_fdot2_f32_bf16(q2[g][i], kp[i], d, false);
          if constexpr (KV == ATTN_INT4) d *= bf.ksc[u];  // a group scale differs between lanes
          s[u][g] = d;
        }
#pragma unroll
        for (int g = 0; g < RC; ++g) {
          s[u][g] = token_sum<LPT>(s[u][g]);
          if constexpr (KV == ATTN_INT8) s[u][g] *= bf.ksc[u];
        }
      }
      if (g0 + TPI > lim[0]) {  // near the end: keys past a row's limit weigh nothing
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int tok = g0 + u * TPW + slot;
#pragma unroll
          for (int g = 0; g < RC; ++g) s[u][g] = tok < lim[g / G] ? s[u][g] : -INFINITY;
        }
      }
      float vv[U][EPL];
#pragma unroll
      for (int u = 0; u < U; ++u) decode_slice<KV>(bf.vr[u], vv[u]);
      // Scores enter the softmax as s*smul (log2 domain, smul > 0).  The
      // reference max m of a slot only moves when a score exceeds it by more
      // than 8, so p <= 256 and the rescale of the accumulators is skipped
      // for the whole wave on most iterations; any reference gives the exact
      // result.
      float tx[RC];
      bool grow = false;
#pragma unroll
      for (int g = 0; g < RC; ++g) {
        float mx = s[0][g];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][g]);
        tx[g] = mx * smul;
        grow |= tx[g] > m[g] + 8.f;
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int g = 0; g < RC; ++g) {
          const float m_new = fmaxf(m[g], tx[g]);
          const float alpha = __builtin_amdgcn_exp2f(m[g] - (m_new == -INFINITY ? 0.f : m_new));
          m[g] = m_new;
          l[g] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
        }
      }
#pragma unroll
      for (int g = 0; g < RC; ++g) {
        const float nm = m[g] == -INFINITY ? 0.f : -m[g];
        float p[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          p[u] = __builtin_amdgcn_exp2f(fmaf(s[u][g], smul, nm));
          l[g] += p[u];
          if constexpr (KV == ATTN_INT8 || KV == ATTN_INT4) p[u] *= bf.vsc[u];
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float x = acc[g][e];
#pragma unroll
          for (int u = 0; u < U; ++u) x = fmaf(p[u], vv[u][e], x);
          acc[g][e] = x;
        }
      }
    };

    // two-stage software pipeline: the next iteration's loads are in flight
    // while the current one is consumed.  Two iterations per trip and a
    // single loop exit: with an exit after each half, the compiler merges
    // the exits into one latch, and its (path-insensitive) wait counters
    // would then drain the in-flight buffer at the top of every trip.
    // (The scheduling barriers keep the compiler from sinking a batch of
    // loads down to its consumer to save registers, which would serialise
    // them.)
    Buf b0, b1;
    int g0 = t0 + wu * TPI;
    const int n_it = g0 < tend ? (tend - g0 + kStride - 1) / kStride : 0;  // iterations of this wave
    if (n_it > 0) {
      issue(g0, b0);
      int k = 0;
      for (; k + 2 <= n_it; k += 2) {
        issue(g0 + kStride, b1);
        __builtin_amdgcn_sched_barrier(0);
        consume(g0, b0);
        issue(g0 + 2 * kStride, b0);  // past the end on the last trip: clamped re-reads
        __builtin_amdgcn_sched_barrier(0);
        consume(g0 + kStride, b1);
        g0 += 2 * kStride;
      }
      if (k < n_it) consume(g0, b0);
    }

    // combine the token slots of the wave (lanes LPT, 2*LPT, ... apart hold the same d slice)
    if constexpr (LPT <= 4) combine_lanes<4, RC, EPL>(m, l, acc);
    if constexpr (LPT <= 8) combine_lanes<8, RC, EPL>(m, l, acc);
    if constexpr (LPT <= 16) combine_lanes<16, RC, EPL>(m, l, acc);
    combine_lanes<32, RC, EPL>(m, l, acc);
    // combine the waves through LDS
    if (slot == 0) {
#pragma unroll
      for (int g = 0; g < RC; ++g) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) red_acc[w][g * D + part * EPL + e] = acc[g][e];
        if (part == 0) {
          red_m[w][g] = m[g];
          red_l[w][g] = l[g];
        }
      }
    }
    if (lane == 0) red_bad[w] = bad_page;
    __syncthreads();
    float vmul = 1.f;
    if constexpr (KV == ATTN_FP8_E4M3) vmul = a.v_scale[hk];
    bool poison = false;
#pragma unroll
    for (int ww = 0; ww < kDecodeWaves; ++ww) poison |= red_bad[ww] != 0;
    // rows s0*G .. s0*G + RC - 1 of the segment's record; a row whose keys all
    // lie past its limit has a zero sum: O = 0, lse = -inf
    const int n_rows = tq_n * G;
    for (int idx = tid; idx < n_rows * D; idx += kDecodeThreads) {
      const int g = idx / D;
      float M = red_m[0][g];
#pragma unroll
      for (int ww = 1; ww < kDecodeWaves; ++ww) M = fmaxf(M, red_m[ww][g]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int ww = 0; ww < kDecodeWaves; ++ww) {
        const float f = red_m[ww][g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red_m[ww][g] - M);
        num = fmaf(f, red_acc[ww][idx], num);
        den = fmaf(f, red_l[ww][g], den);
      }
      const float val = poison ? __builtin_nanf("") : den > 0.f ? num * (vmul / den) : 0.f;
      if (whole) {  // o row (b, s0 + g / G, hk*G + g % G) of [B, n_q, Hq, D]
        const int64_t orow = ((int64_t)b * n_q + s0 + g / G) * a.Hq + (int64_t)hk * G + g % G;
        a.o[orow * D + idx % D] = val;
      } else {
        rec[(int64_t)s0 * G * D + idx] = val;
      }
    }
    if (tid < n_rows) {  // the piece's lse (log2) of each row
      float M = red_m[0][tid];
#pragma unroll
      for (int ww = 1; ww < kDecodeWaves; ++ww) M = fmaxf(M, red_m[ww][tid]);
      float den = 0.f;
#pragma unroll
      for (int ww = 0; ww < kDecodeWaves; ++ww)
        den = fmaf(red_m[ww][tid] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red_m[ww][tid] - M), red_l[ww][tid], den);
      const float v = poison ? __builtin_nanf("") : den > 0.f ? M + __log2f(den) : -INFINITY;
      if (!whole) {
        rec[(int64_t)RT * D + s0 * G + tid] = v;
      } else if (a.lse) {  // lse [B, Hq, n_q]
        a.lse[((int64_t)b * a.Hq + (int64_t)hk * G + tid % G) * n_q + s0 + tid / G] = v * kLn2;
      }
    }
    __syncthreads();  // LDS is reused by the next row chunk
    }  // row chunks
    if (tid == 0 && j0 == 0) {
      // records of this segment: units unit .. (the unit holding its last group)
      const int last = whole ? unit : (int)((seg_end * N - 1) / W);
      a.seg_info[2 * seg] = unit + seg;
      a.seg_info[2 * seg + 1] = last - unit + 1;
    }
    pos = pend;
  }
}

// One wave per output row (b, s, h): merges the records of its segment by
// log-sum-exp, or writes O = 0, lse = -inf for an empty sequence.  Segments
// finished by a single unit were written by the split kernel already.
template <int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeArgs a, int G) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // o row of [B, n_q, Hq, D]
  const int n_q = a.n_q;
  if (row >= (int64_t)a.B * n_q * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int h = (int)(row % a.Hq);
  const int64_t bs = row / a.Hq;
  const int b = (int)(bs / n_q), sq = (int)(bs - (int64_t)b * n_q);
  const int hk = h / G, g = h - hk * G;
  const int seg = b * a.Hkv + hk;
  const int64_t lrow = ((int64_t)b * a.Hq + h) * n_q + sq;  // lse [B, Hq, n_q]
  // both loads in flight together; seg_info is only meaningful for a non-empty sequence
  const int T = clamp_len(a.kv_lens[b], a.max_kv_len);
  const int first = a.seg_info[2 * seg], n = a.seg_info[2 * seg + 1];
  float* orow = a.o + row * D;
  constexpr int CPL = D / 64;  // columns per lane
  if (T == 0) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) orow[lane + 64 * k] = 0.f;
    if (lane == 0 && a.lse) a.lse[lrow] = -INFINITY;
    return;
  }
  if (n <= 1) return;
  const int RT = n_q * G;
  const int REC = decode_record_floats(RT, D);
  dec::merge_row<D, false>(a.part + (int64_t)first * REC, REC, RT, sq * G + g, n, lane, orow,
                           a.lse ? a.lse + lrow : nullptr);
}

template <int KV, int D, int G, int TQ>
attn_status launch_one(DecodeArgs a, hipStream_t stream) {
  const size_t lds = (size_t)(a.B + 1) * sizeof(int64_t);
  auto kern = decode_split_kernel<KV, D, G, TQ>;
  static std::atomic<size_t> lds_set[kMaxDevices];  // the length prefix may pass the default dynamic limit
  attn_status st = raise_lds_limit((const void*)kern, lds, lds_set);
  if (st != ATTN_OK) return st;
  hipLaunchKernelGGL(kern, dim3(a.n_units), dim3(kDecodeThreads), lds, stream, a);
  return check_launch("decode_split");
}

// Query tokens per row chunk: enough to cover n_q in as few chunks as the
// registers allow (TQ * G <= 8).
template <int KV, int D, int G>
attn_status launch_tq(const DecodeArgs& a, hipStream_t stream) {
  constexpr int kMaxTq = 8 / G;
  const int want = std::min(a.n_q, kMaxTq);
  if (want <= 1) return launch_one<KV, D, G, 1>(a, stream);
  if constexpr (kMaxTq >= 2) {
    if (want <= 2) return launch_one<KV, D, G, 2>(a, stream);
  }
  if constexpr (kMaxTq >= 4) {
    if (want <= 4) return launch_one<KV, D, G, 4>(a, stream);
  }
  if constexpr (kMaxTq >= 8) return launch_one<KV, D, G, 8>(a, stream);
  return set_error(ATTN_E_DEVICE, "decode: no row-chunk variant");
}

template <int KV, int D>
attn_status launch_g(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_tq<KV, D, 1>(a, stream);
    case 2: return launch_tq<KV, D, 2>(a, stream);
    case 3: return launch_tq<KV, D, 3>(a, stream);
    case 4: return launch_tq<KV, D, 4>(a, stream);
    case 5: return launch_tq<KV, D, 5>(a, stream);
    case 6: return launch_tq<KV, D, 6>(a, stream);
    case 7: return launch_tq<KV, D, 7>(a, stream);
    case 8: return launch_tq<KV, D, 8>(a, stream);
  }
  return set_error(ATTN_E_UNSUPPORTED, "decode: query heads per KV head must be 1..8 (got %d)", G);
}

template <int KV>
attn_status launch_d(const DecodeArgs& a, int D, int G, hipStream_t stream) {
  return D == 128 ? launch_g<KV, 128>(a, G, stream) : launch_g<KV, 64>(a, G, stream);
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hkv, int rows, int D, int n_units_bound) {
  const size_t segs = (size_t)B * (size_t)Hkv;
  const size_t recs = (size_t)n_units_bound + segs;  // record indices stay below N + segments - 1
  const size_t rec_bytes = (recs * (size_t)decode_record_floats(rows, D) * sizeof(float) + 255) / 256 * 256;
  return rec_bytes + (segs * 2 * sizeof(int32_t) + 255) / 256 * 256;
}

attn_status launch_decode(attn_dtype kv_dt, const DecodeArgs& a0, int D, int G, hipStream_t stream) {
  DecodeArgs a = a0;
  a.G = G;
  const DecodeTuning tu = decode_tuning();
  if (a.n_units <= 0) {
    // one work-group per compute unit: measured faster than filling every
    // resident slot (fewer partial records, and the scan stays bandwidth-bound)
    a.n_units = std::min(kDecodeMaxAutoUnits, tu.units > 0 ? tu.units : device_cu_count());
  }
  const bool valu = tu.path == 1;
  attn_status st;
  a.piece_groups = 0;
  if (decode_mfma_supported(kv_dt, D) && !valu) {
    // Each piece of a run (a segment, or the part of one inside the run) has
    // a fixed cost on the matrix-core kernel: its pipeline start, the wave
    // combine and the record, ~6 us measured, about what one work-group
    // streams in that time (192 KB by a sweep).  Charging every segment that many
    // groups in the split gives a run that reaches into another segment
    // correspondingly fewer keys, so work-groups with several pieces finish
    // with the others.
    const int64_t tok = decode_token_bytes(kv_dt, D) * kDecodeGroup;  // K + V bytes of one group, one KV head
    const int64_t cost = tu.piece_bytes >= 0 ? tu.piece_bytes : kDecodePieceBytes;
    a.piece_groups = (int)std::min<int64_t>(kDecodeMaxPieceGroups, (cost + tok - 1) / tok);
    // the matrix-core split merges split segments itself (last-arriving unit)
    static std::atomic<uint64_t> calls{0};
    a.tag = (calls.fetch_add(1, std::memory_order_relaxed) % ((uint64_t(1) << 48) - 1)) + 1;
    return launch_decode_split_mfma(kv_dt, a, D, stream);
  } else {
    switch (kv_dt) {
      case ATTN_BF16: st = launch_d<ATTN_BF16>(a, D, G, stream); break;
      case ATTN_FP8_E4M3: st = launch_d<ATTN_FP8_E4M3>(a, D, G, stream); break;
      case ATTN_INT8: st = launch_d<ATTN_INT8>(a, D, G, stream); break;
      case ATTN_INT4: st = launch_d<ATTN_INT4>(a, D, G, stream); break;
      default: return set_error(ATTN_E_UNSUPPORTED, "decode: unsupported KV dtype %d", (int)kv_dt);
    }
  }
  if (st != ATTN_OK) return st;
  const int64_t rows = (int64_t)a.B * a.n_q * a.Hq;
  if (D == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a, G);
  else
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a, G);
  return check_launch("decode_merge");
}

}  // namespace attn
