// Split-KV ("flash") decoding: one query token per sequence against a KV
// cache.  The KV sequence of each (sequence, KV head) is cut into chunks; one
// work-group per chunk produces, for all G query heads sharing that KV head,
// the chunk's normalised partial output and its log-sum-exp, and a merge
// kernel combines the chunks exactly (ONNX Runtime PR #28695 analysis,
// section 2: parallel KV scan over idle workers + log-sum-exp reduce).
//
// The caches may be paged (fixed-size pages located through a page table:
// LLM-CoOpt, "Methodology" item 3) and quantised (int8 with a per-token,
// per-KV-head scale; OCP e4m3fn with a per-KV-head scale: LLM-CoOpt
// "Methodology" item 1, ONNX Runtime PR #28695 analysis, section 1); bytes are
// dequantised in registers right after the 16-byte loads.
//
// This is a bandwidth-bound scan, so the vector ALUs do the arithmetic.  The
// lanes of a wave form token slots of D*bytes/16 lanes, each lane owning one
// 16-byte slice of a token's K and V rows; every iteration a wave loads the K
// and V slices of 4 tokens per slot (all loads in flight together), reduces
// the slice dot products across the slot with row-local DPP moves, and
// folds the tokens into a per-slot online softmax (running max, sum and
// output accumulator).  bf16 K is dotted with the exact bf16 query in packed
// bf16 pairs; int8 / fp8 slices are converted to fp32.  At the end the slots
// of a wave, then the four waves, are combined by the same max/rescale rule.
// Pages hold >= 16 tokens, so the page-table entry of each load step is one
// wave-uniform (scalar) read.
#include <math.h>

#include <algorithm>

#include "common.h"

namespace attn {
namespace {

template <int KV>
struct KvTraits;
template <>
struct KvTraits<ATTN_BF16> {
  static constexpr int kBytes = 2;
};
template <>
struct KvTraits<ATTN_FP8_E4M3> {
  static constexpr int kBytes = 1;
};
template <>
struct KvTraits<ATTN_INT8> {
  static constexpr int kBytes = 1;
};

// Decode one 16-byte slice into EPL floats (without scales).
template <int KV>
__device__ __forceinline__ void decode16(uint4 raw, float* out) {
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

// Row index (token row of the cache, without the D dimension).
__device__ __forceinline__ int64_t cache_row(const DecodeArgs& a, int b, int hk, int t) {
  if (a.page_table) {
    const int p = a.page_table[(int64_t)b * a.max_pages + (t >> a.page_shift)];
    return ((int64_t)p * a.Hkv + hk) * a.page_size + (t & (a.page_size - 1));
  }
  return ((int64_t)b * a.Hkv + hk) * a.page_size + t;
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

template <int KV, int D, int G>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
  constexpr int EB = KvTraits<KV>::kBytes;
  constexpr int EPL = 16 / EB;   // elements per lane slice
  constexpr int LPT = D / EPL;   // lanes per token
  constexpr int TPW = 64 / LPT;  // tokens per wave per load step (token slots)
  constexpr int U = EB == 2 ? 4 : 2;  // load steps per iteration (16 tokens per wave at D = 128)
  constexpr int TPI = TPW * U;   // tokens per wave per iteration
  constexpr bool kDot2 = KV == ATTN_BF16;
  __shared__ float red_acc[4][G * D];
  __shared__ float red_m[4][G], red_l[4][G];

  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int slot = lane / LPT, part = lane % LPT;
  const int64_t BHq = (int64_t)a.B * a.Hq;
  const int64_t row0 = (int64_t)b * a.Hq + (int64_t)hk * G;  // first (b, h) row of this group
  const int T = a.kv_lens[b];
  const int t0 = split * a.chunk;
  const int t1 = min(T, t0 + a.chunk);
  if (t0 >= t1) {  // no token in this chunk: an empty partial
    if (tid < G) a.part_lse[(int64_t)split * BHq + row0 + tid] = -INFINITY;
    return;
  }

  // query slices: exact bf16 pairs for the packed dot (bf16 cache), or fp32
  // pre-multiplied by scale*log2(e) (and the fp8 per-head K scale)
  bf16x2 q2[kDot2 ? G : 1][kDot2 ? EPL / 2 : 1];
  float qf[kDot2 ? 1 : G][kDot2 ? 1 : EPL];
  float smul = a.scale_log2;
  {
    const uint16_t* qb = (const uint16_t*)a.q + row0 * D + part * EPL;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; e += 8) {
        const uint4 raw = *(const uint4*)(qb + (int64_t)g * D + e);
        if constexpr (kDot2) {
          const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) q2[g][e / 2 + i] = __builtin_bit_cast(bf16x2, wd[i]);
        } else {
          float tmp[8];
          decode16<ATTN_BF16>(raw, tmp);
          float qmul = a.scale_log2;
          if constexpr (KV == ATTN_FP8_E4M3) qmul *= a.k_scale[hk];
#pragma unroll
          for (int i = 0; i < 8; ++i) qf[g][e + i] = tmp[i] * qmul;
        }
      }
    }
    if constexpr (!kDot2) smul = 1.f;
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const uint8_t* kb = (const uint8_t*)a.k;
  const uint8_t* vb = (const uint8_t*)a.v;
  const int64_t lane_off = (int64_t)part * EPL * EB;

  const int wu = __builtin_amdgcn_readfirstlane(w);  // wave index as a scalar
  const int64_t hk_rows = (int64_t)hk * a.page_size;
  constexpr int kStride = 4 * TPI;  // tokens between a wave's consecutive iterations

  // Loads of one iteration (U steps of TPW tokens).  TPW consecutive tokens
  // from a TPW-aligned index never straddle a page and every step index is
  // wave-uniform, so the page-table entries are scalar loads issued first.
  struct Buf {
    uint4 kr[U], vr[U];
    float ksc[U], vsc[U];
  };
  // Every call issues the same number of vector loads with no branch around
  // them (tokens past the chunk are clamped onto its last token, a cache
  // hit), so the compiler's wait counters keep the next iteration's loads in
  // flight while the current one is consumed.
  auto issue = [&](int g0, Buf& bf) {
    int64_t step_row[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // wave-uniform and inside the sequence; readfirstlane keeps it (and the
      // page-table read) on the scalar unit, off the vector-load counter
      const int tc = __builtin_amdgcn_readfirstlane(min(g0 + u * TPW, t1 - 1));
      if (a.page_table) {
        // read through the constant address space: a scalar (SMEM) load
        const auto* pt = (const __attribute__((address_space(4))) int32_t*)a.page_table;
        const int pg = pt[(int64_t)b * a.max_pages + (tc >> a.page_shift)];
        step_row[u] = (int64_t)pg * a.Hkv * a.page_size + hk_rows - (tc & ~(a.page_size - 1));
      } else {
        step_row[u] = (int64_t)b * a.Hkv * a.page_size + hk_rows;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = step_row[u] + min(g0 + u * TPW + slot, t1 - 1);
      bf.kr[u] = *(const uint4*)(kb + row * (D * EB) + lane_off);
      bf.vr[u] = *(const uint4*)(vb + row * (D * EB) + lane_off);
      if constexpr (KV == ATTN_INT8) {
        bf.ksc[u] = a.k_scale[row];  // q already carries scale*log2(e)
        bf.vsc[u] = a.v_scale[row];
      } else {
        bf.ksc[u] = bf.vsc[u] = 1.f;
      }
    }
  };
  auto consume = [&](int g0, const Buf& bf) {
    // scores of the U tokens of this lane's slot, in the log2 domain
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = g0 + u * TPW + slot < t1;
      if constexpr (kDot2) {
        const uint32_t wd[4] = {bf.kr[u].x, bf.kr[u].y, bf.kr[u].z, bf.kr[u].w};
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) d = __builtin_amdgcn_fdot2_f32_bf16(q2[g][i], __builtin_bit_cast(bf16x2, wd[i]), d, false);
          s[u][g] = d;
        }
      } else {
        float kv[EPL];
        decode16<KV>(bf.kr[u], kv);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) d = fmaf(qf[g][e], kv[e], d);
          s[u][g] = d;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float x = token_sum<LPT>(s[u][g]) * (KV == ATTN_INT8 ? bf.ksc[u] : smul);
        s[u][g] = ok ? x : -INFINITY;
      }
    }
    // online softmax over the slot's tokens, then accumulate P.V
    float vv[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) decode16<KV>(bf.vr[u], vv[u]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][g]);
      const float m_new = fmaxf(m[g], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[g] - m_use);
      m[g] = m_new;
      float lsum = 0.f;
      float p[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = __builtin_amdgcn_exp2f(s[u][g] - m_use);
        lsum += p[u];
        if constexpr (KV == ATTN_INT8) p[u] *= bf.vsc[u];
      }
      l[g] = l[g] * alpha + lsum;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float x = acc[g][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) x = fmaf(p[u], vv[u][e], x);
        acc[g][e] = x;
      }
    }
  };

  // two-stage software pipeline: the next iteration's loads are in flight
  // while the current one is consumed
  Buf b0, b1;
  int g0 = t0 + wu * TPI;
  // (the scheduling barriers keep the compiler from sinking a batch of loads
  // down to its consumer to save registers, which would serialise them)
  if (g0 < t1) {
    issue(g0, b0);
    while (true) {
      const int g1 = g0 + kStride;
      issue(g1, b1);
      __builtin_amdgcn_sched_barrier(0);
      consume(g0, b0);
      if (g1 >= t1) break;
      const int g2 = g1 + kStride;
      issue(g2, b0);
      __builtin_amdgcn_sched_barrier(0);
      consume(g1, b1);
      if (g2 >= t1) break;
      g0 = g2;
    }
  }

  // combine the token slots of the wave (lanes 16/32 apart hold the same d slice)
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float M = fmaxf(m[g], mo);
      const float Mu = M == -INFINITY ? 0.f : M;
      const float fs = __builtin_amdgcn_exp2f(m[g] - Mu), fo = __builtin_amdgcn_exp2f(mo - Mu);
      l[g] = l[g] * fs + lo * fo;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * fs + __shfl_xor(acc[g][e], off) * fo;
      m[g] = M;
    }
  }
  // combine the four waves through LDS
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_acc[w][g * D + part * EPL + e] = acc[g][e];
      if (part == 0) {
        red_m[w][g] = m[g];
        red_l[w][g] = l[g];
      }
    }
  }
  __syncthreads();
  float vmul = 1.f;
  if constexpr (KV == ATTN_FP8_E4M3) vmul = a.v_scale[hk];
  for (int idx = tid; idx < G * D; idx += 256) {
    const int g = idx / D;
    const float M = fmaxf(fmaxf(red_m[0][g], red_m[1][g]), fmaxf(red_m[2][g], red_m[3][g]));
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = red_m[ww][g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red_m[ww][g] - M);
      num = fmaf(f, red_acc[ww][idx], num);
      den = fmaf(f, red_l[ww][g], den);
    }
    a.part_o[((int64_t)split * BHq + row0 + g) * D + (idx - g * D)] = num * (vmul / den);
    if (idx - g * D == 0) a.part_lse[(int64_t)split * BHq + row0 + g] = (M + __log2f(den)) * kLn2;
  }
}

template <int KV, int D, int G>
attn_status launch_one(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.n_splits, a.Hkv, a.B);
  hipLaunchKernelGGL((decode_split_kernel<KV, D, G>), grid, dim3(256), 0, stream, a);
  return check_launch("decode_split");
}

template <int KV, int D>
attn_status launch_g(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_one<KV, D, 1>(a, stream);
    case 2: return launch_one<KV, D, 2>(a, stream);
    case 3: return launch_one<KV, D, 3>(a, stream);
    case 4: return launch_one<KV, D, 4>(a, stream);
    case 5: return launch_one<KV, D, 5>(a, stream);
    case 6: return launch_one<KV, D, 6>(a, stream);
    case 7: return launch_one<KV, D, 7>(a, stream);
    case 8: return launch_one<KV, D, 8>(a, stream);
  }
  return set_error(ATTN_E_UNSUPPORTED, "decode: query heads per KV head must be 1..8 (got %d)", G);
}

template <int KV>
attn_status launch_d(const DecodeArgs& a, int D, int G, hipStream_t stream) {
  return D == 128 ? launch_g<KV, 128>(a, G, stream) : launch_g<KV, 64>(a, G, stream);
}

}  // namespace

DecodePlan plan_decode(int B, int Hq, int Hkv, int max_kv_len, int num_splits) {
  DecodePlan p;
  int chunk;
  if (max_kv_len <= 0) {
    chunk = 16;
  } else if (num_splits > 0) {
    chunk = (max_kv_len + num_splits - 1) / num_splits;
  } else {
    const char* env = getenv("ATTN_DECODE_CHUNK");
    if (env && atoi(env) > 0) {
      chunk = atoi(env);
    } else {
      // enough chunks for ~4096 work-groups (16 per CU), never below 256 tokens each
      const int64_t target = 4096;
      const int64_t work = (int64_t)max_kv_len * std::max(B, 1) * std::max(Hkv, 1);
      chunk = (int)std::max<int64_t>(256, (work + target - 1) / target);
    }
  }
  chunk = (chunk + 15) / 16 * 16;
  p.chunk = chunk;
  p.n_splits = max_kv_len <= 0 ? 1 : (max_kv_len + chunk - 1) / chunk;
  return p;
}

size_t decode_workspace_bytes(int B, int Hq, int D, const DecodePlan& p) {
  const size_t rows = (size_t)p.n_splits * (size_t)B * (size_t)Hq;
  const size_t o_bytes = (rows * (size_t)D * sizeof(float) + 255) / 256 * 256;
  return o_bytes + (rows * sizeof(float) + 255) / 256 * 256;
}

attn_status launch_decode_split(attn_dtype kv_dt, const DecodeArgs& a, int D, int G, hipStream_t stream) {
  switch (kv_dt) {
    case ATTN_BF16: return launch_d<ATTN_BF16>(a, D, G, stream);
    case ATTN_FP8_E4M3: return launch_d<ATTN_FP8_E4M3>(a, D, G, stream);
    case ATTN_INT8: return launch_d<ATTN_INT8>(a, D, G, stream);
    default: break;
  }
  return set_error(ATTN_E_UNSUPPORTED, "decode: unsupported KV dtype %d", (int)kv_dt);
}

}  // namespace attn
