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
// This is a bandwidth-bound scan, so the vector ALUs do the arithmetic: the
// lanes of a wave are split into token slots of D*bytes/16 lanes, each lane
// owning one 16-byte slice of a K (then V) row.
//   pass 1: scores s[t][g] = scale * q_g . k_t  (slice dot + lane reduction)
//           into LDS;
//   stats : per head the chunk max m_g and sum l_g of exp(s - m_g);
//   pass 2: acc_g += p[t][g] * v_t over the chunk, then a reduction over
//           token slots and waves.
#include <math.h>

#include <algorithm>

#include "common.h"

namespace attn {
namespace {

constexpr int kMaxChunkScores = 8192;  // chunk * G floats of scores in LDS

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

template <int KV, int D, int G>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
  constexpr int EB = KvTraits<KV>::kBytes;
  constexpr int EPL = 16 / EB;     // elements per lane slice
  constexpr int LPT = D / EPL;     // lanes per token
  constexpr int TPW = 64 / LPT;    // tokens per wave step
  constexpr int TPB = 4 * TPW;     // tokens per work-group step
  constexpr int U = 4;             // steps unrolled (loads in flight)
  extern __shared__ float smem[];
  float* sc = smem;  // [sub_chunk][G]; reused for the final reduction
  __shared__ float stat_m[G], stat_l[G], stat_a[G];

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
  if (tid < G) {
    stat_m[tid] = -INFINITY;
    stat_l[tid] = 0.f;
  }

  // query slice, pre-multiplied by scale*log2(e) (and the fp8 K scale)
  float qs[G][EPL];
  {
    float qmul = a.scale_log2;
    if constexpr (KV == ATTN_FP8_E4M3) qmul *= a.k_scale[hk];
    const uint16_t* qb = (const uint16_t*)a.q + row0 * D + part * EPL;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; e += 8) {
        const uint4 raw = *(const uint4*)(qb + (int64_t)g * D + e);
        float tmp[8];
        decode16<ATTN_BF16>(raw, tmp);
#pragma unroll
        for (int i = 0; i < 8; ++i) qs[g][e + i] = tmp[i] * qmul;
      }
    }
  }

  const uint8_t* kb = (const uint8_t*)a.k;
  const uint8_t* vb = (const uint8_t*)a.v;
  const int my_off = w * TPW + slot;
  const int sub = a.sub_chunk;  // tokens whose scores fit in LDS at once

  float acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;

  // A chunk longer than `sub` is scanned in sub-chunks with an online
  // rescale of the running (max, sum, accumulator) between them.
  for (int s0 = t0; s0 < t1; s0 += sub) {
    const int s1 = min(t1, s0 + sub);
    const int ns = s1 - s0;
    // ---------------- pass 1: scores
    for (int tb = s0; tb < s1; tb += U * TPB) {
      uint4 raw[U];
      int64_t crow[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = tb + u * TPB + my_off;
        raw[u] = uint4{0, 0, 0, 0};
        crow[u] = 0;
        if (t < s1) {
          crow[u] = cache_row(a, b, hk, t);
          raw[u] = *(const uint4*)(kb + (crow[u] * D + part * EPL) * EB);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = tb + u * TPB + my_off;
        float kv[EPL];
        decode16<KV>(raw[u], kv);
        float dot[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc_s = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc_s = fmaf(qs[g][e], kv[e], acc_s);
          dot[g] = acc_s;
        }
#pragma unroll
        for (int off = 1; off < LPT; off <<= 1) {
#pragma unroll
          for (int g = 0; g < G; ++g) dot[g] += __shfl_xor(dot[g], off);
        }
        if (part == 0 && t < s1) {
          float ks = 1.f;
          if constexpr (KV == ATTN_INT8) ks = a.k_scale[crow[u]];
#pragma unroll
          for (int g = 0; g < G; ++g) sc[(t - s0) * G + g] = dot[g] * ks;
        }
      }
    }
    __syncthreads();

    // ---------------- softmax statistics of the sub-chunk, one wave per head
    for (int g = w; g < G; g += 4) {
      float mx = -INFINITY;
      for (int i = lane; i < ns; i += 64) mx = fmaxf(mx, sc[i * G + g]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_old = stat_m[g];  // -inf before the first sub-chunk
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.f;
      for (int i = lane; i < ns; i += 64) {
        const float p = __builtin_amdgcn_exp2f(sc[i * G + g] - m_new);
        sc[i * G + g] = p;
        sum += p;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
      if (lane == 0) {
        const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);
        stat_a[g] = alpha;
        stat_l[g] = stat_l[g] * alpha + sum;
        stat_m[g] = m_new;
      }
    }
    __syncthreads();

    // ---------------- pass 2: P.V
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float alpha = stat_a[g];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
    }
    for (int tb = s0; tb < s1; tb += U * TPB) {
      uint4 raw[U];
      int64_t crow[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = tb + u * TPB + my_off;
        raw[u] = uint4{0, 0, 0, 0};
        crow[u] = 0;
        if (t < s1) {
          crow[u] = cache_row(a, b, hk, t);
          raw[u] = *(const uint4*)(vb + (crow[u] * D + part * EPL) * EB);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = tb + u * TPB + my_off;
        if (t < s1) {
          float vv[EPL];
          decode16<KV>(raw[u], vv);
          float vsc = 1.f;
          if constexpr (KV == ATTN_INT8) vsc = a.v_scale[crow[u]];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float p = sc[(t - s0) * G + g] * vsc;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, vv[e], acc[g][e]);
          }
        }
      }
    }
    __syncthreads();  // sc is rewritten by the next sub-chunk
  }
  // reduce over the token slots of the wave (lanes with equal `part`)
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] += __shfl_xor(acc[g][e], off);
  }
  float* red = smem;  // [4][G*D]; the last sub-chunk's scores are dead
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[w * G * D + g * D + part * EPL + e] = acc[g][e];
  }
  __syncthreads();
  float vmul = 1.f;
  if constexpr (KV == ATTN_FP8_E4M3) vmul = a.v_scale[hk];
  for (int idx = tid; idx < G * D; idx += 256) {
    const int g = idx / D;
    const float s = red[idx] + red[G * D + idx] + red[2 * G * D + idx] + red[3 * G * D + idx];
    a.part_o[((int64_t)split * BHq + row0 + g) * D + (idx - g * D)] = s * (vmul / stat_l[g]);
  }
  if (tid < G)
    a.part_lse[(int64_t)split * BHq + row0 + tid] = (stat_m[tid] + __log2f(stat_l[tid])) * kLn2;
}

template <int KV, int D, int G>
attn_status launch_one(const DecodeArgs& a, hipStream_t stream) {
  const size_t smem = sizeof(float) * (size_t)std::max(a.sub_chunk * G, 4 * G * D);
  dim3 grid(a.n_splits, a.Hkv, a.B);
  hipLaunchKernelGGL((decode_split_kernel<KV, D, G>), grid, dim3(256), smem, stream, a);
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
  const int G = Hkv > 0 ? std::max(Hq / Hkv, 1) : 1;
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
      // enough chunks for ~2048 work-groups, never below 128 tokens each
      const int64_t target = 2048;
      const int64_t work = (int64_t)max_kv_len * std::max(B, 1) * std::max(Hkv, 1);
      chunk = (int)std::max<int64_t>(128, (work + target - 1) / target);
    }
  }
  chunk = (chunk + 15) / 16 * 16;
  p.chunk = chunk;
  p.sub_chunk = std::min(chunk, std::max(16, kMaxChunkScores / G / 16 * 16));
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
