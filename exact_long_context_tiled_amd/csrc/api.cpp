// C ABI of libattn.so: argument validation and dispatch to the HIP kernels.
// Every check happens before anything is launched, so a call that returns an
// error status has written nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "common.h"

namespace attn {

namespace {
thread_local char g_err[512] = "";
}

attn_status set_error(attn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

attn_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(ATTN_E_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ATTN_OK;
}

int device_cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

attn_status raise_lds_limit(const void* kernel, size_t bytes, std::atomic<size_t>* raised) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(ATTN_E_DEVICE, "cannot query the current device");
  size_t cur = raised[dev].load(std::memory_order_acquire);
  if (bytes <= cur) return ATTN_OK;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
    return set_error(ATTN_E_DEVICE, "cannot raise the dynamic LDS limit to %zu bytes", bytes);
  // keep the largest limit set (another thread may have raised it further meanwhile)
  while (cur < bytes && !raised[dev].compare_exchange_weak(cur, bytes, std::memory_order_acq_rel)) {
  }
  return ATTN_OK;
}

namespace {
std::atomic<int> g_dec_path{0}, g_dec_units{0};
std::atomic<int64_t> g_dec_piece{-1};
}  // namespace

DecodeTuning decode_tuning() {
  return DecodeTuning{g_dec_path.load(std::memory_order_relaxed), g_dec_units.load(std::memory_order_relaxed),
                      g_dec_piece.load(std::memory_order_relaxed)};
}

}  // namespace attn

using namespace attn;

extern "C" attn_status attn_decode_set_tuning(int path, int units, int64_t piece_bytes) {
  if (path != 0 && path != 1) return set_error(ATTN_E_INVALID, "decode tuning: path must be 0 or 1 (got %d)", path);
  if (units < 0 || units > kDecodeMaxAutoUnits)
    return set_error(ATTN_E_INVALID, "decode tuning: units must be in 0..%d (got %d)", kDecodeMaxAutoUnits, units);
  g_dec_path.store(path, std::memory_order_relaxed);
  g_dec_units.store(units, std::memory_order_relaxed);
  g_dec_piece.store(piece_bytes < 0 ? -1 : piece_bytes, std::memory_order_relaxed);
  return ATTN_OK;
}

extern "C" const char* attn_last_error(void) { return g_err; }

namespace {

bool aligned(const void* p, uintptr_t bytes) { return ((uintptr_t)p & (bytes - 1)) == 0; }

// Arguments of a whole-sequence prefill ([B, S, Hq, D] queries against
// [B, T, Hkv, D] keys); validation shared by the bf16 / fp32 and fp8 calls.
attn_status prefill_args(const char* what, const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                         int64_t S, int64_t T, int D, int causal, float scale, float* o, float* lse, PrefillArgs* out,
                         bool* nothing) {
  *nothing = false;
  if (D != 64 && D != 128) return set_error(ATTN_E_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", what, D);
  if (B < 0 || S < 0 || T < 0 || Hq <= 0 || Hkv <= 0)
    return set_error(ATTN_E_INVALID, "%s: negative or zero sizes (B=%d Hq=%d Hkv=%d S=%lld T=%lld)", what, B, Hq,
                     Hkv, (long long)S, (long long)T);
  if (Hq % Hkv) return set_error(ATTN_E_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", what, Hq, Hkv);
  if (causal != 0 && causal != 1) return set_error(ATTN_E_INVALID, "%s: causal must be 0 or 1", what);
  // the kernels scale the row max of the raw scores, which needs scale > 0
  if (!isfinite(scale) || !(scale > 0.f)) return set_error(ATTN_E_INVALID, "%s: scale must be finite and > 0", what);
  if (B > 65535 || Hkv > 65535) return set_error(ATTN_E_UNSUPPORTED, "%s: B and Hkv must be <= 65535", what);
  if (B == 0 || S == 0) {
    *nothing = true;
    return ATTN_OK;
  }
  if (!q || !o || (T > 0 && (!k || !v))) return set_error(ATTN_E_INVALID, "%s: null device pointer", what);
  // 16-byte vector loads of Q, direct 16-byte copies of K/V, 16-byte O stores
  if (!aligned(q, 16) || !aligned(o, 16) || (T > 0 && (!aligned(k, 16) || !aligned(v, 16))))
    return set_error(ATTN_E_INVALID, "%s: q, k, v and o must be 16-byte aligned", what);
  if (!aligned(lse, 4)) return set_error(ATTN_E_INVALID, "%s: lse must be 4-byte aligned", what);
  PrefillArgs a{};
  a.q = q;
  a.k = T > 0 ? k : q;
  a.v = T > 0 ? v : q;
  a.o = o;
  a.lse = lse;
  a.q_ss = (int64_t)Hq * D;
  a.q_sb = S * a.q_ss;
  a.k_ss = (int64_t)Hkv * D;
  a.k_sb = T * a.k_ss;
  a.o_ss = a.q_ss;
  a.o_sb = a.q_sb;
  a.l_sh = S;
  a.l_sb = (int64_t)Hq * S;
  a.n_q = S;
  a.n_k = T;
  a.q_abs0 = T - S;
  a.k_abs0 = 0;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.causal = causal;
  a.accumulate = 0;
  a.scale_log2 = scale * kLog2e;
  *out = a;
  return ATTN_OK;
}

}  // namespace

extern "C" attn_status attn_prefill(attn_dtype dt, const void* q, const void* k, const void* v, int B, int Hq,
                                    int Hkv, int64_t S, int64_t T, int D, int causal, float scale, float* o,
                                    float* lse, void* stream) {
  if (dt != ATTN_BF16 && dt != ATTN_F32)
    return set_error(ATTN_E_UNSUPPORTED, "prefill: dtype must be ATTN_BF16 or ATTN_F32 (got %d)", (int)dt);
  PrefillArgs a;
  bool nothing;
  attn_status st = prefill_args("prefill", q, k, v, B, Hq, Hkv, S, T, D, causal, scale, o, lse, &a, &nothing);
  if (st != ATTN_OK || nothing) return st;
  return dt == ATTN_BF16 ? launch_prefill_bf16(a, D, (hipStream_t)stream)
                         : launch_prefill_f32(a, D, (hipStream_t)stream);
}

extern "C" attn_status attn_prefill_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                        const float* k_scale, const float* v_scale, int B, int Hq, int Hkv,
                                        int64_t S, int64_t T, int D, int causal, float scale, float* o, float* lse,
                                        void* stream) {
  PrefillArgs a;
  bool nothing;
  attn_status st = prefill_args("prefill_fp8", q, k, v, B, Hq, Hkv, S, T, D, causal, scale, o, lse, &a, &nothing);
  if (st != ATTN_OK || nothing) return st;
  if (!q_scale || !k_scale || !v_scale) return set_error(ATTN_E_INVALID, "prefill_fp8: null scale pointer");
  if (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return set_error(ATTN_E_INVALID, "prefill_fp8: scales must be 4-byte aligned");
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return launch_prefill_fp8(a, D, (hipStream_t)stream);
}

namespace {

constexpr int kDecodeMaxQueryTokens = 64;

size_t decode_ws(int B, int Hq, int Hkv, int D, int n_q, int max_kv_len, int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || n_q <= 0 || max_kv_len < 0 || num_splits < 0 || Hq % Hkv) return 0;
  return decode_workspace_bytes(B, Hkv, n_q * (Hq / Hkv), D, num_splits > 0 ? num_splits : kDecodeMaxAutoUnits);
}

// Scratch of the allocation-free decode entry point: a static device array
// (one copy per GPU, resident for the life of the process), found per
// device through hipGetSymbolAddress.  Host code never uses the array's name
// as an address: that is a host-side stand-in.
constexpr size_t kNoAllocScratchBytes = 8u << 20;
static __device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up once per device).
attn_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(ATTN_E_DEVICE, "decode_noalloc: cannot query the current device");
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return set_error(ATTN_E_DEVICE, "decode_noalloc: no address for the scratch array: %s", hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ATTN_OK;
}

// use_scratch: the workspace is the device's static scratch array (the
// workspace arguments are ignored), for callers that cannot allocate.
attn_status decode_impl(attn_dtype kv_dt, const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale, const int32_t* page_table, int max_pages,
                        int page_size, int num_pages, const int32_t* kv_lens, int max_kv_len, int B, int n_q, int Hq,
                        int Hkv, int D, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                        float* o, float* lse, void* stream, bool use_scratch = false) {
  if (kv_dt != ATTN_BF16 && kv_dt != ATTN_INT8 && kv_dt != ATTN_FP8_E4M3 && kv_dt != ATTN_INT4)
    return set_error(ATTN_E_UNSUPPORTED, "decode: KV dtype must be bf16, int8, fp8 e4m3 or int4 (got %d)",
                     (int)kv_dt);
  if (D != 64 && D != 128) return set_error(ATTN_E_UNSUPPORTED, "decode: D must be 64 or 128 (got %d)", D);
  if (B < 0 || Hq <= 0 || Hkv <= 0 || max_kv_len < 0 || num_splits < 0 || n_q <= 0)
    return set_error(ATTN_E_INVALID, "decode: invalid sizes");
  if (n_q > kDecodeMaxQueryTokens)
    return set_error(ATTN_E_UNSUPPORTED, "decode: at most %d query tokens per sequence (got %d)",
                     kDecodeMaxQueryTokens, n_q);
  if (Hq % Hkv) return set_error(ATTN_E_INVALID, "decode: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G > 8) return set_error(ATTN_E_UNSUPPORTED, "decode: at most 8 query heads per KV head (got %d)", G);
  if (!isfinite(scale) || !(scale > 0.f)) return set_error(ATTN_E_INVALID, "decode: scale must be finite and > 0");
  if (num_splits > kDecodeMaxUnits)
    return set_error(ATTN_E_UNSUPPORTED, "decode: at most %d work units (got %d)", kDecodeMaxUnits, num_splits);
  if (B > 4095) return set_error(ATTN_E_UNSUPPORTED, "decode: at most 4095 sequences per call (got %d)", B);
  if (B == 0) return ATTN_OK;
  if (!q || !k_cache || !v_cache || !kv_lens || !o) return set_error(ATTN_E_INVALID, "decode: null device pointer");
  if (kv_dt != ATTN_BF16 && (!k_scale || !v_scale))
    return set_error(ATTN_E_INVALID, "decode: quantised KV needs k_scale and v_scale");
  // 16-byte vector loads of q and of the caches
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return set_error(ATTN_E_INVALID, "decode: q, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(o, 4) || !aligned(lse, 4) || !aligned(kv_lens, 4) || !aligned(page_table, 4) ||
      !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return set_error(ATTN_E_INVALID, "decode: o, lse, kv_lens, page_table and scales must be 4-byte aligned");
  int shift = 0;
  if (page_table) {
    if (page_size < 16 || (page_size & (page_size - 1)))
      return set_error(ATTN_E_INVALID, "decode: paged mode needs a power-of-two page_size >= 16 (got %d)",
                       page_size);
    if (max_pages <= 0 || num_pages <= 0) return set_error(ATTN_E_INVALID, "decode: max_pages/num_pages must be > 0");
    if ((int64_t)max_pages * page_size < max_kv_len)
      return set_error(ATTN_E_INVALID, "decode: max_kv_len %d exceeds max_pages*page_size", max_kv_len);
    while ((1 << shift) < page_size) ++shift;
  } else {
    if (page_size < max_kv_len)
      return set_error(ATTN_E_INVALID, "decode: contiguous cache needs page_size >= max_kv_len");
  }
  // split positions (groups plus the per-segment charge) times unit counts
  // must stay inside int64
  const double groups = (double)B * Hkv * ((max_kv_len + kDecodeGroup - 1) / kDecodeGroup + kDecodeMaxPieceGroups);
  if (groups * (num_splits > 0 ? num_splits : kDecodeMaxAutoUnits) > 4e18)
    return set_error(ATTN_E_UNSUPPORTED, "decode: batch too large");
  const size_t need = decode_ws(B, Hq, Hkv, D, n_q, max_kv_len, num_splits);
  if (use_scratch) {
    if (need > kNoAllocScratchBytes)
      return set_error(ATTN_E_UNSUPPORTED,
                       "decode_noalloc: these sizes need %zu bytes of scratch; the static scratch holds %zu",
                       need, kNoAllocScratchBytes);
    attn_status st = scratch_of_current_device(&workspace);
    if (st != ATTN_OK) return st;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (!workspace || workspace_bytes < need)
    return set_error(ATTN_E_INVALID, "decode: workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (((uintptr_t)workspace) & 255) return set_error(ATTN_E_INVALID, "decode: workspace must be 256-byte aligned");
  DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.num_pages = page_table ? num_pages : 0;
  a.page_size = page_size;
  a.page_shift = shift;
  a.kv_lens = kv_lens;
  a.max_kv_len = max_kv_len;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_q = n_q;
  a.n_units = num_splits;
  a.scale_log2 = scale * kLog2e;
  const size_t segs = (size_t)B * Hkv;
  const size_t rec_bytes =
      ((size_t)((num_splits > 0 ? num_splits : kDecodeMaxAutoUnits) + segs) * decode_record_floats(n_q * G, D) *
           sizeof(float) + 255) / 256 * 256;
  a.part = (float*)workspace;
  a.seg_info = (int32_t*)((char*)workspace + rec_bytes);
  a.o = o;
  a.lse = lse;
  return launch_decode(kv_dt, a, D, G, (hipStream_t)stream);
}

}  // namespace

extern "C" size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_kv_len, int num_splits) {
  return decode_ws(B, Hq, Hkv, D, 1, max_kv_len, num_splits);
}

extern "C" attn_status attn_decode_splitkv(attn_dtype kv_dt, const void* q, const void* k_cache,
                                           const void* v_cache, const float* k_scale, const float* v_scale,
                                           const int32_t* page_table, int max_pages, int page_size, int num_pages,
                                           const int32_t* kv_lens, int max_kv_len, int B, int Hq, int Hkv, int D,
                                           float scale, int num_splits, void* workspace, size_t workspace_bytes,
                                           float* o, float* lse, void* stream) {
  return decode_impl(kv_dt, q, k_cache, v_cache, k_scale, v_scale, page_table, max_pages, page_size, num_pages,
                     kv_lens, max_kv_len, B, 1, Hq, Hkv, D, scale, num_splits, workspace, workspace_bytes, o, lse,
                     stream);
}

extern "C" attn_status attn_decode_splitkv_noalloc(attn_dtype kv_dt, const void* q, const void* k_cache,
                                                   const void* v_cache, const float* k_scale, const float* v_scale,
                                                   const int32_t* page_table, int max_pages, int page_size,
                                                   int num_pages, const int32_t* kv_lens, int max_kv_len, int B,
                                                   int Hq, int Hkv, int D, float scale, int num_splits, float* o,
                                                   float* lse, void* stream) {
  return decode_impl(kv_dt, q, k_cache, v_cache, k_scale, v_scale, page_table, max_pages, page_size, num_pages,
                     kv_lens, max_kv_len, B, 1, Hq, Hkv, D, scale, num_splits, nullptr, 0, o, lse, stream, true);
}

extern "C" size_t attn_decode_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

extern "C" size_t attn_decode_multi_workspace_size(int B, int n_q, int Hq, int Hkv, int D, int max_kv_len,
                                                   int num_splits) {
  return decode_ws(B, Hq, Hkv, D, n_q, max_kv_len, num_splits);
}

extern "C" attn_status attn_decode_multi(attn_dtype kv_dt, const void* q, const void* k_cache, const void* v_cache,
                                         const float* k_scale, const float* v_scale, const int32_t* page_table,
                                         int max_pages, int page_size, int num_pages, const int32_t* kv_lens,
                                         int max_kv_len, int B, int n_q, int Hq, int Hkv, int D, float scale,
                                         int num_splits, void* workspace, size_t workspace_bytes, float* o,
                                         float* lse, void* stream) {
  return decode_impl(kv_dt, q, k_cache, v_cache, k_scale, v_scale, page_table, max_pages, page_size, num_pages,
                     kv_lens, max_kv_len, B, n_q, Hq, Hkv, D, scale, num_splits, workspace, workspace_bytes, o, lse,
                     stream);
}

extern "C" attn_status attn_merge_partials(int n, const float* o_parts, const float* lse_parts, int64_t R, int D,
                                           float* o, float* lse, void* stream) {
  if (n < 0 || R < 0) return set_error(ATTN_E_INVALID, "merge: negative sizes");
  if (D < 1 || D > 1024) return set_error(ATTN_E_UNSUPPORTED, "merge: D must be in 1..1024 (got %d)", D);
  if (R == 0) return ATTN_OK;
  if (!o || (n > 0 && (!o_parts || !lse_parts))) return set_error(ATTN_E_INVALID, "merge: null device pointer");
  if (!aligned(o, 4) || !aligned(lse, 4) || !aligned(o_parts, 4) || !aligned(lse_parts, 4))
    return set_error(ATTN_E_INVALID, "merge: pointers must be 4-byte aligned");
  return launch_merge(n, o_parts, lse_parts, R, D, o, lse, (hipStream_t)stream);
}
