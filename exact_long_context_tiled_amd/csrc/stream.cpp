// Budgeted streaming prefill in the manner of Stream-CQSA (Stream-CQSA
// summary, "Methodology" items 2-4): exact attention split into independent
// (query block, key block) sub-tasks whose device footprint fits a
// caller-given budget; Q/K/V blocks stream from pinned host memory, each
// sub-task's partial result is merged by log-sum-exp into the resident output
// block, and finished output blocks stream back.  Device memory grows with the
// block sizes, not with the sequence length ("Results & findings").
//
// The plan is rectangular: every causally visible (query block, key block)
// pair is exactly one sub-task, fully masked pairs are never scheduled, and a
// query block that sees no key at all gets one sub-task with an empty key
// block (it writes O = 0, lse = -inf).  The block-size controller picks the
// pair (block_q, block_k) that fits the budget with the least host<->device
// traffic plus a fixed per-sub-task charge.
//
// Execution uses three HIP streams: an inbound copy stream (Q blocks and
// double-buffered K/V blocks), the compute stream (one prefill launch per
// sub-task, in accumulate mode after the first sub-task of a query block), and
// an outbound copy stream (O and lse blocks).  Query-side buffers are double
// buffered too, so the copy-out of one query block overlaps the next block's
// compute.  Events order the three streams; all device memory is one arena
// allocated at entry and freed before return.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <vector>

#include "common.h"
#include "stream_common.h"

namespace attn {

namespace streamx {

attn_status check_stream_sizes(attn_dtype dt, int B, int Hq, int Hkv, int64_t S, int64_t T, int D) {
  if (dt != ATTN_BF16 && dt != ATTN_F32) return set_error(ATTN_E_UNSUPPORTED, "stream: dtype must be bf16 or f32");
  if (D != 64 && D != 128) return set_error(ATTN_E_UNSUPPORTED, "stream: D must be 64 or 128 (got %d)", D);
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || S < 0 || T < 0)
    return set_error(ATTN_E_INVALID, "stream: invalid sizes");
  return ATTN_OK;
}

namespace {
bool is_pinned_host(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeHost;
}
}  // namespace

attn_status check_pinned(attn_dtype dt, const void* q, const void* k, const void* v, const float* o,
                         const float* lse, int B, int Hq, int Hkv, int64_t S, int64_t T, int D) {
  const int64_t es = elem_size(dt);
  struct {
    const void* p;
    int64_t bytes;
    const char* name;
  } hb[] = {{q, (int64_t)B * S * Hq * D * es, "q"},
            {k, (int64_t)B * T * Hkv * D * es, "k"},
            {v, (int64_t)B * T * Hkv * D * es, "v"},
            {o, (int64_t)B * S * Hq * D * 4, "o"},
            {lse, (int64_t)B * Hq * S * 4, "lse"}};
  for (auto& h : hb) {
    if (!h.p || h.bytes == 0) continue;
    if (!is_pinned_host(h.p) || !is_pinned_host((const char*)h.p + h.bytes - 1))
      return set_error(ATTN_E_INVALID, "stream: host buffer %s is not pinned host memory", h.name);
  }
  return ATTN_OK;
}

PrefillArgs block_args(const void* q, const void* k, const void* v, float* o, float* lse, int Hq, int Hkv, int D,
                       int64_t n_q, int64_t n_k, int64_t q_abs0, int64_t k_abs0, int causal, int accumulate,
                       float scale_log2) {
  PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.q_sb = 0;
  a.q_ss = (int64_t)Hq * D;
  a.k_sb = 0;
  a.k_ss = (int64_t)Hkv * D;
  a.o_sb = 0;
  a.o_ss = (int64_t)Hq * D;
  a.l_sb = 0;
  a.l_sh = n_q;
  a.n_q = n_q;
  a.n_k = n_k;
  a.q_abs0 = q_abs0;
  a.k_abs0 = k_abs0;
  a.B = 1;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.causal = causal;
  a.accumulate = accumulate;
  a.scale_log2 = scale_log2;
  return a;
}

}  // namespace streamx

namespace {

using streamx::align_up;
using streamx::elem_size;
using streamx::kAlign;
using streamx::kAllocSlack;

struct Plan {
  int64_t bq = 0, bk = 0;
  int64_t nqb = 0, nkb = 0;
  int64_t q_bytes = 0, o_bytes = 0, l_bytes = 0, kv_bytes = 0;  // one buffer each
  int64_t device_bytes = 0;
  int64_t tasks = 0, h2d = 0, d2h = 0;
};

// Key blocks visible to query block qb: [0, count).  0 means "no key at all".
int64_t visible_kblocks(const Plan& p, int64_t qb, int64_t S, int64_t T, int causal) {
  if (T == 0) return 0;
  if (!causal) return p.nkb;
  const int64_t q_hi = std::min(S, (qb + 1) * p.bq);
  const int64_t last = q_hi - 1 + (T - S);  // last key any row of the block sees
  if (last < 0) return 0;
  return std::min(p.nkb, last / p.bk + 1);
}

void fill_sizes(Plan& p, int Hq, int Hkv, int64_t S, int64_t T, int D, attn_dtype dt) {
  const int64_t es = elem_size(dt);
  p.q_bytes = align_up(p.bq * Hq * D * es);
  p.o_bytes = align_up(p.bq * Hq * D * 4);
  p.l_bytes = align_up(p.bq * Hq * 4);
  p.kv_bytes = align_up(p.bk * Hkv * D * es);
  p.device_bytes = 2 * (p.q_bytes + p.o_bytes + p.l_bytes) + 2 * 2 * p.kv_bytes;
  p.nqb = (S + p.bq - 1) / p.bq;
  p.nkb = T > 0 ? (T + p.bk - 1) / p.bk : 0;
}

void count_traffic(Plan& p, int B, int Hq, int Hkv, int64_t S, int64_t T, int D, int causal, attn_dtype dt) {
  const int64_t es = elem_size(dt);
  p.tasks = p.h2d = p.d2h = 0;
  for (int64_t qb = 0; qb < p.nqb; ++qb) {
    const int64_t nq = std::min(S, (qb + 1) * p.bq) - qb * p.bq;
    const int64_t nv = visible_kblocks(p, qb, S, T, causal);
    p.tasks += std::max<int64_t>(nv, 1);
    p.h2d += nq * Hq * D * es;
    for (int64_t kb = 0; kb < nv; ++kb) {
      const int64_t nk = std::min(T, (kb + 1) * p.bk) - kb * p.bk;
      p.h2d += 2 * nk * Hkv * D * es;
    }
    p.d2h += nq * Hq * D * 4 + nq * Hq * 4;
  }
  p.tasks *= B;
  p.h2d *= B;
  p.d2h *= B;
}

// Controller objective: bytes moved over the host link plus a fixed charge
// per sub-task (launch, synchronisation and the lower kernel efficiency of
// short key blocks), expressed in bytes.
constexpr int64_t kTaskCostBytes = 32ll << 20;
int64_t plan_cost(const Plan& p) { return p.h2d + p.d2h + p.tasks * kTaskCostBytes; }

attn_status make_plan(attn_dtype dt, int B, int Hq, int Hkv, int64_t S, int64_t T, int D, int causal,
                      size_t budget, int64_t force_q, int64_t force_k, Plan* out) {
  // keep room for the allocator's rounding of the one arena allocation
  const int64_t raw = budget > (size_t)INT64_MAX ? INT64_MAX : (int64_t)budget;
  const int64_t bud = streamx::usable_budget(budget);
  const int64_t tq = std::max<int64_t>(T, 1);
  auto try_plan = [&](int64_t bq, int64_t bk, Plan* p) {
    p->bq = bq;
    p->bk = bk;
    fill_sizes(*p, Hq, Hkv, S, T, D, dt);
    return p->device_bytes <= bud;
  };
  if (force_q > 0 || force_k > 0) {
    const int64_t bq = force_q > 0 ? std::min(force_q, S) : std::min<int64_t>(S, 4096);
    const int64_t bk = force_k > 0 ? std::min(force_k, tq) : std::min<int64_t>(tq, 4096);
    Plan p;
    if (!try_plan(bq, bk, &p))
      return set_error(ATTN_E_BUDGET, "stream: blocks q=%lld k=%lld need %lld device bytes > budget %lld",
                       (long long)bq, (long long)bk, (long long)(p.device_bytes + kAllocSlack), (long long)raw);
    count_traffic(p, B, Hq, Hkv, S, T, D, causal, dt);
    *out = p;
    return ATTN_OK;
  }
  // candidate key blocks: powers of two from min(T, 32768) down to 64
  bool found = false;
  Plan best;
  for (int64_t bk = std::min<int64_t>(tq, 32768); bk >= 1; bk = bk > 64 ? bk / 2 : 0) {
    Plan p;
    p.bq = 1;
    p.bk = bk;
    fill_sizes(p, Hq, Hkv, S, T, D, dt);
    const int64_t fixed = 4 * p.kv_bytes;
    const int64_t per_q = 2 * (Hq * D * elem_size(dt) + Hq * D * 4 + Hq * 4);
    if (bud <= fixed + 6 * kAlign) continue;
    int64_t bq = (bud - fixed - 6 * kAlign) / per_q;
    if (bq >= S) {
      bq = S;
    } else {
      bq = bq / 128 * 128;
      if (bq < std::min<int64_t>(S, 128)) continue;
    }
    while (bq > 0 && !try_plan(bq, bk, &p)) bq -= 128;  // alignment slack
    if (bq <= 0) continue;
    count_traffic(p, B, Hq, Hkv, S, T, D, causal, dt);
    if (!found || plan_cost(p) < plan_cost(best)) {
      best = p;
      found = true;
    }
    if (bk <= 64) break;
  }
  if (!found)
    return set_error(ATTN_E_BUDGET, "stream: no block sizes fit a device budget of %lld bytes", (long long)raw);
  *out = best;
  return ATTN_OK;
}

}  // namespace

}  // namespace attn

using namespace attn;

extern "C" attn_status attn_stream_plan(attn_dtype dt, int B, int Hq, int Hkv, int64_t S, int64_t T, int D,
                                        int causal, size_t device_budget_bytes, int64_t block_q, int64_t block_k,
                                        int64_t* tasks, int64_t cap, attn_stream_report* plan) {
  attn_status st = streamx::check_stream_sizes(dt, B, Hq, Hkv, S, T, D);
  if (st != ATTN_OK) return st;
  if (block_q < 0 || block_k < 0 || cap < 0) return set_error(ATTN_E_INVALID, "stream: invalid sizes");
  Plan p;
  if (B == 0 || S == 0) {
    if (plan) memset(plan, 0, sizeof(*plan));
    return ATTN_OK;
  }
  st = make_plan(dt, B, Hq, Hkv, S, T, D, causal, device_budget_bytes, block_q, block_k, &p);
  if (st != ATTN_OK) return st;
  if (tasks) {
    int64_t n = 0;
    for (int64_t b = 0; b < B; ++b)
      for (int64_t qb = 0; qb < p.nqb; ++qb) {
        const int64_t nv = visible_kblocks(p, qb, S, T, causal);
        for (int64_t kb = 0; kb < std::max<int64_t>(nv, 1); ++kb) {
          if (n < cap) {
            tasks[3 * n] = b;
            tasks[3 * n + 1] = qb;
            tasks[3 * n + 2] = nv == 0 ? -1 : kb;
          }
          ++n;
        }
      }
  }
  if (plan) {
    plan->tasks = p.tasks;
    plan->h2d_bytes = p.h2d;
    plan->d2h_bytes = p.d2h;
    plan->peak_device_bytes = p.device_bytes;
    plan->block_q = p.bq;
    plan->block_k = p.bk;
    plan->wall_s = plan->kernel_s = 0.0;
  }
  return ATTN_OK;
}

extern "C" attn_status attn_stream_budgeted(attn_dtype dt, const void* q_host, const void* k_host,
                                            const void* v_host, int B, int Hq, int Hkv, int64_t S, int64_t T, int D,
                                            int causal, float scale, size_t device_budget_bytes, int64_t block_q,
                                            int64_t block_k, float* o_host, float* lse_host,
                                            attn_stream_report* report) {
  const auto wall0 = std::chrono::steady_clock::now();
  attn_status st = streamx::check_stream_sizes(dt, B, Hq, Hkv, S, T, D);
  if (st != ATTN_OK) return st;
  if (block_q < 0 || block_k < 0) return set_error(ATTN_E_INVALID, "stream: invalid sizes");
  if (!std::isfinite(scale) || !(scale > 0.f)) return set_error(ATTN_E_INVALID, "stream: scale must be finite and > 0");
  if (B == 0 || S == 0) {
    if (report) memset(report, 0, sizeof(*report));
    return ATTN_OK;
  }
  if (!q_host || !o_host || (T > 0 && (!k_host || !v_host)))
    return set_error(ATTN_E_INVALID, "stream: null host pointer");
  const int64_t es = elem_size(dt);
  // every host buffer must be pinned (page-locked, device-mapped) memory
  st = streamx::check_pinned(dt, q_host, k_host, v_host, o_host, lse_host, B, Hq, Hkv, S, T, D);
  if (st != ATTN_OK) return st;
  Plan p;
  st = make_plan(dt, B, Hq, Hkv, S, T, D, causal, device_budget_bytes, block_q, block_k, &p);
  if (st != ATTN_OK) return st;

  // ---- resources
  char* arena = nullptr;
  hipStream_t s_in = nullptr, s_cmp = nullptr, s_out = nullptr;
  std::vector<hipEvent_t> evs;
  std::vector<hipEvent_t> timing;
  attn_status result = ATTN_OK;
  auto ev = [&](unsigned flags) {
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, flags) != hipSuccess) return (hipEvent_t) nullptr;
    evs.push_back(e);
    return e;
  };
#define ATTN_HIP(call)                                                                         \
  do {                                                                                         \
    hipError_t e_ = (call);                                                                    \
    if (e_ != hipSuccess) {                                                                    \
      result = set_error(ATTN_E_DEVICE, "stream: %s failed: %s", #call, hipGetErrorString(e_)); \
      goto done;                                                                               \
    }                                                                                          \
  } while (0)
  {
    ATTN_HIP(hipMalloc((void**)&arena, (size_t)p.device_bytes));
    ATTN_HIP(hipStreamCreateWithFlags(&s_in, hipStreamNonBlocking));
    ATTN_HIP(hipStreamCreateWithFlags(&s_cmp, hipStreamNonBlocking));
    ATTN_HIP(hipStreamCreateWithFlags(&s_out, hipStreamNonBlocking));
    char* cur = arena;
    char *qbuf[2], *obuf[2], *lbuf[2], *kbuf[2], *vbuf[2];
    for (int s = 0; s < 2; ++s) {
      qbuf[s] = cur, cur += p.q_bytes;
      obuf[s] = cur, cur += p.o_bytes;
      lbuf[s] = cur, cur += p.l_bytes;
    }
    for (int s = 0; s < 2; ++s) {
      kbuf[s] = cur, cur += p.kv_bytes;
      vbuf[s] = cur, cur += p.kv_bytes;
    }
    hipEvent_t ev_q[2], ev_done[2], ev_out[2], ev_kv[2], ev_kv_free[2];
    for (int s = 0; s < 2; ++s) {
      ev_q[s] = ev(hipEventDisableTiming);
      ev_done[s] = ev(hipEventDisableTiming);
      ev_out[s] = ev(hipEventDisableTiming);
      ev_kv[s] = ev(hipEventDisableTiming);
      ev_kv_free[s] = ev(hipEventDisableTiming);
      if (!ev_q[s] || !ev_done[s] || !ev_out[s] || !ev_kv[s] || !ev_kv_free[s]) {
        result = set_error(ATTN_E_DEVICE, "stream: event creation failed");
        goto done;
      }
    }
    const float scale_log2 = scale * kLog2e;
    int64_t job = 0, kv_use = 0;
    for (int64_t b = 0; b < B; ++b) {
      for (int64_t qb = 0; qb < p.nqb; ++qb, ++job) {
        const int s = (int)(job & 1);
        const int64_t q0 = qb * p.bq;
        const int64_t nq = std::min(S, q0 + p.bq) - q0;
        // inbound: Q block, once the slot's previous results have left
        if (job >= 2) ATTN_HIP(hipStreamWaitEvent(s_in, ev_out[s], 0));
        ATTN_HIP(hipMemcpyAsync(qbuf[s], (const char*)q_host + ((b * S + q0) * Hq * D) * es, nq * Hq * D * es,
                                hipMemcpyHostToDevice, s_in));
        ATTN_HIP(hipEventRecord(ev_q[s], s_in));
        ATTN_HIP(hipStreamWaitEvent(s_cmp, ev_q[s], 0));
        const int64_t nv = visible_kblocks(p, qb, S, T, causal);
        for (int64_t kb = 0; kb < std::max<int64_t>(nv, 1); ++kb) {
          PrefillArgs a = streamx::block_args(qbuf[s], nullptr, nullptr, (float*)obuf[s], (float*)lbuf[s], Hq, Hkv,
                                              D, nq, 0, q0 + (T - S), 0, causal, kb > 0, scale_log2);
          if (nv == 0) {  // no visible key: an empty key block writes O = 0, lse = -inf
            a.k = a.v = qbuf[s];
            a.n_k = 0;
            a.k_abs0 = 0;
          } else {
            const int u = (int)(kv_use & 1);
            const int64_t k0 = kb * p.bk;
            const int64_t nk = std::min(T, k0 + p.bk) - k0;
            if (kv_use >= 2) ATTN_HIP(hipStreamWaitEvent(s_in, ev_kv_free[u], 0));
            const size_t off = (size_t)((b * T + k0) * Hkv * D * es);
            ATTN_HIP(hipMemcpyAsync(kbuf[u], (const char*)k_host + off, nk * Hkv * D * es, hipMemcpyHostToDevice,
                                    s_in));
            ATTN_HIP(hipMemcpyAsync(vbuf[u], (const char*)v_host + off, nk * Hkv * D * es, hipMemcpyHostToDevice,
                                    s_in));
            ATTN_HIP(hipEventRecord(ev_kv[u], s_in));
            ATTN_HIP(hipStreamWaitEvent(s_cmp, ev_kv[u], 0));
            a.k = kbuf[u];
            a.v = vbuf[u];
            a.n_k = nk;
            a.k_abs0 = k0;
          }
          hipEvent_t t0 = ev(hipEventDefault), t1 = ev(hipEventDefault);
          if (!t0 || !t1) {
            result = set_error(ATTN_E_DEVICE, "stream: event creation failed");
            goto done;
          }
          timing.push_back(t0);
          timing.push_back(t1);
          ATTN_HIP(hipEventRecord(t0, s_cmp));
          st = dt == ATTN_BF16 ? launch_prefill_bf16(a, D, s_cmp) : launch_prefill_f32(a, D, s_cmp);
          if (st != ATTN_OK) {
            result = st;
            goto done;
          }
          ATTN_HIP(hipEventRecord(t1, s_cmp));
          if (nv > 0) {
            ATTN_HIP(hipEventRecord(ev_kv_free[kv_use & 1], s_cmp));
            ++kv_use;
          }
        }
        // outbound: O and lse of this query block
        ATTN_HIP(hipEventRecord(ev_done[s], s_cmp));
        ATTN_HIP(hipStreamWaitEvent(s_out, ev_done[s], 0));
        ATTN_HIP(hipMemcpyAsync((char*)o_host + (b * S + q0) * Hq * D * 4, obuf[s], nq * Hq * D * 4,
                                hipMemcpyDeviceToHost, s_out));
        if (lse_host)
          ATTN_HIP(hipMemcpy2DAsync((char*)lse_host + ((int64_t)b * Hq * S + q0) * 4, (size_t)S * 4, lbuf[s],
                                    (size_t)nq * 4, (size_t)nq * 4, (size_t)Hq, hipMemcpyDeviceToHost, s_out));
        ATTN_HIP(hipEventRecord(ev_out[s], s_out));
      }
    }
    ATTN_HIP(hipStreamSynchronize(s_in));
    ATTN_HIP(hipStreamSynchronize(s_cmp));
    ATTN_HIP(hipStreamSynchronize(s_out));
    double ksum = 0.0;
    for (size_t i = 0; i + 1 < timing.size(); i += 2) {
      float ms = 0.f;
      ATTN_HIP(hipEventElapsedTime(&ms, timing[i], timing[i + 1]));
      ksum += ms * 1e-3;
    }
    if (report) {
      report->tasks = p.tasks;
      report->h2d_bytes = p.h2d;
      report->d2h_bytes = p.d2h;
      report->peak_device_bytes = p.device_bytes;
      report->block_q = p.bq;
      report->block_k = p.bk;
      report->kernel_s = ksum;
    }
  }
done:
#undef ATTN_HIP
  // drain before releasing anything (error paths included)
  if (s_in) (void)hipStreamSynchronize(s_in);
  if (s_cmp) (void)hipStreamSynchronize(s_cmp);
  if (s_out) (void)hipStreamSynchronize(s_out);
  for (hipEvent_t e : evs) (void)hipEventDestroy(e);
  if (s_in) (void)hipStreamDestroy(s_in);
  if (s_cmp) (void)hipStreamDestroy(s_cmp);
  if (s_out) (void)hipStreamDestroy(s_out);
  if (arena) (void)hipFree(arena);
  if (result == ATTN_OK && report)
    report->wall_s = std::chrono::duration<double>(std::chrono::steady_clock::now() - wall0).count();
  return result;
}
