// Budgeted streaming prefill over cyclic quorums (Stream-CQSA summary,
// "Methodology" items 1-3: the CQS Divide).
//
// Query and key positions are cut into the same number N of blocks (block x
// holds queries [x*bq, (x+1)*bq) and keys [x*bk, (x+1)*bk)).  A base quorum
// D = {d_0 = 0, d_1, ..., d_{k-1}} is a planar difference set modulo N: every
// nonzero residue is d_a - d_b for exactly one ordered pair (a, b).  Quorum i
// is D + i (mod N); any two quorums intersect (the quorum property) and
// quorum i holds the ordered block pair (x, y), x != y, for exactly one i,
// namely i = x - d_a where d_a - d_b = x - y.  The diagonal pair (x, x) lies
// in every quorum through x and is taken by quorum i = x (a = b = 0).  So the
// N quorum sub-tasks compute every (query block, key block) pair exactly
// once; causally invisible pairs are dropped, and a query block that sees no
// key at all gets one empty pair in sub-task x (it writes O = 0, lse = -inf).
//
// One sub-task = one quorum of one sequence: the Q/K/V blocks of its members
// are copied in, each of its pairs is one prefill launch merged by
// log-sum-exp into the query block's (O, lse), and the touched (O, lse)
// blocks go back to host memory.  A query block's running (O, lse) lives in
// the caller's host output between sub-tasks and is copied in again by the
// next sub-task that adds pairs to it (the host swap of intermediates in the
// streaming scheduler).  Two sub-task slots are double-buffered across three
// HIP streams (in-copies, compute, out-copies); a block whose running result
// was written back by the immediately preceding sub-task is copied in last,
// after that write-back has finished.
//
// Planar difference sets come from Singer's construction for prime p: with
// x primitive in GF(p^3) = GF(p)[x]/(f), the exponents i in [0, p^2+p+1)
// whose x^i has a zero constant coefficient form a difference set of p + 1
// residues modulo p^2 + p + 1 (the points of one line of the projective
// plane PG(2, p)).  N = 1 (one block) and N = 3 ({0, 1}) are the trivial
// cases.
#include <string.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <mutex>
#include <vector>

#include "common.h"
#include "stream_common.h"

namespace attn {
namespace {

using streamx::align_up;
using streamx::elem_size;

constexpr int kMaxPrime = 127;  // largest p used: N = 16257, quorums of 128 blocks

bool is_prime(int p) {
  if (p < 2) return false;
  for (int d = 2; d * d <= p; ++d)
    if (p % d == 0) return false;
  return true;
}

// Supported N in increasing order, with their quorum sizes.
struct CqsSize {
  int64_t n;
  int k;
  int p;  // 0 for the trivial sizes
};
const std::vector<CqsSize>& cqs_sizes() {
  static const std::vector<CqsSize> sizes = [] {
    std::vector<CqsSize> v{{1, 1, 0}, {3, 2, 0}};
    for (int p = 2; p <= kMaxPrime; ++p)
      if (is_prime(p)) v.push_back({(int64_t)p * p + p + 1, p + 1, p});
    return v;
  }();
  return sizes;
}

// Arithmetic in GF(p)[x]/(f), f = x^3 - c2 x^2 - c1 x - c0; elements are
// coefficient triples (a0, a1, a2) of a0 + a1 x + a2 x^2.
struct Cubic {
  int64_t p, c0, c1, c2;
  void mul(const int64_t* a, const int64_t* b, int64_t* r) const {
    int64_t t[5] = {0, 0, 0, 0, 0};
    for (int i = 0; i < 3; ++i)
      for (int j = 0; j < 3; ++j) t[i + j] = (t[i + j] + a[i] * b[j]) % p;
    for (int d = 4; d >= 3; --d) {  // x^d = x^(d-3) (c2 x^2 + c1 x + c0)
      t[d - 1] = (t[d - 1] + t[d] * c2) % p;
      t[d - 2] = (t[d - 2] + t[d] * c1) % p;
      t[d - 3] = (t[d - 3] + t[d] * c0) % p;
    }
    r[0] = t[0], r[1] = t[1], r[2] = t[2];
  }
  bool x_pow_is_one(int64_t e) const {
    int64_t r[3] = {1, 0, 0}, b[3] = {0, 1, 0};
    for (; e > 0; e >>= 1) {
      if (e & 1) mul(r, b, r);
      mul(b, b, b);
    }
    return r[0] == 1 && r[1] == 0 && r[2] == 0;
  }
};

// Singer difference set for prime p, shifted so that it starts at 0, sorted.
// x has order exactly p^3 - 1 (so f is irreducible and x primitive) iff
// x^(p^3-1) = 1 and x^((p^3-1)/r) != 1 for every prime r dividing p^3 - 1.
bool singer_set(int p, std::vector<int64_t>* out) {
  const int64_t n = (int64_t)p * p + p + 1;
  const int64_t order = (int64_t)p * p * p - 1;
  std::vector<int64_t> primes;
  {
    int64_t m = order;
    for (int64_t r = 2; r * r <= m; ++r)
      if (m % r == 0) {
        primes.push_back(r);
        while (m % r == 0) m /= r;
      }
    if (m > 1) primes.push_back(m);
  }
  for (int64_t c0 = 1; c0 < p; ++c0)
    for (int64_t c1 = 0; c1 < p; ++c1)
      for (int64_t c2 = 0; c2 < p; ++c2) {
        const Cubic f{p, c0, c1, c2};
        if (!f.x_pow_is_one(order)) continue;
        bool primitive = true;
        for (int64_t r : primes) primitive = primitive && !f.x_pow_is_one(order / r);
        if (!primitive) continue;
        // exponents e in [0, N) with a zero constant coefficient of x^e
        std::vector<int64_t> d;
        int64_t a[3] = {1, 0, 0};
        const int64_t xx[3] = {0, 1, 0};
        for (int64_t e = 0; e < n; ++e) {
          if (a[0] == 0) d.push_back(e);
          f.mul(a, xx, a);
        }
        if ((int)d.size() != p + 1) return false;
        const int64_t s = d[0];
        for (auto& e : d) e -= s;
        std::sort(d.begin(), d.end());
        *out = d;
        return true;
      }
  return false;
}

// Every nonzero residue modulo n is a difference of exactly one ordered pair.
bool is_planar_difference_set(const std::vector<int64_t>& d, int64_t n) {
  std::vector<int> seen((size_t)n, 0);
  for (size_t a = 0; a < d.size(); ++a)
    for (size_t b = 0; b < d.size(); ++b)
      if (a != b) ++seen[(size_t)(((d[a] - d[b]) % n + n) % n)];
  for (int64_t r = 1; r < n; ++r)
    if (seen[(size_t)r] != 1) return false;
  return seen[0] == 0;
}

attn_status base_quorum(const CqsSize& c, std::vector<int64_t>* out) {
  static std::mutex mu;
  static std::vector<std::pair<int64_t, std::vector<int64_t>>> cache;
  std::lock_guard<std::mutex> lock(mu);
  for (auto& e : cache)
    if (e.first == c.n) {
      *out = e.second;
      return ATTN_OK;
    }
  std::vector<int64_t> d;
  if (c.n == 1) d = {0};
  else if (c.n == 3) d = {0, 1};
  else if (!singer_set(c.p, &d) || !is_planar_difference_set(d, c.n))
    return set_error(ATTN_E_DEVICE, "stream_cqs: no difference set for N = %lld", (long long)c.n);
  cache.push_back({c.n, d});
  *out = d;
  return ATTN_OK;
}

struct CqsPlan {
  int64_t n = 0, k = 0;
  std::vector<int64_t> base;
  int64_t bq = 0, bk = 0;
  int64_t q_bytes = 0, o_bytes = 0, l_bytes = 0, kv_bytes = 0, device_bytes = 0;
  int64_t tasks = 0, pairs = 0, h2d = 0, d2h = 0;
};

void cqs_sizes_for(CqsPlan& p, int64_t n, int k, int Hq, int Hkv, int64_t S, int64_t T, int D, attn_dtype dt) {
  const int64_t es = elem_size(dt);
  p.n = n;
  p.k = k;
  p.bq = (S + n - 1) / n;
  p.bk = T > 0 ? (T + n - 1) / n : 0;
  p.q_bytes = align_up(p.bq * Hq * D * es);
  p.o_bytes = align_up(p.bq * Hq * D * 4);
  p.l_bytes = align_up(p.bq * Hq * 4);
  p.kv_bytes = align_up(std::max<int64_t>(p.bk, 1) * Hkv * D * es);
  // two sub-task slots, each with k query-side and k key-side blocks
  p.device_bytes = 2 * (int64_t)k * (p.q_bytes + p.o_bytes + p.l_bytes + 2 * p.kv_bytes);
}

struct Geometry {
  int64_t S, T;
  int causal;
  const CqsPlan* p;
  int64_t q_rows(int64_t x) const { return std::max<int64_t>(0, std::min(S, (x + 1) * p->bq) - x * p->bq); }
  int64_t k_rows(int64_t y) const {
    return p->bk == 0 ? 0 : std::max<int64_t>(0, std::min(T, (y + 1) * p->bk) - y * p->bk);
  }
  // absolute position of the last query of block x (bottom-right alignment)
  int64_t last_abs(int64_t x) const { return x * p->bq + q_rows(x) - 1 + (T - S); }
  bool sees_any(int64_t x) const { return T > 0 && (!causal || last_abs(x) >= 0); }
  bool visible(int64_t x, int64_t y) const { return !causal || y * p->bk <= last_abs(x); }
};

// The pairs of quorum sub-task i in execution order: fn(a, x, b, y) with
// x = base[a] + i and y = base[b] + i (mod N); b = y = -1 marks the empty
// pair of a query block that sees no key.
template <class F>
void for_task_pairs(const Geometry& g, int64_t i, F&& fn) {
  const CqsPlan& p = *g.p;
  for (int a = 0; a < p.k; ++a) {
    const int64_t x = (p.base[a] + i) % p.n;
    if (g.q_rows(x) == 0) continue;
    if (!g.sees_any(x)) {
      if (a == 0) fn(a, x, -1, (int64_t)-1);
      continue;
    }
    for (int b = 0; b < p.k; ++b) {
      if (a == b && a != 0) continue;  // the diagonal belongs to quorum x only
      const int64_t y = (p.base[b] + i) % p.n;
      if (g.k_rows(y) == 0 || !g.visible(x, y)) continue;
      fn(a, x, b, y);
    }
  }
}

// Host<->device bytes of the plan (one sequence's pattern times B).
void cqs_count(CqsPlan& p, int B, int Hq, int Hkv, int64_t S, int64_t T, int D, int causal, attn_dtype dt) {
  const int64_t es = elem_size(dt);
  Geometry g{S, T, causal, &p};
  std::vector<int64_t> writer((size_t)p.n, -1);  // sub-task that last wrote a block's running result
  std::vector<char> qin((size_t)p.k), kin((size_t)p.k);
  int64_t tasks = 0, pairs = 0, h2d = 0, d2h = 0;
  for (int64_t i = 0; i < p.n; ++i) {
    std::fill(qin.begin(), qin.end(), 0);
    std::fill(kin.begin(), kin.end(), 0);
    int64_t np = 0;
    for_task_pairs(g, i, [&](int a, int64_t, int b, int64_t) {
      qin[a] = 1;
      if (b >= 0) kin[b] = 1;
      ++np;
    });
    if (np == 0) continue;
    ++tasks;
    pairs += np;
    for (int a = 0; a < p.k; ++a) {
      const int64_t x = (p.base[a] + i) % p.n, y = x;
      if (kin[a]) h2d += 2 * g.k_rows(y) * Hkv * D * es;
      if (!qin[a]) continue;
      const int64_t nq = g.q_rows(x);
      h2d += nq * Hq * D * es;
      // an earlier sub-task's running result comes back from the host, the
      // previous sub-task's is copied on the device
      const int64_t wr = writer[(size_t)x];
      if (wr >= 0 && wr != tasks - 2) h2d += nq * Hq * D * 4 + nq * Hq * 4;
      d2h += nq * Hq * D * 4 + nq * Hq * 4;
      writer[(size_t)x] = tasks - 1;
    }
  }
  p.tasks = tasks * B;
  p.pairs = pairs * B;
  p.h2d = h2d * B;
  p.d2h = d2h * B;
}

attn_status make_cqs_plan(attn_dtype dt, int B, int Hq, int Hkv, int64_t S, int64_t T, int D, int causal,
                          size_t budget, int64_t force_n, CqsPlan* out) {
  const int64_t bud = streamx::usable_budget(budget);
  const int64_t span = std::max<int64_t>(std::max(S, T), 1);
  const CqsSize* pick = nullptr;
  CqsPlan p;
  for (const CqsSize& c : cqs_sizes()) {
    if (force_n > 0 && c.n != force_n) continue;
    cqs_sizes_for(p, c.n, c.k, Hq, Hkv, S, T, D, dt);
    if (p.device_bytes <= bud) {
      pick = &c;
      break;
    }
    if (force_n > 0) break;
    if (c.n >= span) break;  // blocks are single positions: larger N only grows the quorums
  }
  if (force_n > 0) {
    bool known = false;
    for (const CqsSize& c : cqs_sizes()) known |= c.n == force_n;
    if (!known)
      return set_error(ATTN_E_UNSUPPORTED,
                       "stream_cqs: no cyclic difference set of size %lld (supported: 1, 3, p*p+p+1 for prime "
                       "p <= %d)",
                       (long long)force_n, kMaxPrime);
  }
  if (!pick)
    return set_error(ATTN_E_BUDGET, "stream_cqs: no quorum size fits a device budget of %lld bytes",
                     (long long)budget);
  attn_status st = base_quorum(*pick, &p.base);
  if (st != ATTN_OK) return st;
  cqs_count(p, B, Hq, Hkv, S, T, D, causal, dt);
  *out = p;
  return ATTN_OK;
}

void fill_info(const CqsPlan& p, attn_cqs_info* info) {
  if (!info) return;
  memset(info, 0, sizeof(*info));
  info->n_blocks = p.n;
  info->quorum_size = p.k;
  info->pairs = p.pairs;
  for (int64_t a = 0; a < p.k && a < ATTN_CQS_MAX_QUORUM; ++a) info->base[a] = p.base[(size_t)a];
}

void fill_report(const CqsPlan& p, attn_stream_report* r) {
  if (!r) return;
  r->tasks = p.tasks;
  r->h2d_bytes = p.h2d;
  r->d2h_bytes = p.d2h;
  r->peak_device_bytes = p.device_bytes;
  r->block_q = p.bq;
  r->block_k = p.bk;
  r->wall_s = r->kernel_s = 0.0;
}

}  // namespace
}  // namespace attn

using namespace attn;

extern "C" attn_status attn_stream_cqs_plan(attn_dtype dt, int B, int Hq, int Hkv, int64_t S, int64_t T, int D,
                                            int causal, size_t device_budget_bytes, int64_t n_blocks, int64_t* pairs,
                                            int64_t cap, attn_cqs_info* info, attn_stream_report* plan) {
  attn_status st = streamx::check_stream_sizes(dt, B, Hq, Hkv, S, T, D);
  if (st != ATTN_OK) return st;
  if (n_blocks < 0 || cap < 0) return set_error(ATTN_E_INVALID, "stream_cqs: invalid sizes");
  if (B == 0 || S == 0) {
    if (info) memset(info, 0, sizeof(*info));
    if (plan) memset(plan, 0, sizeof(*plan));
    return ATTN_OK;
  }
  CqsPlan p;
  st = make_cqs_plan(dt, B, Hq, Hkv, S, T, D, causal, device_budget_bytes, n_blocks, &p);
  if (st != ATTN_OK) return st;
  if (pairs) {
    Geometry g{S, T, causal, &p};
    int64_t m = 0;
    for (int64_t b = 0; b < B; ++b)
      for (int64_t i = 0; i < p.n; ++i)
        for_task_pairs(g, i, [&](int, int64_t x, int, int64_t y) {
          if (m < cap) {
            pairs[4 * m] = b;
            pairs[4 * m + 1] = i;
            pairs[4 * m + 2] = x;
            pairs[4 * m + 3] = y;
          }
          ++m;
        });
  }
  fill_info(p, info);
  fill_report(p, plan);
  return ATTN_OK;
}

extern "C" attn_status attn_stream_cqs(attn_dtype dt, const void* q_host, const void* k_host, const void* v_host,
                                       int B, int Hq, int Hkv, int64_t S, int64_t T, int D, int causal, float scale,
                                       size_t device_budget_bytes, int64_t n_blocks, float* o_host, float* lse_host,
                                       attn_cqs_info* info, attn_stream_report* report) {
  const auto wall0 = std::chrono::steady_clock::now();
  attn_status st = streamx::check_stream_sizes(dt, B, Hq, Hkv, S, T, D);
  if (st != ATTN_OK) return st;
  if (n_blocks < 0) return set_error(ATTN_E_INVALID, "stream_cqs: invalid sizes");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return set_error(ATTN_E_INVALID, "stream_cqs: scale must be finite and > 0");
  if (B == 0 || S == 0) {
    if (info) memset(info, 0, sizeof(*info));
    if (report) memset(report, 0, sizeof(*report));
    return ATTN_OK;
  }
  if (!q_host || !o_host || (T > 0 && (!k_host || !v_host)))
    return set_error(ATTN_E_INVALID, "stream_cqs: null host pointer");
  st = streamx::check_pinned(dt, q_host, k_host, v_host, o_host, lse_host, B, Hq, Hkv, S, T, D);
  if (st != ATTN_OK) return st;
  CqsPlan p;
  st = make_cqs_plan(dt, B, Hq, Hkv, S, T, D, causal, device_budget_bytes, n_blocks, &p);
  if (st != ATTN_OK) return st;

  const int64_t es = elem_size(dt);
  const int64_t K = p.k;
  char* arena = nullptr;
  float* lse_tmp = nullptr;  // pinned host lse when the caller passes none (running results need it)
  // copy streams per direction.  Two measured slower than one on the 2^20-token
  // workload (29-30 s against 20-22 s wall), so one it is; the scheduling
  // below is written for any count.
  constexpr int kCopyStreams = 1;
  hipStream_t s_in[kCopyStreams] = {}, s_out[kCopyStreams] = {}, s_cmp = nullptr;
  std::vector<hipEvent_t> evs;
  std::vector<hipEvent_t> timing;
  attn_status result = ATTN_OK;
  auto ev = [&](unsigned flags) {
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, flags) != hipSuccess) return (hipEvent_t) nullptr;
    evs.push_back(e);
    return e;
  };
#define ATTN_HIP(call)                                                                             \
  do {                                                                                             \
    hipError_t e_ = (call);                                                                        \
    if (e_ != hipSuccess) {                                                                        \
      result = set_error(ATTN_E_DEVICE, "stream_cqs: %s failed: %s", #call, hipGetErrorString(e_)); \
      goto done;                                                                                   \
    }                                                                                              \
  } while (0)
  {
    ATTN_HIP(hipMalloc((void**)&arena, (size_t)p.device_bytes));
    float* lse_h = lse_host;
    if (!lse_h) {
      ATTN_HIP(hipHostMalloc((void**)&lse_tmp, (size_t)B * Hq * S * 4, hipHostMallocDefault));
      lse_h = lse_tmp;
    }
    for (int c = 0; c < kCopyStreams; ++c) {
      ATTN_HIP(hipStreamCreateWithFlags(&s_in[c], hipStreamNonBlocking));
      ATTN_HIP(hipStreamCreateWithFlags(&s_out[c], hipStreamNonBlocking));
    }
    ATTN_HIP(hipStreamCreateWithFlags(&s_cmp, hipStreamNonBlocking));
    // slot s: K query-side blocks (Q, O, lse) then K key-side blocks (K, V)
    std::vector<char*> qbuf(2 * K), obuf(2 * K), lbuf(2 * K), kbuf(2 * K), vbuf(2 * K);
    {
      char* cur = arena;
      for (int s = 0; s < 2; ++s)
        for (int64_t a = 0; a < K; ++a) {
          qbuf[s * K + a] = cur, cur += p.q_bytes;
          obuf[s * K + a] = cur, cur += p.o_bytes;
          lbuf[s * K + a] = cur, cur += p.l_bytes;
          kbuf[s * K + a] = cur, cur += p.kv_bytes;
          vbuf[s * K + a] = cur, cur += p.kv_bytes;
        }
    }
    // per slot: inbound copies landed (one per copy stream), compute done,
    // write-back done (one per copy stream)
    hipEvent_t ev_in[2][kCopyStreams], ev_done[2], ev_out[2][kCopyStreams];
    for (int s = 0; s < 2; ++s) {
      bool ok = true;
      for (int c = 0; c < kCopyStreams; ++c) {
        ev_in[s][c] = ev(hipEventDisableTiming);
        ev_out[s][c] = ev(hipEventDisableTiming);
        ok = ok && ev_in[s][c] && ev_out[s][c];
      }
      ev_done[s] = ev(hipEventDisableTiming);
      if (!ok || !ev_done[s]) {
        result = set_error(ATTN_E_DEVICE, "stream_cqs: event creation failed");
        goto done;
      }
    }
    const float scale_log2 = scale * kLog2e;
    Geometry g{S, T, causal, &p};
    // per (sequence, block): index of the sub-task that last wrote its running result, -1 = none
    std::vector<int64_t> last_writer((size_t)(B * p.n), -1);
    struct Pair {
      int a, b;
      int64_t x, y;
    };
    std::vector<Pair> prs;
    std::vector<char> qin((size_t)K), kin((size_t)K);
    int64_t job = 0;
    int64_t prev_i = -1;  // quorum index of sub-task job - 1
    for (int64_t b = 0; b < B; ++b) {
      for (int64_t i = 0; i < p.n; ++i) {
        prs.clear();
        for_task_pairs(g, i, [&](int a, int64_t x, int bb, int64_t y) { prs.push_back({a, bb, x, y}); });
        if (prs.empty()) continue;
        const int s = (int)(job & 1);
        std::fill(qin.begin(), qin.end(), 0);
        std::fill(kin.begin(), kin.end(), 0);
        for (const Pair& pr : prs) {
          qin[(size_t)pr.a] = 1;
          if (pr.b >= 0) kin[(size_t)pr.b] = 1;
        }
        int64_t* lw = &last_writer[(size_t)(b * p.n)];
        // ---- inbound.  The slot's Q, K and V buffers are free once sub-task
        // job-2 has computed; its O and lse buffers once that sub-task has
        // written them back, so those copies come last.  (Every stream also
        // follows every inbound copy of the previous sub-task: its
        // device-to-device reads come from the slot written next.)
        for (int c = 0; c < kCopyStreams; ++c) {
          if (job >= 2) ATTN_HIP(hipStreamWaitEvent(s_in[c], ev_done[s], 0));
          for (int c2 = 0; c2 < kCopyStreams; ++c2)
            if (job >= 1) ATTN_HIP(hipStreamWaitEvent(s_in[c], ev_in[1 - s][c2], 0));
        }
        int ci = 0;  // inbound copies alternate between the copy streams
        for (int64_t a = 0; a < K; ++a) {
          const int64_t y = (p.base[(size_t)a] + i) % p.n;
          if (!kin[(size_t)a]) continue;
          const int64_t nk = g.k_rows(y);
          const size_t off = (size_t)((b * T + y * p.bk) * Hkv * D * es);
          ATTN_HIP(hipMemcpyAsync(kbuf[s * K + a], (const char*)k_host + off, nk * Hkv * D * es,
                                  hipMemcpyHostToDevice, s_in[ci++ % kCopyStreams]));
          ATTN_HIP(hipMemcpyAsync(vbuf[s * K + a], (const char*)v_host + off, nk * Hkv * D * es,
                                  hipMemcpyHostToDevice, s_in[ci++ % kCopyStreams]));
        }
        // query blocks; running results of earlier sub-tasks from the host, and
        // those of the previous sub-task (consecutive quorums share a block)
        // straight from its slot on the device: that needs only its compute,
        // not its write-back, which then overlaps this sub-task
        for (int pass = 0; pass < 3; ++pass) {
          if (pass == 1 && job >= 2)
            for (int c = 0; c < kCopyStreams; ++c)
              for (int c2 = 0; c2 < kCopyStreams; ++c2) ATTN_HIP(hipStreamWaitEvent(s_in[c], ev_out[s][c2], 0));
          if (pass == 2) {
            bool any = false;
            for (int64_t a = 0; a < K; ++a)
              any |= qin[(size_t)a] && lw[(p.base[(size_t)a] + i) % p.n] == job - 1 && job >= 1;
            if (!any) break;
            for (int c = 0; c < kCopyStreams; ++c) ATTN_HIP(hipStreamWaitEvent(s_in[c], ev_done[1 - s], 0));
          }
          for (int64_t a = 0; a < K; ++a) {
            if (!qin[(size_t)a]) continue;
            const int64_t x = (p.base[(size_t)a] + i) % p.n;
            const int64_t nq = g.q_rows(x), x0 = x * p.bq;
            if (pass == 0) {
              ATTN_HIP(hipMemcpyAsync(qbuf[s * K + a], (const char*)q_host + ((b * S + x0) * Hq * D) * es,
                                      nq * Hq * D * es, hipMemcpyHostToDevice, s_in[ci++ % kCopyStreams]));
              continue;
            }
            const int64_t w = lw[x];
            if (w < 0 || (pass == 1) != (w < job - 1)) continue;
            if (pass == 2) {
              int64_t ap = -1;  // the block's place in the previous sub-task's quorum
              for (int64_t c = 0; c < K; ++c)
                if ((p.base[(size_t)c] + prev_i) % p.n == x) {
                  ap = c;
                  break;
                }
              if (ap < 0) {
                result = set_error(ATTN_E_DEVICE, "stream_cqs: block %lld not in the previous quorum", (long long)x);
                goto done;
              }
              hipStream_t sc = s_in[ci++ % kCopyStreams];
              ATTN_HIP(hipMemcpyAsync(obuf[s * K + a], obuf[(1 - s) * K + ap], nq * Hq * D * 4,
                                      hipMemcpyDeviceToDevice, sc));
              ATTN_HIP(hipMemcpyAsync(lbuf[s * K + a], lbuf[(1 - s) * K + ap], nq * Hq * 4,
                                      hipMemcpyDeviceToDevice, sc));
              continue;
            }
            ATTN_HIP(hipMemcpyAsync(obuf[s * K + a], (const char*)o_host + (b * S + x0) * Hq * D * 4,
                                    nq * Hq * D * 4, hipMemcpyHostToDevice, s_in[ci % kCopyStreams]));
            ATTN_HIP(hipMemcpy2DAsync(lbuf[s * K + a], (size_t)nq * 4, (const char*)lse_h + ((b * Hq) * S + x0) * 4,
                                      (size_t)S * 4, (size_t)nq * 4, (size_t)Hq, hipMemcpyHostToDevice,
                                      s_in[ci++ % kCopyStreams]));
          }
        }
        for (int c = 0; c < kCopyStreams; ++c) ATTN_HIP(hipEventRecord(ev_in[s][c], s_in[c]));
        // ---- compute: one prefill launch per pair, merged into the query block's running result
        for (int c = 0; c < kCopyStreams; ++c) ATTN_HIP(hipStreamWaitEvent(s_cmp, ev_in[s][c], 0));
        hipEvent_t t0 = ev(hipEventDefault), t1 = ev(hipEventDefault);
        if (!t0 || !t1) {
          result = set_error(ATTN_E_DEVICE, "stream_cqs: event creation failed");
          goto done;
        }
        timing.push_back(t0);
        timing.push_back(t1);
        ATTN_HIP(hipEventRecord(t0, s_cmp));
        std::fill(kin.begin(), kin.end(), 0);  // reused: query block already merged into in this sub-task
        for (const Pair& pr : prs) {
          const int64_t nq = g.q_rows(pr.x);
          const int acc = lw[pr.x] >= 0 || kin[(size_t)pr.a];
          kin[(size_t)pr.a] = 1;
          PrefillArgs a = streamx::block_args(qbuf[s * K + pr.a], nullptr, nullptr, (float*)obuf[s * K + pr.a],
                                              (float*)lbuf[s * K + pr.a], Hq, Hkv, D, nq, 0,
                                              pr.x * p.bq + (T - S), 0, causal, acc, scale_log2);
          if (pr.y < 0) {  // no visible key: an empty key block writes O = 0, lse = -inf
            a.k = a.v = qbuf[s * K + pr.a];
          } else {
            a.k = kbuf[s * K + pr.b];
            a.v = vbuf[s * K + pr.b];
            a.n_k = g.k_rows(pr.y);
            a.k_abs0 = pr.y * p.bk;
          }
          st = dt == ATTN_BF16 ? launch_prefill_bf16(a, D, s_cmp) : launch_prefill_f32(a, D, s_cmp);
          if (st != ATTN_OK) {
            result = st;
            goto done;
          }
        }
        ATTN_HIP(hipEventRecord(t1, s_cmp));
        ATTN_HIP(hipEventRecord(ev_done[s], s_cmp));
        // ---- outbound: every query block this sub-task merged into
        // (after the previous sub-task's write-back too: a block both wrote
        // must reach the host in sub-task order)
        for (int c = 0; c < kCopyStreams; ++c) {
          ATTN_HIP(hipStreamWaitEvent(s_out[c], ev_done[s], 0));
          if (job >= 1)
            for (int c2 = 0; c2 < kCopyStreams; ++c2) ATTN_HIP(hipStreamWaitEvent(s_out[c], ev_out[1 - s][c2], 0));
        }
        int co = 0;
        for (int64_t a = 0; a < K; ++a) {
          if (!qin[(size_t)a]) continue;
          const int64_t x = (p.base[(size_t)a] + i) % p.n;
          const int64_t nq = g.q_rows(x), x0 = x * p.bq;
          ATTN_HIP(hipMemcpyAsync((char*)o_host + (b * S + x0) * Hq * D * 4, obuf[s * K + a], nq * Hq * D * 4,
                                  hipMemcpyDeviceToHost, s_out[co % kCopyStreams]));
          ATTN_HIP(hipMemcpy2DAsync((char*)lse_h + ((b * Hq) * S + x0) * 4, (size_t)S * 4, lbuf[s * K + a],
                                    (size_t)nq * 4, (size_t)nq * 4, (size_t)Hq, hipMemcpyDeviceToHost,
                                    s_out[co++ % kCopyStreams]));
          lw[x] = job;
        }
        for (int c = 0; c < kCopyStreams; ++c) ATTN_HIP(hipEventRecord(ev_out[s][c], s_out[c]));
        prev_i = i;
        ++job;
      }
    }
    for (int c = 0; c < kCopyStreams; ++c) ATTN_HIP(hipStreamSynchronize(s_in[c]));
    ATTN_HIP(hipStreamSynchronize(s_cmp));
    for (int c = 0; c < kCopyStreams; ++c) ATTN_HIP(hipStreamSynchronize(s_out[c]));
    double ksum = 0.0;
    for (size_t t = 0; t + 1 < timing.size(); t += 2) {
      float ms = 0.f;
      ATTN_HIP(hipEventElapsedTime(&ms, timing[t], timing[t + 1]));
      ksum += ms * 1e-3;
    }
    fill_info(p, info);
    if (report) {
      fill_report(p, report);
      report->kernel_s = ksum;
    }
  }
done:
#undef ATTN_HIP
  for (int c = 0; c < kCopyStreams; ++c)
    if (s_in[c]) (void)hipStreamSynchronize(s_in[c]);
  if (s_cmp) (void)hipStreamSynchronize(s_cmp);
  for (int c = 0; c < kCopyStreams; ++c)
    if (s_out[c]) (void)hipStreamSynchronize(s_out[c]);
  for (hipEvent_t e : evs) (void)hipEventDestroy(e);
  for (int c = 0; c < kCopyStreams; ++c) {
    if (s_in[c]) (void)hipStreamDestroy(s_in[c]);
    if (s_out[c]) (void)hipStreamDestroy(s_out[c]);
  }
  if (s_cmp) (void)hipStreamDestroy(s_cmp);
  if (arena) (void)hipFree(arena);
  if (lse_tmp) (void)hipHostFree(lse_tmp);
  if (result == ATTN_OK && report)
    report->wall_s = std::chrono::duration<double>(std::chrono::steady_clock::now() - wall0).count();
  return result;
}
