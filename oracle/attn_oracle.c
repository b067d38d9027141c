/*
 * fp64 CPU oracle for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only tests/, the smoke check and the bench's CPU-baseline
 * leg do.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes is the plain definition, written out naively:
 *
 *   O[b,i,h,:] = sum_j softmax_j( scale * <q_{b,i,h}, k_{b,j,hkv}> ) v_{b,j,hkv}
 *   lse[b,h,i] = log sum_j exp( scale * <q, k_j> )          (natural log)
 *
 * over the visible keys j only.  Sources:
 *  - exact attention A = softmax(QK^T)V: Stream-CQSA summary (euno.news),
 *    "Methodology" item 2 (CQS Divide); the page omits the scale, which is
 *    taken here as an explicit argument (1/sqrt(D) in every workload);
 *  - grouped-query attention, query head h reads KV head floor(h / G),
 *    G = Hq / Hkv: LLM-CoOpt summary, "Methodology" item 2 (Opt-GQA);
 *  - causal visibility from the absolute query position (past length + local
 *    index): ONNX Runtime PR #33328 analysis, section 1 (scoring); with
 *    S queries and T keys, query i sits at position i + T - S and sees key j
 *    iff j <= i + T - S;
 *  - fixed-size KV pages addressed through a page table: LLM-CoOpt summary,
 *    "Methodology" item 3 (Opt-Pa);
 *  - quantised KV (int8, fp8) decoded before use: ONNX Runtime PR #28695
 *    analysis, introduction and section 1; LLM-CoOpt "Methodology" item 1
 *    (FP8 KV).  int8: value = code * per-(token, KV head) scale.  fp8: OCP
 *    e4m3fn (bias 7, no infinities, S.1111.111 = NaN) times a per-KV-head
 *    scale.  int4 (named beside int8 in the ONNX Runtime PR #28695
 *    analysis, introduction; the page fixes no layout, so this one is a
 *    plain reading of it): signed
 *    two's-complement 4-bit codes, element 2i in the low nibble of byte i and
 *    element 2i+1 in its high nibble, value = code * the scale of the
 *    element's 32-element group of its (token, KV head) row;
 *  - merge of partial results by log-sum-exp: ONNX Runtime PR #28695
 *    analysis, section 2 (flash decoding, reduce phase).
 *
 * A query row with no visible key gets O = 0 and lse = -inf (the pages name
 * masked-row handling without fixing a value; this is the reading adopted).
 *
 * Every score row is materialised in full (no blocking, no online softmax).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the oracle runs on (OpenMP team size). */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the threads of later calls (n >= 1); only the timing of the oracle
   changes, every row is computed the same way on any thread. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8_E4M3 = 2, OR_INT8 = 3, OR_INT4 = 4 };

enum { OR_INT4_GROUP = 32 }; /* elements per int4 scale group */

/* ---- element decoders, each written from its format definition ---- */

static double dec_bf16(uint16_t bits) {
  /* bf16 is the upper half of an IEEE binary32 */
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double oracle_e4m3fn_value(uint8_t code) {
  /* OCP 8-bit float E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa;
   * exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities. */
  int s = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

double oracle_bf16_value(uint16_t bits) { return dec_bf16(bits); }

static double dec_elem(int dt, const void* base, int64_t idx) {
  switch (dt) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_BF16: return dec_bf16(((const uint16_t*)base)[idx]);
    case OR_FP8_E4M3: return oracle_e4m3fn_value(((const uint8_t*)base)[idx]);
    case OR_INT8: return (double)((const int8_t*)base)[idx];
    case OR_INT4: {
      uint8_t byte = ((const uint8_t*)base)[idx / 2];
      int nib = (idx % 2) ? (byte >> 4) : (byte & 15);
      return (double)(nib >= 8 ? nib - 16 : nib); /* 4-bit two's complement */
    }
  }
  return NAN;
}

typedef struct {
  int kv_dtype;
  const void *k, *v;
  const float *k_scale, *v_scale;
  const int32_t* page_table; /* NULL: contiguous */
  int64_t max_pages, page_size, Hkv, D, B, T;
  int contiguous_bthd; /* 1: [B,T,Hkv,D] prefill layout; 0: [P,Hkv,ps,D] cache layout */
} kv_store;

/* Linear index (in elements, without D) of token j of sequence b, KV head hk. */
static int64_t kv_row(const kv_store* s, int64_t b, int64_t j, int64_t hk) {
  if (s->contiguous_bthd) return (b * s->T + j) * s->Hkv + hk;
  int64_t page, off;
  if (s->page_table) {
    page = s->page_table[b * s->max_pages + j / s->page_size];
    off = j % s->page_size;
  } else {
    page = b; /* contiguous cache: one page of page_size tokens per sequence */
    off = j;
  }
  return (page * s->Hkv + hk) * s->page_size + off;
}

static double kv_value(const kv_store* s, const void* base, const float* scale, int64_t row, int64_t hk,
                       int64_t d) {
  double x = dec_elem(s->kv_dtype, base, row * s->D + d);
  if (s->kv_dtype == OR_INT8) x *= (double)scale[row];          /* per token, per KV head */
  else if (s->kv_dtype == OR_FP8_E4M3) x *= (double)scale[hk];  /* per KV head */
  else if (s->kv_dtype == OR_INT4) x *= (double)scale[row * (s->D / OR_INT4_GROUP) + d / OR_INT4_GROUP];
  return x;
}

/* One query row against its visible keys; scratch holds n_keys doubles. */
static void one_row(const kv_store* s, const double* qv, int64_t b, int64_t hk, int64_t n_vis, double scale,
                    double* scratch, double* o, double* lse) {
  int64_t D = s->D;
  if (n_vis <= 0) {
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int64_t j = 0; j < n_vis; ++j) {
    int64_t row = kv_row(s, b, j, hk);
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += qv[d] * kv_value(s, s->k, s->k_scale, row, hk, d);
    scratch[j] = scale * dot;
    if (scratch[j] > m) m = scratch[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < n_vis; ++j) {
    scratch[j] = exp(scratch[j] - m);
    l += scratch[j];
  }
  for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
  for (int64_t j = 0; j < n_vis; ++j) {
    int64_t row = kv_row(s, b, j, hk);
    double p = scratch[j] / l;
    for (int64_t d = 0; d < D; ++d) o[d] += p * kv_value(s, s->v, s->v_scale, row, hk, d);
  }
  *lse = m + log(l);
}

/*
 * Attention in fp64.
 *   q: [B, S, Hq, D] of q_dtype (f32, bf16 bits or e4m3fn bytes); q_scale [Hq]
 *      (nullable) multiplies query head h (the per-head scale of e4m3 queries).
 *   KV (prefill layout, layout=0): k, v [B, T, Hkv, D]; kv_lens may be NULL (all T).
 *   KV (cache layout,  layout=1): k, v [P, Hkv, page_size, D] through page_table
 *       [B, max_pages] int32, or contiguous [B, Hkv, page_size, D] when
 *       page_table is NULL.  Scales: int8 -> [P or B, Hkv, page_size] fp32,
 *       fp8 -> [Hkv] fp32, otherwise NULL.  kv_lens [B] required.
 *   causal: query i of sequence b sees key j iff j <= i + T_b - S.
 *   rows: NULL (all S query rows) or n_rows query indices.
 *   Out: o [B, n_rows, Hq, D] f64, lse [B, Hq, n_rows] f64.
 * Returns 0 on success, nonzero on bad arguments or allocation failure.
 */
int oracle_attention(int q_dtype, const void* q, const float* q_scale, int kv_dtype, int layout, const void* k,
                     const void* v,
                     const float* k_scale, const float* v_scale, const int32_t* page_table, int64_t max_pages,
                     int64_t page_size, const int64_t* kv_lens, int64_t B, int64_t Hq, int64_t Hkv, int64_t S,
                     int64_t T, int64_t D, int causal, double scale, const int64_t* rows, int64_t n_rows,
                     double* o, double* lse) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || S < 0 || T < 0 || D <= 0) return 1;
  if (layout == 1 && !kv_lens) return 1;
  if (!rows) n_rows = S;
  int64_t G = Hq / Hkv;
  kv_store st = {kv_dtype, k, v, k_scale, v_scale, page_table, max_pages, page_size, Hkv, D, B, T, layout == 0};
  int64_t max_t = T;
  if (kv_lens)
    for (int64_t b = 0; b < B; ++b)
      if (kv_lens[b] > max_t) max_t = kv_lens[b];
  int64_t total = B * n_rows * Hq;
  int err = 0;
#pragma omp parallel
  {
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(max_t > 0 ? max_t : 1));
    double* qv = (double*)malloc(sizeof(double) * (size_t)D);
    if (!scratch || !qv) {
#pragma omp atomic write
      err = 2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t w = 0; w < total; ++w) {
        int64_t h = w % Hq;
        int64_t r = (w / Hq) % n_rows;
        int64_t b = w / (Hq * n_rows);
        int64_t i = rows ? rows[r] : r;
        int64_t hk = h / G;
        int64_t Tb = kv_lens ? kv_lens[b] : T;
        int64_t n_vis = Tb;
        if (causal) {
          int64_t last = i + Tb - S; /* last visible key index */
          n_vis = last + 1 < Tb ? last + 1 : Tb;
        }
        double qs = q_scale ? (double)q_scale[h] : 1.0;
        for (int64_t d = 0; d < D; ++d) qv[d] = qs * dec_elem(q_dtype, q, ((b * S + i) * Hq + h) * D + d);
        one_row(&st, qv, b, hk, n_vis, scale, scratch, o + ((b * n_rows + r) * Hq + h) * D,
                lse + (b * Hq + h) * n_rows + r);
      }
    }
    free(scratch);
    free(qv);
  }
  return err;
}

/*
 * Log-sum-exp merge of n partial results of the same rows (fp64).
 *   o_parts [n, R, D] (each normalised by its own softmax sum), lse_parts [n, R];
 *   a partial with lse = -inf covers no key and carries no weight.
 *   O = sum_c w_c O_c / sum_c w_c with w_c = exp(lse_c - M), M = max_c lse_c;
 *   lse = M + log sum_c w_c.  All partials empty -> O = 0, lse = -inf.
 */
int oracle_merge(int64_t n, const double* o_parts, const double* lse_parts, int64_t R, int64_t D, double* o,
                 double* lse) {
  if (n < 0 || R < 0 || D <= 0) return 1;
  for (int64_t r = 0; r < R; ++r) {
    double M = -INFINITY;
    for (int64_t c = 0; c < n; ++c)
      if (lse_parts[c * R + r] > M) M = lse_parts[c * R + r];
    double* orow = o + r * D;
    for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
    if (M == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double wsum = 0.0;
    for (int64_t c = 0; c < n; ++c) {
      double w = exp(lse_parts[c * R + r] - M);
      wsum += w;
      for (int64_t d = 0; d < D; ++d) orow[d] += w * o_parts[(c * R + r) * D + d];
    }
    for (int64_t d = 0; d < D; ++d) orow[d] /= wsum;
    lse[r] = M + log(wsum);
  }
  return 0;
}
