/*
 * fa_oracle.c -- plain, slow, fp64 CPU reference for exact attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library: it has its own input
 * decoders and its own reading of the shapes.
 *
 * What it computes (the plain definition of the method that the pages
 * dissect; FlashAttention, Dao et al. 2022, cited by "FlashAttention on
 * SM120 reusing the SM80 forward", reference [8]):
 *
 *   for every sequence b, query head h, query row i of that sequence
 *     g    = h / (Hq / Hkv)                       (grouped-query heads)
 *     A_i  = { j : 0 <= j < sk_b  and  (not causal or j <= i + sk_b - sq_b) }
 *     s_ij = softmax_scale * sum_d q[i,h,d] * k[j,g,d]           (j in A_i)
 *     if A_i is empty:  O[i,h,:] = 0,  LSE[h,i] = -inf
 *     else:             M = max_j s_ij,  Z = sum_j exp(s_ij - M)
 *                       LSE[h,i] = M + ln Z
 *                       O[i,h,:] = sum_j exp(s_ij - M) / Z * v[j,g,:]
 *
 * The zero-output / minus-infinity LSE rule for rows with no admissible key
 * is the epilogue's store_zero path shown in "FlashAttention core algorithm:
 * forward pass" (consumer loop, epilogue excerpt).  The causal mask is
 * aligned bottom-right (query i of a sequence with sq queries and sk keys
 * sees keys up to i + sk - sq); with sq == sk this is the usual lower
 * triangle.  Every entry of a row of S is computed before its softmax: no
 * online rescaling, no blocking of the key axis.
 *
 * Inputs are decoded exactly to double: bf16 bit patterns (upper half of an
 * IEEE binary32) or OCP fp8 e4m3 ("e4m3fn": bias 7, no infinities, S.1111.111
 * is NaN) bytes times a per-tensor descale, the FP8 descale convention of the
 * forward-pass page (q and k descales multiply the scores, the v descale the
 * output).
 *
 * Layouts (token-major, contiguous):
 *   Q [total_q][Hq][D], K [total_k][Hkv][D], V [total_k][Hkv][Dv]
 *   O [total_q][Hq][Dv] (double), LSE [Hq][total_q] (double)
 *   cu_seqlens == NULL: fixed length, total_q = batch*seqlen_q,
 *                       total_k = batch*seqlen_k
 *   else int32[2*(batch+1)]: query offsets cu[0..batch], key offsets
 *                            cu[batch+1 .. 2*batch+1]
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math: IEEE double).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BF16 0
#define ORACLE_E4M3 1

/* ---- exact decoders ---------------------------------------------------- */

double oracle_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16; /* bf16 is the top half of a binary32 */
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double oracle_e4m3_to_double(uint8_t byte) {
  int sign = (byte >> 7) & 1;
  int expo = (byte >> 3) & 0xF;
  int mant = byte & 0x7;
  double mag;
  if (expo == 0xF && mant == 0x7) return NAN; /* the only NaN encodings */
  if (expo == 0)
    mag = ldexp((double)mant / 8.0, 1 - 7); /* subnormal: 0.mmm * 2^-6 */
  else
    mag = ldexp(1.0 + (double)mant / 8.0, expo - 7);
  return sign ? -mag : mag;
}

void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_double(in[i]);
}

void oracle_decode_e4m3(const uint8_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_double(in[i]);
}

/* ---- problem description ----------------------------------------------- */

typedef struct {
  const void* q;
  const void* k;
  const void* v;
  int dtype; /* ORACLE_BF16 or ORACLE_E4M3 */
  int batch, hq, hkv, seqlen_q, seqlen_k;
  const int32_t* cu; /* NULL or 2*(batch+1) offsets */
  int d, dv;
  double scale;
  int causal;
  double dq, dk, dvs; /* descales (1.0 for bf16) */
} prob_t;

static double elem(const prob_t* p, const void* base, int64_t idx, double descale) {
  if (p->dtype == ORACLE_BF16) return oracle_bf16_to_double(((const uint16_t*)base)[idx]);
  return oracle_e4m3_to_double(((const uint8_t*)base)[idx]) * descale;
}

static void seq_bounds(const prob_t* p, int b, int64_t* q0, int* sq, int64_t* k0, int* sk) {
  if (p->cu) {
    *q0 = p->cu[b];
    *sq = p->cu[b + 1] - p->cu[b];
    *k0 = p->cu[p->batch + 1 + b];
    *sk = p->cu[p->batch + 2 + b] - p->cu[p->batch + 1 + b];
  } else {
    *q0 = (int64_t)b * p->seqlen_q;
    *sq = p->seqlen_q;
    *k0 = (int64_t)b * p->seqlen_k;
    *sk = p->seqlen_k;
  }
}

/* Key j is admissible for query i (A_i above). */
static int admissible(const prob_t* p, int i, int j, int sq, int sk) {
  if (j < 0 || j >= sk) return 0;
  if (p->causal && (int64_t)j > (int64_t)i + sk - sq) return 0;
  return 1;
}

/*
 * One output row: O row (dv doubles), its LSE, and optionally the
 * probability row P (sk doubles, 0 for inadmissible keys).  s is scratch of
 * at least sk doubles.
 */
static void attention_row(const prob_t* p, int b, int h, int i, double* o_row, double* lse,
                          double* p_row, double* s) {
  int64_t q0, k0;
  int sq, sk;
  seq_bounds(p, b, &q0, &sq, &k0, &sk);
  const int g = h / (p->hq / p->hkv);
  const int64_t qbase = ((q0 + i) * p->hq + h) * (int64_t)p->d;
  int any = 0;
  double m = -INFINITY;
  for (int j = 0; j < sk; ++j) {
    if (!admissible(p, i, j, sq, sk)) continue;
    const int64_t kbase = ((k0 + j) * p->hkv + g) * (int64_t)p->d;
    double dot = 0.0;
    for (int d = 0; d < p->d; ++d)
      dot += elem(p, p->q, qbase + d, p->dq) * elem(p, p->k, kbase + d, p->dk);
    s[j] = p->scale * dot;
    if (!any || s[j] > m) m = s[j];
    any = 1;
  }
  for (int e = 0; e < p->dv; ++e) o_row[e] = 0.0;
  if (p_row)
    for (int j = 0; j < sk; ++j) p_row[j] = 0.0;
  if (!any) {
    *lse = -INFINITY;
    return;
  }
  double z = 0.0;
  for (int j = 0; j < sk; ++j)
    if (admissible(p, i, j, sq, sk)) z += exp(s[j] - m);
  *lse = m + log(z);
  for (int j = 0; j < sk; ++j) {
    if (!admissible(p, i, j, sq, sk)) continue;
    const double pij = exp(s[j] - m) / z;
    if (p_row) p_row[j] = pij;
    const int64_t vbase = ((k0 + j) * p->hkv + g) * (int64_t)p->dv;
    for (int e = 0; e < p->dv; ++e) o_row[e] += pij * elem(p, p->v, vbase + e, p->dvs);
  }
}

static int fill_prob(prob_t* p, const void* q, const void* k, const void* v, int dtype, int batch,
                     int hq, int hkv, int seqlen_q, int seqlen_k, const int32_t* cu, int d, int dv,
                     double scale, int causal, const double* descales) {
  if (!q || !k || !v || batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || d <= 0 || dv <= 0 ||
      seqlen_q < 0 || seqlen_k < 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_E4M3))
    return -1;
  p->q = q;
  p->k = k;
  p->v = v;
  p->dtype = dtype;
  p->batch = batch;
  p->hq = hq;
  p->hkv = hkv;
  p->seqlen_q = seqlen_q;
  p->seqlen_k = seqlen_k;
  p->cu = cu;
  p->d = d;
  p->dv = dv;
  p->scale = scale;
  p->causal = causal;
  p->dq = p->dk = p->dvs = 1.0;
  if (dtype == ORACLE_E4M3) {
    if (!descales) return -1;
    p->dq = descales[0];
    p->dk = descales[1];
    p->dvs = descales[2];
  }
  return 0;
}

static int max_sk(const prob_t* p) {
  if (!p->cu) return p->seqlen_k;
  int mx = 0;
  for (int b = 0; b < p->batch; ++b) {
    int sk = p->cu[p->batch + 2 + b] - p->cu[p->batch + 1 + b];
    if (sk > mx) mx = sk;
  }
  return mx;
}

/*
 * Whole forward: O [total_q][Hq][Dv], LSE [Hq][total_q] (doubles).
 * Returns 0, or -1 on a malformed call.  Parallel over (b, h, row).
 */
int oracle_fwd(const void* q, const void* k, const void* v, int dtype, int batch, int hq, int hkv,
               int seqlen_q, int seqlen_k, const int32_t* cu, int d, int dv, double scale,
               int causal, const double* descales, double* o, double* lse) {
  prob_t p;
  if (fill_prob(&p, q, k, v, dtype, batch, hq, hkv, seqlen_q, seqlen_k, cu, d, dv, scale, causal,
                descales))
    return -1;
  const int64_t total_q = cu ? cu[batch] : (int64_t)batch * seqlen_q;
  const int skmax = max_sk(&p);
  /* work items: (b, h, i) enumerated over every sequence */
  int64_t n_items = 0;
  for (int b = 0; b < batch; ++b) {
    int64_t q0, k0;
    int sq, sk;
    seq_bounds(&p, b, &q0, &sq, &k0, &sk);
    n_items += (int64_t)sq * hq;
  }
  int err = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(skmax > 0 ? skmax : 1));
    if (!s) {
#pragma omp atomic write
      err = -1;
    }
#pragma omp for schedule(dynamic, 64)
    for (int64_t it = 0; it < n_items; ++it) {
      if (!s) continue;
      /* map the flat item back to (b, i, h) */
      int64_t rem = it;
      int b = 0;
      for (;; ++b) {
        int64_t q0, k0;
        int sq, sk;
        seq_bounds(&p, b, &q0, &sq, &k0, &sk);
        if (rem < (int64_t)sq * hq) break;
        rem -= (int64_t)sq * hq;
      }
      int64_t q0, k0;
      int sq, sk;
      seq_bounds(&p, b, &q0, &sq, &k0, &sk);
      const int i = (int)(rem / hq), h = (int)(rem % hq);
      double l;
      attention_row(&p, b, h, i, o + ((q0 + i) * hq + h) * (int64_t)dv, &l, NULL, s);
      lse[(int64_t)h * total_q + q0 + i] = l;
    }
    free(s);
  }
  return err;
}

/*
 * Selected rows only: rows[3*r .. 3*r+2] = (b, h, i) with i the row inside
 * sequence b.  O rows go to o_rows[r*Dv ..], LSE to lse_rows[r].  Used to
 * check sampled outputs at sizes where the whole forward is too slow.
 */
int oracle_fwd_rows(const void* q, const void* k, const void* v, int dtype, int batch, int hq,
                    int hkv, int seqlen_q, int seqlen_k, const int32_t* cu, int d, int dv,
                    double scale, int causal, const double* descales, const int32_t* rows,
                    int64_t n_rows, double* o_rows, double* lse_rows) {
  prob_t p;
  if (fill_prob(&p, q, k, v, dtype, batch, hq, hkv, seqlen_q, seqlen_k, cu, d, dv, scale, causal,
                descales))
    return -1;
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t q0, k0;
    int sq, sk;
    const int b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
    if (b < 0 || b >= batch || h < 0 || h >= hq) return -1;
    seq_bounds(&p, b, &q0, &sq, &k0, &sk);
    if (i < 0 || i >= sq) return -1;
  }
  const int skmax = max_sk(&p);
  int err = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(skmax > 0 ? skmax : 1));
    if (!s) {
#pragma omp atomic write
      err = -1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!s) continue;
      attention_row(&p, rows[3 * r], rows[3 * r + 1], rows[3 * r + 2], o_rows + r * (int64_t)dv,
                    lse_rows + r, NULL, s);
    }
    free(s);
  }
  return err;
}

/*
 * The probability row P[i, :] (length sk of sequence b, zeros for masked
 * keys) of one (b, h, i), plus its O row and LSE.  Exposes the explicit
 * softmax so tests can check that each row sums to one.
 */
int oracle_probs_row(const void* q, const void* k, const void* v, int dtype, int batch, int hq,
                     int hkv, int seqlen_q, int seqlen_k, const int32_t* cu, int d, int dv,
                     double scale, int causal, const double* descales, int b, int h, int i,
                     double* p_row, double* o_row, double* lse) {
  prob_t p;
  if (fill_prob(&p, q, k, v, dtype, batch, hq, hkv, seqlen_q, seqlen_k, cu, d, dv, scale, causal,
                descales))
    return -1;
  int64_t q0, k0;
  int sq, sk;
  if (b < 0 || b >= batch || h < 0 || h >= hq) return -1;
  seq_bounds(&p, b, &q0, &sq, &k0, &sk);
  if (i < 0 || i >= sq) return -1;
  double* s = (double*)malloc(sizeof(double) * (size_t)(sk > 0 ? sk : 1));
  if (!s) return -1;
  attention_row(&p, b, h, i, o_row, lse, p_row, s);
  free(s);
  return 0;
}

int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
