/*
 * sdpa_oracle.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * A plain, slow, obviously correct fp64 CPU definition of scaled-dot-product
 * attention, used only by tests/, the package smoke check and the benchmark's
 * CPU-baseline leg to check the HIP kernels.  It shares no code, header, table
 * or helper with the GPU library.
 *
 * What it computes (the definition the pages' blocked algorithm reaches):
 *   "Xe SDPA Forward Mainloop -- Key Loops + Shapes", section "Full simplified
 *   pseudocode": softmax(Q K^T * scale + mask) V, streamed over K blocks with an
 *   online softmax.  The online rescale is an identity in real arithmetic, so
 *   this oracle evaluates the plain two-pass definition row by row instead:
 *       s_j = scale * sum_d Q[i,d] K[j,d]          for every visible key j
 *       m   = max_j s_j,  w_j = exp(s_j - m),  l = sum_j w_j
 *       O_i = sum_j (w_j / l) V[j,:],   lse_i = m + ln l
 *   GQA head map ("xe2-sdp-kernels", section "GQA layout"): query head h reads
 *   KV head h / (head_q / head_kv).
 *   Causal visibility (bottom-right aligned): key j is visible to query i iff
 *   j <= i + kv_len - q_len.  A row with no visible key (possible when
 *   q_len > kv_len, or kv_len == 0) yields O = 0 and lse = -inf instead of the
 *   0/0 the same page ("Correctness testing") names as the usual NaN source.
 *
 * Inputs are raw element bits; each element is widened exactly to double on
 * the fly (bf16, fp16, OCP fp8 e4m3fn, fp32, fp64) and multiplied by the
 * tensor's per-tensor dequantisation scale (1.0 for non-fp8 inputs).
 *
 * Layouts (row-major, batch outermost):
 *   Q [B, Sq, Hq, D], K [B, Sk, Hkv, D], V [B, Sk, Hkv, Dv].
 * Output rows are addressed as r = (b*Sq + i)*Hq + h, i.e. O [B, Sq, Hq, Dv].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_FP8_E4M3 = 2, ORC_F32 = 3, ORC_F64 = 4 };

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_decode_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double orc_decode_bf16(uint16_t b) {
  int s = b >> 15, e = (b >> 7) & 255, m = b & 127;
  double v;
  if (e == 0) v = ldexp((double)m, -133);
  else if (e == 255) v = m ? NAN : INFINITY;
  else v = ldexp((double)(128 + m), e - 134);
  return s ? -v : v;
}

/* OCP fp8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 fraction bits, no
 * infinities; only S.1111.111 is NaN, so the largest finite value is 448. */
double orc_decode_e4m3(uint8_t x) {
  int s = x >> 7, e = (x >> 3) & 15, m = x & 7;
  double v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
  switch (dtype) {
    case ORC_F16: return orc_decode_f16(((const uint16_t*)base)[idx]);
    case ORC_BF16: return orc_decode_bf16(((const uint16_t*)base)[idx]);
    case ORC_FP8_E4M3: return orc_decode_e4m3(((const uint8_t*)base)[idx]);
    case ORC_F32: return (double)((const float*)base)[idx];
    default: return ((const double*)base)[idx];
  }
}

/*
 * Computes attention for n_rows query rows.
 *   rows     : n_rows triples (b, i, h); NULL means every row in natural order
 *              r = (b*Sq + i)*Hq + h, with n_rows = B*Sq*Hq.
 *   out      : [n_rows, d_v] doubles (required).
 *   lse      : [n_rows] doubles, natural-log sum-exp of the scaled scores, or
 *              NULL.
 *   probs    : [n_rows, kv_len] doubles holding the softmax row (0 where the
 *              key is masked), or NULL.  Meant for small shapes only.
 *   n_threads: OpenMP threads (<= 0 keeps the runtime default).
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
int orc_sdpa_rows(int batch, int q_len, int kv_len, int head_q, int head_kv,
                  int d_qk, int d_v, int q_dtype, int kv_dtype, const void* q,
                  const void* k, const void* v, double q_scale, double k_scale,
                  double v_scale, double scale, int causal, int64_t n_rows,
                  const int64_t* rows, double* out, double* lse, double* probs,
                  int n_threads) {
  if (batch < 0 || q_len < 0 || kv_len < 0 || head_q <= 0 || head_kv <= 0 ||
      d_qk <= 0 || d_v <= 0 || head_q % head_kv != 0 || out == NULL)
    return -1;
  if (rows == NULL) n_rows = (int64_t)batch * q_len * head_q;
  if (n_rows == 0) return 0;
  const int group = head_q / head_kv;
  int failed = 0;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif

#pragma omp parallel reduction(| : failed)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
    double* qd = (double*)malloc(sizeof(double) * (size_t)d_qk);
    if (s == NULL || qd == NULL) {
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < n_rows; ++r) {
        int64_t b, i, h;
        if (rows) {
          b = rows[3 * r];
          i = rows[3 * r + 1];
          h = rows[3 * r + 2];
        } else {
          h = r % head_q;
          i = (r / head_q) % q_len;
          b = r / ((int64_t)head_q * q_len);
        }
        double* o = out + r * d_v;
        double* p = probs ? probs + r * kv_len : NULL;
        for (int c = 0; c < d_v; ++c) o[c] = 0.0;
        if (p)
          for (int64_t j = 0; j < kv_len; ++j) p[j] = 0.0;

        /* last visible key of this row */
        int64_t last = kv_len - 1;
        if (causal && i + (int64_t)kv_len - q_len < last) last = i + (int64_t)kv_len - q_len;
        if (last < 0) {
          if (lse) lse[r] = -INFINITY;
          continue;
        }
        const int64_t g = h / group;
        const int64_t q_off = ((b * q_len + i) * head_q + h) * d_qk;
        for (int d = 0; d < d_qk; ++d) qd[d] = load_elem(q, q_dtype, q_off + d) * q_scale;

        /* pass 1: scores and their maximum */
        double m = -INFINITY;
        for (int64_t j = 0; j <= last; ++j) {
          const int64_t k_off = ((b * kv_len + j) * head_kv + g) * d_qk;
          double acc = 0.0;
          for (int d = 0; d < d_qk; ++d) acc += qd[d] * (load_elem(k, kv_dtype, k_off + d) * k_scale);
          s[j] = scale * acc;
          if (s[j] > m) m = s[j];
        }
        /* pass 2: exponentials, their sum, and the weighted sum of V rows */
        double l = 0.0;
        for (int64_t j = 0; j <= last; ++j) {
          s[j] = exp(s[j] - m);
          l += s[j];
        }
        for (int64_t j = 0; j <= last; ++j) {
          const double w = s[j] / l;
          const int64_t v_off = ((b * kv_len + j) * head_kv + g) * d_v;
          for (int c = 0; c < d_v; ++c) o[c] += w * (load_elem(v, kv_dtype, v_off + c) * v_scale);
          if (p) p[j] = w;
        }
        if (lse) lse[r] = m + log(l);
      }
    }
    free(s);
    free(qd);
  }
  return failed ? -2 : 0;
}

/* Number of threads an OpenMP parallel region would use right now. */
int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
