/*
 * CPU oracle for paged decode attention, plain C, float64.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests and by the bench's CPU-baseline
 * leg, never by the product path. It shares no code with the HIP library.
 *
 * For each sequence i and query head h it walks positions p < seq_lens[i],
 * dereferences the block table at p / block_size and reads the row at offset
 * p % block_size (the per-position lookup of the single-decode-step
 * pseudo-code on the zenaique.com page "Walk through paged attention end to
 * end ..."), then computes an exact softmax over the scaled scores and the
 * weighted sum of V rows. Query head h reads KV head h / (Hq / Hkv).
 * seq_len 0 gives zeros. Inputs are fp32 values, bf16 bit patterns or (for
 * 8-bit pools) FP8 E4M3 codes with one scale per pool, converted exactly to
 * double. Plain scalar loops; OpenMP splits the
 * (sequence, query head) pairs over threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Value of one FP8 E4M3 code (OCP "fn" variant): sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits; exponent 0 holds the subnormals m * 2^-9,
 * S.1111.111 is NaN, and there are no infinities. */
static double e4m3_value(uint8_t code) {
  const double sign = (code & 0x80) ? -1.0 : 1.0;
  const int e = (code >> 3) & 0xF, m = code & 0x7;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0) return sign * (double)m * ldexp(1.0, -9);
  return sign * (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);
}

/* Element idx of an array of dtype 0 (float32), 1 (bf16 bit patterns) or 2
 * (FP8 E4M3 codes), converted exactly to double. */
static double load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == 0) return (double)((const float*)base)[idx];
  if (dtype == 2) return e4m3_value(((const uint8_t*)base)[idx]);
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* The decode over q of q_dtype and pools of kv_dtype whose elements read as
 * their value times k_mul (K) or v_mul (V). Returns 0 on success, -1 on bad
 * arguments, -2 on a block id outside the pool, -3 on allocation failure.
 * `out` is [B][Hq][D] double. */
static int decode_impl(const void* q, int q_dtype, const void* k_pool, const void* v_pool,
                       int kv_dtype, double k_mul, double v_mul, const int32_t* block_tables,
                       int max_blocks, const int32_t* seq_lens, int num_seqs, int num_q_heads,
                       int num_kv_heads, int head_dim, int block_size, int num_blocks,
                       float scale, double* out, int num_threads) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return -1;
  if (head_dim <= 0 || block_size <= 0) return -1;
  const int group = num_q_heads / num_kv_heads;
  const int64_t n_pairs = (int64_t)num_seqs * num_q_heads;
  int err = 0;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
  for (int64_t pair = 0; pair < n_pairs; ++pair) {
    const int i = (int)(pair / num_q_heads);
    const int h = (int)(pair % num_q_heads);
    const int g = h / group;
    const int L = seq_lens[i];
    double* o = out + pair * head_dim;
    for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
    if (L <= 0) continue;
    if ((L + block_size - 1) / block_size > max_blocks) { err = -1; continue; }
    double* scores = (double*)malloc(sizeof(double) * (size_t)L);
    double* qv = (double*)malloc(sizeof(double) * (size_t)head_dim);
    if (!scores || !qv) { free(scores); free(qv); err = -3; continue; }
    for (int d = 0; d < head_dim; ++d) qv[d] = load_elem(q, pair * head_dim + d, q_dtype);
    double m = -INFINITY;
    int bad = 0;
    for (int p = 0; p < L; ++p) {
      const int32_t phys = block_tables[(int64_t)i * max_blocks + p / block_size];
      const int off = p % block_size;
      if (phys < 0 || phys >= num_blocks) { bad = 1; break; }
      const int64_t row = (((int64_t)phys * num_kv_heads + g) * block_size + off) * head_dim;
      double s = 0.0;
      for (int d = 0; d < head_dim; ++d)
        s += qv[d] * (load_elem(k_pool, row + d, kv_dtype) * k_mul);
      s *= (double)scale;
      scores[p] = s;
      if (s > m) m = s;
    }
    if (bad) { free(scores); free(qv); err = -2; continue; }
    double denom = 0.0;
    for (int p = 0; p < L; ++p) {
      const double w = exp(scores[p] - m);
      denom += w;
      const int32_t phys = block_tables[(int64_t)i * max_blocks + p / block_size];
      const int off = p % block_size;
      const int64_t row = (((int64_t)phys * num_kv_heads + g) * block_size + off) * head_dim;
      for (int d = 0; d < head_dim; ++d)
        o[d] += w * (load_elem(v_pool, row + d, kv_dtype) * v_mul);
    }
    for (int d = 0; d < head_dim; ++d) o[d] /= denom;
    free(scores);
    free(qv);
  }
  return err;
}

/* q, pools and the decode of one dtype: 0 float32, 1 bf16. */
int pa_oracle_decode(const void* q, const void* k_pool, const void* v_pool, int dtype,
                     const int32_t* block_tables, int max_blocks, const int32_t* seq_lens,
                     int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int num_blocks, float scale, double* out,
                     int num_threads) {
  if (dtype != 0 && dtype != 1) return -1;
  return decode_impl(q, dtype, k_pool, v_pool, dtype, 1.0, 1.0, block_tables, max_blocks,
                     seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, scale, out, num_threads);
}

/* 8-bit pools: q in bf16, pools of FP8 E4M3 codes; attention reads each K
 * element as code value * k_scale and each V element as code value *
 * v_scale (the scales taken as their float32 values). */
int pa_oracle_decode_e4m3(const void* q, const void* k_codes, const void* v_codes,
                          float k_scale, float v_scale, const int32_t* block_tables,
                          int max_blocks, const int32_t* seq_lens, int num_seqs,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int num_blocks, float scale, double* out, int num_threads) {
  return decode_impl(q, 1, k_codes, v_codes, 2, (double)k_scale, (double)v_scale,
                     block_tables, max_blocks, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, scale, out, num_threads);
}

/* Number of threads an OpenMP parallel region would use. */
int pa_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
