/*
 * Oracle for paged decode attention and KV append.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do. It shares no code, header or constant with the HIP path.
 *
 * Every function is plain, slow and written to be checked by eye against the
 * pages it follows:
 *
 *   - "Solving the LLM Memory Wall: A Deep Dive into PagedAttention",
 *     section "1. The Mathematical Foundation": the attention output is
 *     ordinary scaled dot-product attention, a_j = q . k_j * scale and
 *     o = sum_j softmax_j(a) v_j, over the tokens of the sequence; paging only
 *     changes where k_j and v_j are fetched from.
 *   - "PagedAttention: Virtual Memory Guide for LLM Inference", section "The
 *     Mathematics of Block Translation": token i of a sequence lives in
 *     logical block floor(i / B) at offset i mod B, and the block table maps
 *     the logical block to a physical frame.
 *   - Same page 2, "Implementation": the cache is two tensors
 *     [num_blocks, block_size, heads, head_dim] (K and V), and writing one
 *     token stores its [heads, head_dim] row at [frame, offset].
 *
 * Arithmetic is fp64 throughout. Stored fp32 / fp16 / bf16 elements are
 * widened exactly, each decoded from its format definition (sign, biased
 * exponent, fraction) with ldexp, so nothing is rounded before accumulation.
 * The softmax is the exact two-pass form: maximum, exponentials, sum, divide.
 * Sums run over tokens in logical order.
 *
 * Parity status: every exported function is pinned by the CPU test-suite
 * (worked examples from the pages, closed forms, invariants and a rational
 * brute force), so none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage dtype codes used by this oracle's interface. */
#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2

#define ORACLE_OK 0
#define ORACLE_BAD_ARG -1
#define ORACLE_BAD_FRAME -2
#define ORACLE_NO_MEMORY -3

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1F;
  int frac = h & 0x3FF;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24); /* subnormal: frac * 2^(1-15-10) */
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/2^10) * 2^(expo-15) */
  }
  return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
static double decode_bf16(uint16_t b) {
  int sign = (b >> 15) & 1;
  int expo = (b >> 7) & 0xFF;
  int frac = b & 0x7F;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -133); /* subnormal: frac * 2^(1-127-7) */
  } else if (expo == 255) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(128 + frac), expo - 134); /* (1 + frac/2^7) * 2^(expo-127) */
  }
  return sign ? -mag : mag;
}

static size_t elem_size(int dtype) { return dtype == ORACLE_F32 ? 4 : 2; }

/* Element idx of an array stored in dtype, widened exactly to double. */
static double load(const void* base, int dtype, int64_t idx) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
  if (dtype == ORACLE_F16) return decode_f16(((const uint16_t*)base)[idx]);
  return decode_bf16(((const uint16_t*)base)[idx]);
}

static int valid_dtype(int dtype) {
  return dtype == ORACLE_F32 || dtype == ORACLE_F16 || dtype == ORACLE_BF16;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the following calls use (n >= 1); for timing the oracle. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Softmax attention of one query over n key/value rows (definition above).
 * q[e], key(j)[e] and val(j)[e] are given as strided views of stored arrays:
 * element e of row j is at row_off[j] + e. Writes out[0..D).
 */
static void attend_rows(const void* q, int64_t q_off, const void* kc, const void* vc,
                        const int64_t* row_off, int64_t n, int D, double scale,
                        int dtype, double* a, double* out) {
  if (n <= 0) {
    for (int e = 0; e < D; ++e) out[e] = 0.0;
    return;
  }
  for (int64_t j = 0; j < n; ++j) {
    double dot = 0.0;
    for (int e = 0; e < D; ++e) dot += load(q, dtype, q_off + e) * load(kc, dtype, row_off[j] + e);
    a[j] = scale * dot;
  }
  double m = a[0];
  for (int64_t j = 1; j < n; ++j)
    if (a[j] > m) m = a[j];
  double z = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    a[j] = exp(a[j] - m);
    z += a[j];
  }
  for (int e = 0; e < D; ++e) {
    double acc = 0.0;
    for (int64_t j = 0; j < n; ++j) acc += a[j] * load(vc, dtype, row_off[j] + e);
    out[e] = acc / z;
  }
}

/*
 * Paged decode attention.
 *
 *   q            [S, H, D] stored dtype
 *   k_cache      [NB, B, H, D] stored dtype (frame, offset, head, element)
 *   v_cache      [NB, B, H, D]
 *   block_tables [S, max_blocks] int32: logical block -> physical frame
 *   context_lens [S] int32: tokens of each sequence (the query's own included)
 *   out          [S, H, D] double
 *
 * For each sequence s and head h, token i (0 <= i < ctx) is read from frame
 * block_tables[s][i / B] at offset i % B. ctx <= 0 gives a zero output.
 * Returns ORACLE_BAD_FRAME if a table entry that is read lies outside
 * [0, NB), ORACLE_OK otherwise.
 */
int oracle_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int S, int H, int D, int B, int64_t NB, int max_blocks,
                        double scale, int dtype, double* out) {
  if (S < 0 || H <= 0 || D <= 0 || B <= 0 || NB <= 0 || max_blocks < 0 || !valid_dtype(dtype))
    return ORACLE_BAD_ARG;
  int status = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int s = 0; s < S; ++s) {
    for (int h = 0; h < H; ++h) {
      int64_t ctx = context_lens[s];
      double* o = out + ((int64_t)s * H + h) * D;
      if (ctx > (int64_t)max_blocks * B) {
#pragma omp atomic write
        status = ORACLE_BAD_ARG;
        continue;
      }
      int64_t* row_off = (int64_t*)malloc(sizeof(int64_t) * (ctx > 0 ? ctx : 1));
      double* a = (double*)malloc(sizeof(double) * (ctx > 0 ? ctx : 1));
      if (!row_off || !a) {
        free(row_off);
        free(a);
#pragma omp atomic write
        status = ORACLE_NO_MEMORY;
        continue;
      }
      int bad = 0;
      for (int64_t i = 0; i < ctx; ++i) {
        int64_t b = i / B;       /* logical block */
        int64_t off = i % B;     /* offset inside the block */
        int64_t f = block_tables[(int64_t)s * max_blocks + b];
        if (f < 0 || f >= NB) {
          bad = 1;
          break;
        }
        row_off[i] = ((f * B + off) * H + h) * D;
      }
      if (bad) {
#pragma omp atomic write
        status = ORACLE_BAD_FRAME;
      } else {
        attend_rows(q, ((int64_t)s * H + h) * D, k_cache, v_cache, row_off, ctx, D, scale,
                    dtype, a, o);
      }
      free(row_off);
      free(a);
    }
  }
  return status;
}

/*
 * Contiguous (unpaged) attention: the same definition over keys and values
 * stored back to back per sequence.
 *
 *   q       [S, H, D]
 *   k, v    [T, H, D] with sequence s owning rows seq_start[s] .. seq_start[s+1]-1
 *   out     [S, H, D] double
 */
int oracle_dense_attention(const void* q, const void* k, const void* v, const int64_t* seq_start,
                           int S, int H, int D, double scale, int dtype, double* out) {
  if (S < 0 || H <= 0 || D <= 0 || !valid_dtype(dtype)) return ORACLE_BAD_ARG;
  int status = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int s = 0; s < S; ++s) {
    for (int h = 0; h < H; ++h) {
      int64_t n = seq_start[s + 1] - seq_start[s];
      int64_t* row_off = (int64_t*)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
      double* a = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
      if (!row_off || !a) {
        free(row_off);
        free(a);
#pragma omp atomic write
        status = ORACLE_NO_MEMORY;
        continue;
      }
      for (int64_t j = 0; j < n; ++j) row_off[j] = ((seq_start[s] + j) * H + h) * D;
      attend_rows(q, ((int64_t)s * H + h) * D, k, v, row_off, n, D, scale, dtype, a,
                  out + ((int64_t)s * H + h) * D);
      free(row_off);
      free(a);
    }
  }
  return status;
}

/*
 * Causal multi-query (prefill) attention through the block tables.
 *
 *   q            [T, H, D]: sequence s owns rows query_start[s] .. query_start[s+1]-1
 *   query_start  [S + 1] int32, non-decreasing, query_start[0] = 0
 *   out          [T, H, D] double
 *
 * The n_s queries of sequence s are its last n_s tokens: query r sits at
 * position p = ctx_s - n_s + r and attends to tokens 0 .. p, the causal sum
 * o_i = sum_{j <= i} softmax_j(a_ij) v_j of "Solving the LLM Memory Wall"
 * ("1. The Mathematical Foundation"), each token fetched through the table as
 * in oracle_paged_decode. Requires n_s <= ctx_s.
 */
int oracle_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_start, int S, int H, int D, int B, int64_t NB,
                         int max_blocks, double scale, int dtype, double* out) {
  if (S < 0 || H <= 0 || D <= 0 || B <= 0 || NB <= 0 || max_blocks < 0 || !valid_dtype(dtype))
    return ORACLE_BAD_ARG;
  for (int s = 0; s < S; ++s) {
    int64_t n = (int64_t)query_start[s + 1] - query_start[s];
    if (n < 0 || n > context_lens[s] || context_lens[s] > (int64_t)max_blocks * B) return ORACLE_BAD_ARG;
  }
  int status = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int s = 0; s < S; ++s) {
    for (int h = 0; h < H; ++h) {
      int64_t ctx = context_lens[s];
      int64_t n = (int64_t)query_start[s + 1] - query_start[s];
      int64_t* row_off = (int64_t*)malloc(sizeof(int64_t) * (ctx > 0 ? ctx : 1));
      double* a = (double*)malloc(sizeof(double) * (ctx > 0 ? ctx : 1));
      if (!row_off || !a) {
        free(row_off);
        free(a);
#pragma omp atomic write
        status = ORACLE_NO_MEMORY;
        continue;
      }
      int bad = 0;
      for (int64_t i = 0; i < ctx; ++i) {
        int64_t f = block_tables[(int64_t)s * max_blocks + i / B];
        if (f < 0 || f >= NB) {
          bad = 1;
          break;
        }
        row_off[i] = ((f * B + i % B) * H + h) * D;
      }
      if (bad) {
#pragma omp atomic write
        status = ORACLE_BAD_FRAME;
      } else {
        for (int64_t r = 0; r < n; ++r) {
          int64_t t = query_start[s] + r;        /* query row */
          int64_t pos = ctx - n + r;              /* its position in the sequence */
          attend_rows(q, (t * H + h) * D, k_cache, v_cache, row_off, pos + 1, D, scale, dtype, a,
                      out + (t * H + h) * D);
        }
      }
      free(row_off);
      free(a);
    }
  }
  return status;
}

/*
 * Attention computed over context partitions of P tokens and merged by the
 * log-sum-exp rule: partition p yields m_p = max a, l_p = sum exp(a - m_p),
 * acc_p = sum exp(a - m_p) v; then with M = max_p m_p,
 * o = sum_p exp(m_p - M) acc_p / sum_p exp(m_p - M) l_p.
 * This is an exact rewriting of the softmax; it exists to pin that algebra
 * against oracle_paged_decode. Inputs as for oracle_paged_decode.
 */
int oracle_paged_decode_split(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int S, int H, int D, int B, int64_t NB, int max_blocks,
                              double scale, int dtype, int P, double* out) {
  if (S < 0 || H <= 0 || D <= 0 || B <= 0 || NB <= 0 || P <= 0 || !valid_dtype(dtype))
    return ORACLE_BAD_ARG;
  int status = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int s = 0; s < S; ++s) {
    for (int h = 0; h < H; ++h) {
      int64_t ctx = context_lens[s];
      double* o = out + ((int64_t)s * H + h) * D;
      int64_t nparts = (ctx + P - 1) / P;
      double* m = (double*)malloc(sizeof(double) * (nparts > 0 ? nparts : 1));
      double* l = (double*)malloc(sizeof(double) * (nparts > 0 ? nparts : 1));
      double* acc = (double*)calloc((size_t)(nparts > 0 ? nparts : 1) * D, sizeof(double));
      double* a = (double*)malloc(sizeof(double) * P);
      if (!m || !l || !acc || !a) {
        free(m); free(l); free(acc); free(a);
#pragma omp atomic write
        status = ORACLE_NO_MEMORY;
        continue;
      }
      int bad = 0;
      for (int64_t p = 0; p < nparts && !bad; ++p) {
        int64_t lo = p * P, hi = lo + P < ctx ? lo + P : ctx;
        for (int64_t i = lo; i < hi; ++i) {
          int64_t f = block_tables[(int64_t)s * max_blocks + i / B];
          if (f < 0 || f >= NB) { bad = 1; break; }
          int64_t row = ((f * B + i % B) * H + h) * D;
          double dot = 0.0;
          for (int e = 0; e < D; ++e)
            dot += load(q, dtype, ((int64_t)s * H + h) * D + e) * load(k_cache, dtype, row + e);
          a[i - lo] = scale * dot;
        }
        if (bad) break;
        m[p] = a[0];
        for (int64_t i = 1; i < hi - lo; ++i) if (a[i] > m[p]) m[p] = a[i];
        l[p] = 0.0;
        for (int64_t i = lo; i < hi; ++i) {
          int64_t f = block_tables[(int64_t)s * max_blocks + i / B];
          int64_t row = ((f * B + i % B) * H + h) * D;
          double w = exp(a[i - lo] - m[p]);
          l[p] += w;
          for (int e = 0; e < D; ++e) acc[p * D + e] += w * load(v_cache, dtype, row + e);
        }
      }
      if (bad) {
#pragma omp atomic write
        status = ORACLE_BAD_FRAME;
      } else if (nparts == 0) {
        for (int e = 0; e < D; ++e) o[e] = 0.0;
      } else {
        double M = m[0];
        for (int64_t p = 1; p < nparts; ++p) if (m[p] > M) M = m[p];
        double L = 0.0;
        for (int64_t p = 0; p < nparts; ++p) L += exp(m[p] - M) * l[p];
        for (int e = 0; e < D; ++e) {
          double num = 0.0;
          for (int64_t p = 0; p < nparts; ++p) num += exp(m[p] - M) * acc[p * D + e];
          o[e] = num / L;
        }
      }
      free(m); free(l); free(acc); free(a);
    }
  }
  return status;
}

/*
 * KV append: for token n with slot_mapping[n] = slot >= 0, copy the bytes of
 * k_new[n] and v_new[n] (each [H, D]) into frame slot / B at offset slot % B
 * of k_cache and v_cache. A negative slot is skipped. Returns
 * ORACLE_BAD_FRAME if a slot lies past the pool (nothing is written for it).
 */
int oracle_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                     int64_t N, int H, int D, int B, int64_t NB, int dtype,
                     void* k_cache, void* v_cache) {
  if (N < 0 || H <= 0 || D <= 0 || B <= 0 || NB <= 0 || !valid_dtype(dtype)) return ORACLE_BAD_ARG;
  size_t row_bytes = (size_t)H * D * elem_size(dtype);
  int status = ORACLE_OK;
  for (int64_t n = 0; n < N; ++n) {
    int64_t slot = slot_mapping[n];
    if (slot < 0) continue;
    int64_t frame = slot / B, off = slot % B;
    if (frame >= NB) {
      status = ORACLE_BAD_FRAME;
      continue;
    }
    size_t dst = (size_t)(frame * B + off) * row_bytes;
    memcpy((char*)k_cache + dst, (const char*)k_new + (size_t)n * row_bytes, row_bytes);
    memcpy((char*)v_cache + dst, (const char*)v_new + (size_t)n * row_bytes, row_bytes);
  }
  return status;
}

/*
 * Block translation as a gather: for each sequence s, rows
 * cache[block_tables[s][i / B]][i % B] for i < context_lens[s] are copied
 * into out, sequences back to back ([sum ctx, H, D], stored dtype).
 */
int oracle_gather(const void* cache, const int32_t* block_tables, const int32_t* context_lens,
                  int S, int H, int D, int B, int64_t NB, int max_blocks, int dtype, void* out) {
  if (S < 0 || H <= 0 || D <= 0 || B <= 0 || NB <= 0 || !valid_dtype(dtype)) return ORACLE_BAD_ARG;
  size_t row_bytes = (size_t)H * D * elem_size(dtype);
  int64_t dst_row = 0;
  for (int s = 0; s < S; ++s) {
    for (int64_t i = 0; i < context_lens[s]; ++i) {
      int64_t f = block_tables[(int64_t)s * max_blocks + i / B];
      if (f < 0 || f >= NB) return ORACLE_BAD_FRAME;
      memcpy((char*)out + (size_t)dst_row * row_bytes,
             (const char*)cache + (size_t)(f * B + i % B) * row_bytes, row_bytes);
      ++dst_row;
    }
  }
  return ORACLE_OK;
}

/* Exact widening of n stored elements to double (used by host-side checks). */
int oracle_widen(const void* src, int64_t n, int dtype, double* dst) {
  if (n < 0 || !valid_dtype(dtype)) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < n; ++i) dst[i] = load(src, dtype, i);
  return ORACLE_OK;
}
