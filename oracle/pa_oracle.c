/*
 * pa_oracle.c -- CPU oracle for paged attention.  TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct model of what the paged-attention path
 * computes, in double precision.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the HIP library never calls it and
 * the two share no source, header, table or helper.
 *
 * What it follows (page title, then section):
 *  - Attention: paper notes "PagedAttention: Efficient Memory Management for
 *    Large Language Model Serving with PagedAttention" (unpurerationalist.github.io),
 *    section 3.1, block-wise attention equation: the weight of a key is
 *    exp(q.k/sqrt(d)) over the sum of exp(q.k'/sqrt(d)) over every valid key
 *    of every block, and the output is the weight-sum of the values.  The
 *    Korean review (mz-moonzoo.tistory.com/116, section 4.1 "PagedAttention")
 *    gives the same numerator / denominator / weighted sum.
 *  - Position -> slot: "KV 캐시 관리와 PagedAttention"
 *    (llm-systems-engineering.pages.dev), section on linking token order to
 *    storage: logical block = pos / B, offset = pos % B, then the block table
 *    maps the logical block to a physical block; all counts start at 0.
 *  - Valid positions: same page, section on attention over scattered KV: the
 *    current token's own K/V take part, and slots past the context length (and
 *    other requests' blocks) do not.
 *  - Cache write: review section 5.1 (fused reshape and block write): new K/V
 *    rows go to the slot the block table gives.
 *  - Block copy: "KV 캐시 관리와 PagedAttention", copy-on-write section: the
 *    whole shared block is copied into a freshly allocated block, keeping the
 *    K/V already in it.
 *
 * Readings where the pages are silent: a sequence with zero context produces a
 * zero output; a negative slot in a slot mapping means "skip this token";
 * duplicate slots, duplicate copy destinations, or a destination that is also a
 * source are rejected; a prefill query j of a chunk that starts after c cached
 * tokens sees positions 0..c+j.
 *
 * Layouts: caches [num_blocks][num_heads][block_size][head_dim]; q and outputs
 * [rows][num_heads][head_dim]; block tables [num_seqs][max_blocks] int32;
 * context lengths int32; slot and block mappings int64.  Element types:
 * 0 = fp32, 1 = fp16, 2 = bf16 (bit patterns).  Softmax is the two-pass form
 * (max, then exponentials and their sum) in double precision.
 *
 * Error codes: 0 ok, -1 table entry outside the pool, -2 slot outside the
 * pool, -3 duplicate slot, -4 bad copy mapping, -5 bad argument,
 * -6 out of memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

/* IEEE binary16 -> double, from the format's definition:
 * sign | 5-bit exponent (bias 15) | 10-bit fraction. */
static double half_to_double(uint16_t h) {
  int negative = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double mag;
  if (e == 0) {
    mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 * 2^-10 */
  } else if (e == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(1024 + frac), e - 25); /* 1.frac * 2^(e-15) */
  }
  return negative ? -mag : mag;
}

/* bf16 is the upper half of an IEEE binary32. */
static double bf16_to_double(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double element(const void *base, int64_t index, int dtype) {
  if (dtype == ORACLE_F32) return (double)((const float *)base)[index];
  uint16_t raw = ((const uint16_t *)base)[index];
  return dtype == ORACLE_F16 ? half_to_double(raw) : bf16_to_double(raw);
}

static int element_bytes(int dtype) { return dtype == ORACLE_F32 ? 4 : 2; }

/* Widen n stored elements to double (exposed so tests can pin the decoding). */
int oracle_to_f64(double *out, const void *in, int64_t n, int dtype) {
  if (dtype < 0 || dtype > 2 || n < 0) return -5;
  for (int64_t i = 0; i < n; ++i) out[i] = element(in, i, dtype);
  return 0;
}

/* Logical position -> flat cache slot (physical block * B + offset). */
int64_t oracle_slot(const int32_t *table_row, int64_t position, int32_t block_size) {
  int64_t logical_block = position / block_size;
  int64_t offset_in_block = position % block_size;
  return (int64_t)table_row[logical_block] * block_size + offset_in_block;
}

/* Element index of (flat slot, head, dim 0) in a [N][H][B][D] cache. */
static int64_t cache_row(int64_t slot, int32_t head, int32_t num_heads, int32_t block_size,
                         int32_t head_dim) {
  int64_t physical_block = slot / block_size;
  int64_t offset_in_block = slot % block_size;
  return ((physical_block * num_heads + head) * block_size + offset_in_block) * head_dim;
}

/*
 * Attention of one query row (head `head`) over the first n positions of one
 * sequence.  logits is caller scratch of at least n doubles.
 */
static int attend_one(double *out, const void *q, int64_t q_row, const void *k_cache,
                      const void *v_cache, const int32_t *table_row, int64_t n, int32_t head,
                      int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                      double scale, int dtype, double *logits) {
  if (n == 0) {
    for (int32_t d = 0; d < head_dim; ++d) out[d] = 0.0;
    return 0;
  }
  /* 1. gather each valid key through the block table and score it */
  for (int64_t pos = 0; pos < n; ++pos) {
    int32_t physical = table_row[pos / block_size];
    if (physical < 0 || physical >= num_blocks) return -1;
    int64_t k_row = cache_row(oracle_slot(table_row, pos, block_size), head, num_heads,
                              block_size, head_dim);
    double dot = 0.0;
    for (int32_t d = 0; d < head_dim; ++d)
      dot += element(q, q_row + d, dtype) * element(k_cache, k_row + d, dtype);
    logits[pos] = scale * dot;
  }
  /* 2. softmax over exactly n positions: max, exponentials, their sum */
  double max_logit = logits[0];
  for (int64_t pos = 1; pos < n; ++pos)
    if (logits[pos] > max_logit) max_logit = logits[pos];
  double denom = 0.0;
  for (int64_t pos = 0; pos < n; ++pos) {
    logits[pos] = exp(logits[pos] - max_logit);
    denom += logits[pos];
  }
  /* 3. weighted sum of the values */
  for (int32_t d = 0; d < head_dim; ++d) out[d] = 0.0;
  for (int64_t pos = 0; pos < n; ++pos) {
    int64_t v_row = cache_row(oracle_slot(table_row, pos, block_size), head, num_heads,
                              block_size, head_dim);
    for (int32_t d = 0; d < head_dim; ++d) out[d] += logits[pos] * element(v_cache, v_row + d, dtype);
  }
  for (int32_t d = 0; d < head_dim; ++d) out[d] /= denom;
  return 0;
}

static void set_threads(int32_t threads) {
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
}

/* Threads an OpenMP region would use now (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Decode: one query per sequence.  out is double [num_seqs][num_heads][head_dim].
 */
int oracle_decode(double *out, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, int32_t max_blocks, const int32_t *context_lens,
                  int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size,
                  int64_t num_blocks, double scale, int32_t dtype, int32_t threads) {
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || dtype < 0 || dtype > 2)
    return -5;
  int64_t longest = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (context_lens[s] < 0 || context_lens[s] > (int64_t)max_blocks * block_size) return -5;
    if (context_lens[s] > longest) longest = context_lens[s];
  }
  set_threads(threads);
  int status = 0;
#pragma omp parallel
  {
    double *logits = (double *)malloc(sizeof(double) * (size_t)(longest > 0 ? longest : 1));
    if (!logits) {
#pragma omp atomic write
      status = -6;
    }
#pragma omp for collapse(2) schedule(dynamic)
    for (int32_t s = 0; s < num_seqs; ++s)
      for (int32_t h = 0; h < num_heads; ++h) {
        if (!logits) continue;
        int64_t row = ((int64_t)s * num_heads + h) * head_dim;
        int rc = attend_one(out + row, q, row, k_cache, v_cache,
                            block_tables + (int64_t)s * max_blocks, context_lens[s], h, num_heads,
                            head_dim, block_size, num_blocks, scale, dtype, logits);
        if (rc) {
#pragma omp atomic write
          status = rc;
        }
      }
    free(logits);
  }
  return status;
}

/*
 * Chunked prefill: sequence s owns query rows cu_q_lens[s]..cu_q_lens[s+1]-1;
 * context_lens[s] counts the cached tokens plus the chunk, so the chunk starts
 * at c = context_lens[s] - q_len and query j sees positions 0..c+j.
 * out is double [total_queries][num_heads][head_dim].
 */
int oracle_prefill_chunk(double *out, const void *q, const int32_t *cu_q_lens, const void *k_cache,
                         const void *v_cache, const int32_t *block_tables, int32_t max_blocks,
                         const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                         int32_t head_dim, int32_t block_size, int64_t num_blocks, double scale,
                         int32_t dtype, int32_t threads) {
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || dtype < 0 || dtype > 2)
    return -5;
  int64_t longest = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int64_t q_len = (int64_t)cu_q_lens[s + 1] - cu_q_lens[s];
    if (q_len < 0 || q_len > context_lens[s]) return -5;
    if (context_lens[s] > (int64_t)max_blocks * block_size) return -5;
    if (context_lens[s] > longest) longest = context_lens[s];
  }
  set_threads(threads);
  int status = 0;
#pragma omp parallel
  {
    double *logits = (double *)malloc(sizeof(double) * (size_t)(longest > 0 ? longest : 1));
    if (!logits) {
#pragma omp atomic write
      status = -6;
    }
#pragma omp for collapse(2) schedule(dynamic)
    for (int32_t s = 0; s < num_seqs; ++s)
      for (int32_t h = 0; h < num_heads; ++h) {
        if (!logits) continue;
        int64_t first = cu_q_lens[s];
        int64_t q_len = (int64_t)cu_q_lens[s + 1] - first;
        int64_t cached = (int64_t)context_lens[s] - q_len;
        for (int64_t j = 0; j < q_len; ++j) {
          int64_t row = ((first + j) * num_heads + h) * head_dim;
          int rc = attend_one(out + row, q, row, k_cache, v_cache,
                              block_tables + (int64_t)s * max_blocks, cached + j + 1, h, num_heads,
                              head_dim, block_size, num_blocks, scale, dtype, logits);
          if (rc) {
#pragma omp atomic write
            status = rc;
          }
        }
      }
    free(logits);
  }
  return status;
}

static int compare_i64(const void *a, const void *b) {
  int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
  return (x > y) - (x < y);
}

/*
 * Cache write: for every token t with slot_mapping[t] >= 0, copy the raw bytes
 * of key[t][h][:] into k_cache at (slot / B, h, slot % B, :) for every head h,
 * and likewise value into v_cache.  key/value rows are token_stride elements
 * apart (heads are contiguous within a token).
 */
int oracle_reshape_and_cache(void *k_cache, void *v_cache, const void *key, const void *value,
                             int64_t key_token_stride, int64_t value_token_stride,
                             const int64_t *slot_mapping, int64_t num_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             int32_t dtype) {
  if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || dtype < 0 || dtype > 2)
    return -5;
  int64_t *sorted = (int64_t *)malloc(sizeof(int64_t) * (size_t)(num_tokens ? num_tokens : 1));
  if (!sorted) return -6;
  int64_t kept = 0;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    if (slot >= num_blocks * block_size) {
      free(sorted);
      return -2;
    }
    sorted[kept++] = slot;
  }
  qsort(sorted, (size_t)kept, sizeof(int64_t), compare_i64);
  for (int64_t i = 1; i < kept; ++i)
    if (sorted[i] == sorted[i - 1]) {
      free(sorted);
      return -3;
    }
  free(sorted);
  const int eb = element_bytes(dtype);
  const size_t row_bytes = (size_t)head_dim * eb;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    for (int32_t h = 0; h < num_heads; ++h) {
      int64_t dst = cache_row(slot, h, num_heads, block_size, head_dim);
      memcpy((char *)k_cache + dst * eb, (const char *)key + (t * key_token_stride + (int64_t)h * head_dim) * eb,
             row_bytes);
      memcpy((char *)v_cache + dst * eb,
             (const char *)value + (t * value_token_stride + (int64_t)h * head_dim) * eb, row_bytes);
    }
  }
  return 0;
}

/*
 * Block copy: for every layer l and every pair (src, dst) of block_mapping,
 * copy the whole block (block_bytes bytes, all heads and all slots) from
 * src to dst in k_caches[l] and in v_caches[l].  Destinations must be distinct
 * and must not be sources, which makes the result independent of order.
 */
int oracle_copy_blocks(void *const *k_caches, void *const *v_caches, int32_t num_layers,
                       const int64_t *block_mapping, int64_t num_pairs, int64_t block_bytes,
                       int64_t num_blocks) {
  if (num_layers < 0 || num_pairs < 0 || block_bytes <= 0) return -5;
  for (int64_t i = 0; i < num_pairs; ++i) {
    int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return -4;
    for (int64_t j = 0; j < num_pairs; ++j) {
      if (j != i && block_mapping[2 * j + 1] == dst) return -4; /* repeated destination */
      if (block_mapping[2 * j] == dst) return -4;               /* destination is a source */
    }
  }
  for (int32_t l = 0; l < num_layers; ++l)
    for (int64_t i = 0; i < num_pairs; ++i) {
      int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
      memcpy((char *)k_caches[l] + dst * block_bytes, (const char *)k_caches[l] + src * block_bytes,
             (size_t)block_bytes);
      memcpy((char *)v_caches[l] + dst * block_bytes, (const char *)v_caches[l] + src * block_bytes,
             (size_t)block_bytes);
    }
  return 0;
}
