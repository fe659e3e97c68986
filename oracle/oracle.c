/*
 * oracle.c — plain fp64 CPU oracle for single-token paged decode attention,
 * the plain byte-level definition of the two cache writes around it
 * (appending a decode token, copy-on-write block copy) and the block-wise
 * eviction scores (end of this file).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source, header or helper with the
 * gfx950 library.
 *
 * What it computes, following the pages step by step:
 *
 *  "39 · PagedAttention", §2 "The paged version":
 *    1. walk the logical blocks of the request in order, following the
 *       block table to each physical block, and score every key in it;
 *    2. with all scores in hand, apply one softmax over all of them;
 *    3. walk the blocks again and sum the values weighted by the softmax.
 *  The same page (§1, the IMPORTANT box) states that the result is ordinary
 *  attention softmax(q K^T * scale) V over the request's tokens in logical
 *  order ("FlashAttention vs PagedAttention", "What does FlashAttention
 *  optimize?" gives softmax(QK^T/sqrt(d))V).  So this oracle gathers each
 *  (sequence, KV head)'s tokens through the table into contiguous fp64 rows
 *  and runs the textbook two-pass softmax on them, in logical token order.
 *
 *  Merge of partials ("39 · PagedAttention", §3 "On the GPU", the merge
 *  equation, printed garbled with its two equations run together): two
 *  partial results over disjoint token sets, each holding its largest score
 *  m, its sum of exponentials l = sum exp(s - m) and its unnormalised
 *  weighted value sum o = sum exp(s - m) v, combine as
 *      m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m), o = o1 e^(m1-m) + o2 e^(m2-m)
 *  and out = o / l.  The page prints only the m and l lines; the o line is
 *  the reading that makes out = o / l equal the one-softmax result.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - query head h reads KV head h / (Hq / Hkv) (consecutive grouping);
 *  - tokens 0 .. L-1 of the table are attended, nothing else (no mask is
 *    needed for a single decode query);
 *  - slots of the last block beyond L are not part of the result;
 *  - L = 0 gives an all-zero output;
 *  - an empty partial is (m = -inf, l = 0, o = 0) and is the identity of
 *    the merge.
 *
 * Storage layouts it reads (the library defines them; restated here from
 * their definition, not shared):
 *    q        [S][Hq][D]
 *    k_pool   [num_blocks][Hkv][B][D]     (token-major tile)
 *    v_pool   [num_blocks][Hkv][B/S][D][S] (value rows transposed within
 *                                          groups of S tokens; S = 16 when
 *                                          B is a multiple of 16, else S = B)
 *    tables   int32 [S][max_blocks_per_seq]
 * Element types: 0 = IEEE binary32, 1 = IEEE binary16, 2 = bfloat16.
 * Every element is widened to fp64 exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* IEEE 754 binary16 to double, from the format: 1 sign bit, 5 exponent bits
 * (bias 15), 10 fraction bits; exponent 0 encodes subnormals
 * fraction * 2^-24, exponent 31 encodes inf / NaN. */
double oracle_f16_to_f64(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f;
  const int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(0x400 | f), e - 25); /* 1.f * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 to double: the 16 bits are the upper half of a binary32. */
double oracle_bf16_to_f64(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void* base, int dtype, int64_t i) {
  switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[i];
    case ORC_F16: return oracle_f16_to_f64(((const uint16_t*)base)[i]);
    default: return oracle_bf16_to_f64(((const uint16_t*)base)[i]);
  }
}

/* Widen n elements of `dtype` to fp64. */
void oracle_to_f64(const void* src, int32_t dtype, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = elem(src, dtype, i);
}

/* Step 1 of "The paged version": gather the L tokens of (sequence b, KV
 * head g) through the block table into contiguous fp64 K[L][D], V[L][D].
 * Returns 0, or -1 when a table entry that is read is out of range. */
int oracle_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables,
                  int32_t b, int32_t g, int64_t L, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                  int32_t max_blocks_per_seq, int32_t dtype, double* K, double* V) {
  const int64_t D = head_dim, B = block_size, H = num_kv_heads;
  const int64_t S = (B % 16 == 0) ? 16 : B; /* tokens per transposed V group */
  for (int64_t t = 0; t < L; ++t) {
    const int64_t j = t / B;    /* logical block */
    const int64_t slot = t % B; /* position inside the block */
    if (j >= max_blocks_per_seq) return -1;
    const int64_t phys = block_tables[(int64_t)b * max_blocks_per_seq + j];
    if (phys < 0 || phys >= num_blocks) return -1;
    const int64_t tile = (phys * H + g) * B * D; /* same tile base in both pools */
    for (int64_t d = 0; d < D; ++d) {
      K[t * D + d] = elem(k_pool, dtype, tile + slot * D + d);
      V[t * D + d] = elem(v_pool, dtype, tile + (slot / S) * D * S + d * S + slot % S);
    }
  }
  return 0;
}

/* Steps 2-3 on contiguous rows: scores s_t = scale * q.K[t]; one softmax
 * over all L scores (max-subtracted, two passes); out = sum_t w_t V[t].
 * `s` is caller scratch of L doubles.  L = 0 gives out = 0. */
void oracle_attention(const double* q, const double* K, const double* V, int64_t L,
                      int64_t D, double scale, double* out, double* s) {
  for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
  if (L <= 0) return;
  double m = -INFINITY;
  for (int64_t t = 0; t < L; ++t) {
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += q[d] * K[t * D + d];
    s[t] = scale * dot;
    if (s[t] > m) m = s[t];
  }
  double z = 0.0;
  for (int64_t t = 0; t < L; ++t) {
    s[t] = exp(s[t] - m);
    z += s[t];
  }
  for (int64_t t = 0; t < L; ++t) {
    const double w = s[t] / z;
    for (int64_t d = 0; d < D; ++d) out[d] += w * V[t * D + d];
  }
}

/* Partial over tokens [t0, t1) of contiguous rows: m = max score,
 * l = sum exp(s - m), o = sum exp(s - m) V[t] (not normalised).
 * An empty range gives (-inf, 0, 0). */
void oracle_partial(const double* q, const double* K, const double* V, int64_t t0,
                    int64_t t1, int64_t D, double scale, double* m_out, double* l_out,
                    double* o) {
  for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
  double m = -INFINITY;
  for (int64_t t = t0; t < t1; ++t) {
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += q[d] * K[t * D + d];
    const double s = scale * dot;
    if (s > m) m = s;
  }
  double l = 0.0;
  for (int64_t t = t0; t < t1; ++t) {
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += q[d] * K[t * D + d];
    const double p = exp(scale * dot - m);
    l += p;
    for (int64_t d = 0; d < D; ++d) o[d] += p * V[t * D + d];
  }
  *m_out = m;
  *l_out = l;
}

/* The merge equation of §3: combine two partials.  A partial with
 * m = -inf (empty) contributes nothing; merging two empties is empty. */
void oracle_merge(double m1, double l1, const double* o1, double m2, double l2,
                  const double* o2, int64_t D, double* m_out, double* l_out, double* o) {
  const double m = m1 > m2 ? m1 : m2;
  const double a1 = (m1 == -INFINITY) ? 0.0 : exp(m1 - m);
  const double a2 = (m2 == -INFINITY) ? 0.0 : exp(m2 - m);
  for (int64_t d = 0; d < D; ++d) o[d] = o1[d] * a1 + o2[d] * a2;
  *m_out = m;
  *l_out = l1 * a1 + l2 * a2;
}

/* Whole operation: out[b][h][:] in fp64 for every sequence and query head.
 * Parallel over (sequence, KV head) units; num_threads <= 0 keeps the
 * OpenMP default.  Returns 0, -1 on a table error, -2 on bad sizes,
 * -3 on allocation failure. */
int oracle_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* seq_lens,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                        int32_t max_blocks_per_seq, int32_t dtype, double scale,
                        double* out, int32_t num_threads) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_q_heads % num_kv_heads != 0)
    return -2;
  const int64_t D = head_dim;
  const int64_t G = num_q_heads / num_kv_heads;
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  int status = 0;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    const int32_t b = (int32_t)(u / num_kv_heads);
    const int32_t g = (int32_t)(u % num_kv_heads);
    const int64_t L = seq_lens[b] > 0 ? seq_lens[b] : 0;
    const int64_t rows = L > 0 ? L : 1;
    double* K = (double*)malloc(sizeof(double) * rows * D);
    double* V = (double*)malloc(sizeof(double) * rows * D);
    double* s = (double*)malloc(sizeof(double) * rows);
    double* qh = (double*)malloc(sizeof(double) * D);
    if (!K || !V || !s || !qh) {
#pragma omp atomic write
      status = -3;
    } else if (seq_lens[b] < 0 ||
               oracle_gather(k_pool, v_pool, block_tables, b, g, L, num_kv_heads,
                             head_dim, block_size, num_blocks, max_blocks_per_seq,
                             dtype, K, V) != 0) {
#pragma omp atomic write
      status = -1;
    } else {
      for (int64_t k = 0; k < G; ++k) {
        const int64_t h = g * G + k;
        const int64_t qoff = ((int64_t)b * num_q_heads + h) * D;
        oracle_to_f64((const char*)q + qoff * (dtype == ORC_F32 ? 4 : 2), dtype, D, qh);
        oracle_attention(qh, K, V, L, D, scale, out + qoff, s);
      }
    }
    free(K);
    free(V);
    free(s);
    free(qh);
  }
  return status;
}

/* Threads the OpenMP runtime will use for a parallel region. */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------
 * Writing the cache (pure data movement: element bits are copied, never
 * converted, so the oracle works on raw bytes of `esize` per element).
 * ------------------------------------------------------------------ */

/* Append one token per sequence ("PagedAttention: The Cache Was Storing
 * Nothing", §2.2: the block table maps logical blocks to physical ones;
 * only the last block of a request is partly filled).  For every sequence
 * b with t = positions[b] >= 0: the key row k_new[b][g][:] of every KV
 * head g is written at logical position t, i.e. physical block
 * block_tables[b][t / B], slot t % B, of k_pool, and v_new[b][g][:] at the
 * same place of v_pool.  Sequences are handled in order b = 0, 1, ...
 * Layout as restated at the top of this file: K element (slot, d) of a
 * tile at slot*D + d, V element at (slot/16)*D*16 + d*16 + slot%16.
 * Returns 0, or -1 if a position or a table entry is out of range
 * (nothing more is written then). */
int oracle_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                  const int32_t* block_tables, const int32_t* positions, int32_t num_seqs,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t num_blocks, int32_t max_blocks_per_seq, int32_t esize) {
  const int64_t D = head_dim, B = block_size, H = num_kv_heads;
  const int64_t G = (B % 16 == 0) ? 16 : B; /* tokens per transposed V group */
  for (int64_t b = 0; b < num_seqs; ++b) {
    const int64_t t = positions[b];
    if (t < 0) continue;
    const int64_t j = t / B, slot = t % B;
    if (j >= max_blocks_per_seq) return -1;
    const int64_t phys = block_tables[b * max_blocks_per_seq + j];
    if (phys < 0 || phys >= num_blocks) return -1;
    for (int64_t g = 0; g < H; ++g) {
      const int64_t tile = (phys * H + g) * B * D;
      const int64_t src = (b * H + g) * D;
      for (int64_t d = 0; d < D; ++d) {
        const int64_t kdst = tile + slot * D + d;
        const int64_t vdst = tile + (slot / G) * D * G + d * G + slot % G;
        memcpy((char*)k_pool + kdst * esize, (const char*)k_new + (src + d) * esize, esize);
        memcpy((char*)v_pool + vdst * esize, (const char*)v_new + (src + d) * esize, esize);
      }
    }
  }
  return 0;
}

/* Copy-on-write block copy (same page, §2.3: a shared block is copied only
 * when a sequence diverges and writes into it).  For i = 0 .. n-1 in
 * order, physical block dst[i] of each pool becomes a copy of block
 * src[i]: all KV heads and slots, i.e. the block_bytes = Hkv*B*D*esize
 * bytes starting at block*block_bytes.  Returns 0, or -1 if an id is out
 * of range (nothing more is copied then). */
int oracle_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst,
                       int32_t n, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, int32_t esize) {
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * esize;
  for (int32_t i = 0; i < n; ++i) {
    if (src[i] < 0 || src[i] >= num_blocks || dst[i] < 0 || dst[i] >= num_blocks) return -1;
    memmove((char*)k_pool + dst[i] * block_bytes, (const char*)k_pool + src[i] * block_bytes,
            block_bytes);
    memmove((char*)v_pool + dst[i] * block_bytes, (const char*)v_pool + src[i] * block_bytes,
            block_bytes);
  }
  return 0;
}

/* ------------------------------------------------------------------
 * Block-wise eviction scoring ("PagedEviction: Structured Block-wise KV
 * Cache Pruning for Efficient Large Language Model Inference", the review's
 * "Core claim" and "What carries the argument"): token importance
 * S_t = ||V_t||_2 / ||K_t||_2 from the cached rows; a block's score is the
 * mean of S_t over its tokens; in decode, when the most recent block of a
 * sequence has just filled, the block with the lowest mean is evicted.
 * Readings (the page is silent on them): a token's key / value row is its
 * whole row of the layer, every KV head; every full block of the sequence
 * is a candidate; the lowest logical index wins a tie.
 * ------------------------------------------------------------------ */

/* scores[b][j] (fp64, [num_seqs][max_blocks_per_seq]) for every full block
 * j < L / B of every sequence, NaN elsewhere; evict[b] = the lowest-scoring
 * full block when L > 0 and L % B == 0, else -1.  Returns 0, or -1 when a
 * table entry that is read is out of range. */
int oracle_block_scores(const void* k_pool, const void* v_pool, const int32_t* block_tables,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                        int32_t max_blocks_per_seq, int32_t dtype, double* scores,
                        int32_t* evict) {
  const int64_t D = head_dim, B = block_size, H = num_kv_heads, M = max_blocks_per_seq;
  const int64_t G = (B % 16 == 0) ? 16 : B; /* tokens per transposed V group */
  for (int64_t b = 0; b < num_seqs; ++b) {
    const int64_t L = seq_lens[b] < 0 ? 0 : seq_lens[b];
    const int64_t full = L / B;
    for (int64_t j = 0; j < M; ++j) scores[b * M + j] = NAN;
    for (int64_t j = 0; j < full; ++j) {
      const int64_t phys = block_tables[b * M + j];
      if (phys < 0 || phys >= num_blocks) return -1;
      double ratio_sum = 0.0;
      for (int64_t slot = 0; slot < B; ++slot) {
        double kk = 0.0, vv = 0.0; /* squared norms of the token's rows, all heads */
        for (int64_t g = 0; g < H; ++g) {
          const int64_t base = (phys * H + g) * B * D;
          for (int64_t d = 0; d < D; ++d) {
            const double k = elem(k_pool, dtype, base + slot * D + d);
            const double v = elem(v_pool, dtype, base + (slot / G) * D * G + d * G + slot % G);
            kk += k * k;
            vv += v * v;
          }
        }
        ratio_sum += sqrt(vv) / sqrt(kk);
      }
      scores[b * M + j] = ratio_sum / (double)B;
    }
    evict[b] = -1;
    if (L > 0 && L % B == 0) {
      double best = INFINITY;
      int64_t arg = 0;
      for (int64_t j = 0; j < full; ++j) {
        if (scores[b * M + j] < best) {
          best = scores[b * M + j];
          arg = j;
        }
      }
      evict[b] = (int32_t)arg;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------
 * Paged prefill: many query rows per sequence, causal.
 *
 * "FlashAttention vs PagedAttention", "How prefill and decode change the
 * diagnosis": prefill scores many prompt positions at once against a cache
 * whose length differs from the number of queries.  "Paging the KV cache
 * with a fused mask" ("What carries the argument", and its list of
 * assumptions: masking a query to its own keys leaves exact attention
 * unchanged) maps every query to its own sequence's pages.
 * Readings (the pages print no convention):
 *  - sequence b contributes n_b = q_start[b+1] - q_start[b] query rows,
 *    rows q_start[b] .. q_start[b+1]-1 of q and out; they are its NEWEST
 *    n_b tokens, already in the cache, so row i sits at position
 *    p = L_b - n_b + i (chunked prefill: L_b - n_b earlier tokens are
 *    cached from before);
 *  - causal: row i attends tokens 0 .. p of the table, nothing later;
 *  - n_b = 1 is single-token decode, n_b = L_b a whole prompt.
 * Each row is plain softmax attention over its p + 1 gathered tokens.
 * Returns 0, -1 on a table error, -2 on bad sizes (including n_b < 0 or
 * n_b > L_b), -3 on allocation failure.
 * ------------------------------------------------------------------ */
int oracle_paged_prefill(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* q_start, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, int32_t max_blocks_per_seq, int32_t dtype,
                         double scale, double* out, int32_t num_threads) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_q_heads % num_kv_heads != 0)
    return -2;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t n = (int64_t)q_start[b + 1] - q_start[b];
    if (n < 0 || seq_lens[b] < 0 || n > seq_lens[b]) return -2;
  }
  const int64_t D = head_dim;
  const int64_t G = num_q_heads / num_kv_heads;
  const size_t qsize = dtype == ORC_F32 ? 4 : 2;
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  int status = 0;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    const int32_t b = (int32_t)(u / num_kv_heads);
    const int32_t g = (int32_t)(u % num_kv_heads);
    const int64_t Lb = seq_lens[b];
    const int64_t n = (int64_t)q_start[b + 1] - q_start[b];
    const int64_t rows = Lb > 0 ? Lb : 1;
    double* K = (double*)malloc(sizeof(double) * rows * D);
    double* V = (double*)malloc(sizeof(double) * rows * D);
    double* s = (double*)malloc(sizeof(double) * rows);
    double* qrow = (double*)malloc(sizeof(double) * D);
    if (!K || !V || !s || !qrow) {
#pragma omp atomic write
      status = -3;
    } else if (oracle_gather(k_pool, v_pool, block_tables, b, g, Lb, num_kv_heads, head_dim,
                             block_size, num_blocks, max_blocks_per_seq, dtype, K, V) != 0) {
#pragma omp atomic write
      status = -1;
    } else {
      for (int64_t i = 0; i < n; ++i) {
        const int64_t row = q_start[b] + i;  /* row of q and out */
        const int64_t p = Lb - n + i;        /* its position in the sequence */
        for (int64_t k = 0; k < G; ++k) {
          const int64_t off = (row * num_q_heads + g * G + k) * D;
          oracle_to_f64((const char*)q + off * qsize, dtype, D, qrow);
          oracle_attention(qrow, K, V, p + 1, D, scale, out + off, s);  /* tokens 0 .. p */
        }
      }
    }
    free(K);
    free(V);
    free(s);
    free(qrow);
  }
  return status;
}
