/*
 * oracle.c -- plain, slow, obviously correct CPU model of paged decode
 * attention. TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark call it; the product path never does.
 * It shares no code, header or table with the GPU library: the layout and
 * the arithmetic below are written out again from their definitions.
 *
 * Single-threaded. Floating point in double precision (the pages fix no
 * precision for the attention itself, so the oracle computes the definition
 * as exactly as a double allows); the decode also has a single-precision
 * twin (oracle_decode_f32), the naive fp32 loop, whose error the double
 * version measures. Built with -O2 -ffp-contract=off and no
 * fast-math, so every operation is the one written here.
 *
 * Sources (page title, then section):
 *   [SLS] "Scaling LLM serving" -- "The KV cache" (per-token size product,
 *         grouped-query heads), "Managing the cache: PagedAttention".
 *   [M23] "Module 23: Serving" -- 23.1 "The Memory Wall" (the KV-memory
 *         equation), 23.2 "Prefill and Decode" (decode reads the whole KV
 *         cache for one new token per sequence), 23.4 "Paged Attention"
 *         (16-token blocks, per-sequence table from positions to blocks).
 *   [DSS] "Designing an LLM serving system" -- "What it must do, and at what
 *         size", "Paged attention" (indirection, non-contiguous blocks,
 *         sharing, copy on write).
 *
 * Layout, restated from the library's documented contract:
 *   block = 16 tokens; position p of sequence s lives in physical block
 *   table[s][p / 16], slot p % 16.
 *   K pool element (blk, h, t, i): ((blk * n_kv + h) * 16 + t) * d + i
 *   V pool element (blk, h, t, i): ((blk * n_kv + h) * d + i) * 16 + t
 *   Query head j uses KV head j / (n_q / n_kv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BLOCK 16

/* A bf16 value is the upper half of an IEEE binary32; widening is exact. */
static double bf16_value(uint16_t bits) {
  uint32_t word = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &word, sizeof f);
  return (double)f;
}

static size_t k_index(int64_t blk, int h, int t, int i, int n_kv, int d) {
  return (size_t)((((int64_t)blk * n_kv + h) * ORACLE_BLOCK + t) * d + i);
}

static size_t v_index(int64_t blk, int h, int t, int i, int n_kv, int d) {
  return (size_t)((((int64_t)blk * n_kv + h) * d + i) * ORACLE_BLOCK + t);
}

/* ------------------------------------------------------------------------
 * KV-cache bytes ([M23] 23.1: 2 x layers x kv_heads x d_head x L x B x
 * bytes). Exact in 64-bit integers. */
uint64_t oracle_kv_bytes(int64_t n_layers, int64_t n_kv_heads, int64_t d_head,
                         int64_t context_len, int64_t batch,
                         int64_t bytes_per_value) {
  return (uint64_t)2 * (uint64_t)n_layers * (uint64_t)n_kv_heads *
         (uint64_t)d_head * (uint64_t)context_len * (uint64_t)batch *
         (uint64_t)bytes_per_value;
}

/* ------------------------------------------------------------------------
 * Append: the token at position ctx_s - 1 of each sequence goes to slot
 * (table[s][(ctx_s - 1) / 16], (ctx_s - 1) % 16). Bit copy.
 * Returns 0, or -1 (nothing written for that sequence) on an invalid
 * context length or block id; the other sequences are still written. */
int oracle_kv_append(uint16_t* k_pool, uint16_t* v_pool, const uint16_t* k_new,
                     const uint16_t* v_new, const int32_t* block_tables,
                     const int32_t* context_lens, int num_seqs,
                     int max_blocks_per_seq, int num_blocks, int n_kv, int d) {
  int status = 0;
  for (int s = 0; s < num_seqs; ++s) {
    int ctx = context_lens[s];
    if (ctx < 1 || ctx > ORACLE_BLOCK * max_blocks_per_seq) {
      status = -1;
      continue;
    }
    int pos = ctx - 1;
    int32_t blk = block_tables[(size_t)s * max_blocks_per_seq + pos / ORACLE_BLOCK];
    if (blk < 0 || blk >= num_blocks) {
      status = -1;
      continue;
    }
    int slot = pos % ORACLE_BLOCK;
    for (int h = 0; h < n_kv; ++h) {
      for (int i = 0; i < d; ++i) {
        size_t src = ((size_t)s * n_kv + h) * d + i;
        k_pool[k_index(blk, h, slot, i, n_kv, d)] = k_new[src];
        v_pool[v_index(blk, h, slot, i, n_kv, d)] = v_new[src];
      }
    }
  }
  return status;
}

/* ------------------------------------------------------------------------
 * Write of arbitrary tokens ([M23] 23.4: a token's position selects its
 * block through the sequence's table): token i of the source goes to row
 * seq_rows[i] at position positions[i], i.e. slot (table[row][pos / 16],
 * pos % 16). Bit copy. Returns 0, or -1 if some token was skipped (row,
 * position or block id out of range); the others are still written. */
int oracle_kv_write(uint16_t* k_pool, uint16_t* v_pool, const uint16_t* k_src,
                    const uint16_t* v_src, const int32_t* block_tables,
                    const int32_t* seq_rows, const int32_t* positions, int n_tokens,
                    int num_seqs, int max_blocks_per_seq, int num_blocks, int n_kv,
                    int d) {
  int status = 0;
  for (int tok = 0; tok < n_tokens; ++tok) {
    int row = seq_rows[tok];
    int pos = positions[tok];
    if (row < 0 || row >= num_seqs || pos < 0 || pos >= ORACLE_BLOCK * max_blocks_per_seq) {
      status = -1;
      continue;
    }
    int32_t blk = block_tables[(size_t)row * max_blocks_per_seq + pos / ORACLE_BLOCK];
    if (blk < 0 || blk >= num_blocks) {
      status = -1;
      continue;
    }
    int slot = pos % ORACLE_BLOCK;
    for (int h = 0; h < n_kv; ++h) {
      for (int i = 0; i < d; ++i) {
        size_t src = ((size_t)tok * n_kv + h) * d + i;
        k_pool[k_index(blk, h, slot, i, n_kv, d)] = k_src[src];
        v_pool[v_index(blk, h, slot, i, n_kv, d)] = v_src[src];
      }
    }
  }
  return status;
}

/* ------------------------------------------------------------------------
 * Copy on write ([DSS] "Paged attention"): block dst[p] becomes a copy of
 * block src[p], K and V, every head and slot. */
int oracle_copy_blocks(uint16_t* k_pool, uint16_t* v_pool, const int32_t* src,
                       const int32_t* dst, int n_pairs, int num_blocks,
                       int n_kv, int d) {
  int status = 0;
  size_t per_block = (size_t)n_kv * ORACLE_BLOCK * d;
  for (int p = 0; p < n_pairs; ++p) {
    if (src[p] < 0 || src[p] >= num_blocks || dst[p] < 0 || dst[p] >= num_blocks) {
      status = -1;
      continue;
    }
    for (size_t e = 0; e < per_block; ++e) {
      k_pool[(size_t)dst[p] * per_block + e] = k_pool[(size_t)src[p] * per_block + e];
      v_pool[(size_t)dst[p] * per_block + e] = v_pool[(size_t)src[p] * per_block + e];
    }
  }
  return status;
}

/* ------------------------------------------------------------------------
 * One output row: the attention of query row q_row (d values, bf16 bits)
 * over the ctx cached tokens of one sequence, reached through its table,
 * for KV head h. Softmax written as its definition with the maximum
 * subtracted first (the shift leaves the ratios unchanged and keeps exp()
 * finite):
 *   z_t = scale * sum_i q_i k_{t,i}
 *   w_t = exp(z_t - max_u z_u),   out_i = (sum_t w_t v_{t,i}) / (sum_t w_t)
 * Returns 0, or -1 with NaN written on an invalid block id or ctx < 1. */
int oracle_decode_row(double* out_row, const uint16_t* q_row,
                      const uint16_t* k_pool, const uint16_t* v_pool,
                      const int32_t* table_row, int ctx, int num_blocks,
                      int n_kv, int h, int d, double scale) {
  if (ctx < 1) {
    for (int i = 0; i < d; ++i) out_row[i] = NAN;
    return -1;
  }
  for (int b = 0; b < (ctx + ORACLE_BLOCK - 1) / ORACLE_BLOCK; ++b) {
    if (table_row[b] < 0 || table_row[b] >= num_blocks) {
      for (int i = 0; i < d; ++i) out_row[i] = NAN;
      return -1;
    }
  }
  double* z = (double*)malloc(sizeof(double) * (size_t)ctx);
  if (!z) return -2;

  for (int t = 0; t < ctx; ++t) {
    int32_t blk = table_row[t / ORACLE_BLOCK];
    int slot = t % ORACLE_BLOCK;
    double dot = 0.0;
    for (int i = 0; i < d; ++i)
      dot += bf16_value(q_row[i]) * bf16_value(k_pool[k_index(blk, h, slot, i, n_kv, d)]);
    z[t] = scale * dot;
  }

  double zmax = z[0];
  for (int t = 1; t < ctx; ++t)
    if (z[t] > zmax) zmax = z[t];

  double denom = 0.0;
  for (int t = 0; t < ctx; ++t) {
    z[t] = exp(z[t] - zmax); /* z now holds the unnormalised weights */
    denom += z[t];
  }

  for (int i = 0; i < d; ++i) {
    double num = 0.0;
    for (int t = 0; t < ctx; ++t) {
      int32_t blk = table_row[t / ORACLE_BLOCK];
      num += z[t] * bf16_value(v_pool[v_index(blk, h, t % ORACLE_BLOCK, i, n_kv, d)]);
    }
    out_row[i] = num / denom;
  }
  free(z);
  return 0;
}

/* ------------------------------------------------------------------------
 * The whole decode step of one layer: every sequence s, every query head j
 * (KV head j / G). out is double [num_seqs][n_q][d]. Returns 0, or -1 if any
 * sequence was invalid (its rows are NaN). */
int oracle_decode(double* out, const uint16_t* q, const uint16_t* k_pool,
                  const uint16_t* v_pool, const int32_t* block_tables,
                  const int32_t* context_lens, int num_seqs,
                  int max_blocks_per_seq, int num_blocks, int n_q, int n_kv,
                  int d, double scale) {
  if (n_kv <= 0 || n_q % n_kv != 0) return -3;
  int group = n_q / n_kv;
  int status = 0;
  for (int s = 0; s < num_seqs; ++s) {
    int ctx = context_lens[s];
    int bad_ctx = ctx > ORACLE_BLOCK * max_blocks_per_seq;
    for (int j = 0; j < n_q; ++j) {
      double* row = out + ((size_t)s * n_q + j) * d;
      if (bad_ctx) {
        for (int i = 0; i < d; ++i) row[i] = NAN;
        status = -1;
        continue;
      }
      int rc = oracle_decode_row(row, q + ((size_t)s * n_q + j) * d, k_pool,
                                 v_pool, block_tables + (size_t)s * max_blocks_per_seq,
                                 ctx, num_blocks, n_kv, j / group, d, scale);
      if (rc == -2) return -2;
      if (rc != 0) status = -1;
    }
  }
  return status;
}

/* ------------------------------------------------------------------------
 * The same decode in single precision: the naive two-pass softmax of one
 * query row with every operation in float, in the order written ([M23]
 * 23.2 and [SLS] "The KV cache": one query row attends to every cached
 * token of its sequence through the table). A product of two bf16 values
 * is exact in float; the dot products, the exponentials (expf), the sums
 * and the division round to float. oracle_decode_row above computes the
 * same definition in double and is this function's twin: the difference
 * between the two is this function's own rounding error. Returns as
 * oracle_decode_row. */
static float bf16_float(uint16_t bits) {
  uint32_t word = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &word, sizeof f);
  return f;
}

int oracle_decode_row_f32(float* out_row, const uint16_t* q_row,
                          const uint16_t* k_pool, const uint16_t* v_pool,
                          const int32_t* table_row, int ctx, int num_blocks,
                          int n_kv, int h, int d, float scale) {
  if (ctx < 1) {
    for (int i = 0; i < d; ++i) out_row[i] = NAN;
    return -1;
  }
  for (int b = 0; b < (ctx + ORACLE_BLOCK - 1) / ORACLE_BLOCK; ++b) {
    if (table_row[b] < 0 || table_row[b] >= num_blocks) {
      for (int i = 0; i < d; ++i) out_row[i] = NAN;
      return -1;
    }
  }
  float* w = (float*)malloc(sizeof(float) * (size_t)ctx);
  if (!w) return -2;

  /* scores: w[p] = scale * (q . k_p) */
  for (int p = 0; p < ctx; ++p) {
    int32_t block = table_row[p / ORACLE_BLOCK];
    int in_block = p % ORACLE_BLOCK;
    float qk = 0.0f;
    for (int i = 0; i < d; ++i)
      qk += bf16_float(q_row[i]) * bf16_float(k_pool[k_index(block, h, in_block, i, n_kv, d)]);
    w[p] = scale * qk;
  }

  float top = w[0];
  for (int p = 1; p < ctx; ++p)
    if (w[p] > top) top = w[p];

  float total = 0.0f;
  for (int p = 0; p < ctx; ++p) {
    w[p] = expf(w[p] - top); /* w now holds the unnormalised weights */
    total += w[p];
  }

  for (int i = 0; i < d; ++i) {
    float acc = 0.0f;
    for (int p = 0; p < ctx; ++p) {
      int32_t block = table_row[p / ORACLE_BLOCK];
      int in_block = p % ORACLE_BLOCK;
      acc += w[p] * bf16_float(v_pool[v_index(block, h, in_block, i, n_kv, d)]);
    }
    out_row[i] = acc / total;
  }
  free(w);
  return 0;
}

/* oracle_decode with oracle_decode_row_f32 for every row; out is float
 * [num_seqs][n_q][d]. Returns as oracle_decode. */
int oracle_decode_f32(float* out, const uint16_t* q, const uint16_t* k_pool,
                      const uint16_t* v_pool, const int32_t* block_tables,
                      const int32_t* context_lens, int num_seqs,
                      int max_blocks_per_seq, int num_blocks, int n_q, int n_kv,
                      int d, float scale) {
  if (n_kv <= 0 || n_q % n_kv != 0) return -3;
  int group = n_q / n_kv;
  int status = 0;
  for (int s = 0; s < num_seqs; ++s) {
    int ctx = context_lens[s];
    int too_long = ctx > ORACLE_BLOCK * max_blocks_per_seq;
    for (int j = 0; j < n_q; ++j) {
      float* row = out + ((size_t)s * n_q + j) * d;
      if (too_long) {
        for (int i = 0; i < d; ++i) row[i] = NAN;
        status = -1;
        continue;
      }
      int kv_head = j / group;
      const uint16_t* q_row = q + ((size_t)s * n_q + j) * d;
      const int32_t* table_row = block_tables + (size_t)s * max_blocks_per_seq;
      int rc = oracle_decode_row_f32(row, q_row, k_pool, v_pool, table_row, ctx, num_blocks,
                                     n_kv, kv_head, d, scale);
      if (rc == -2) return -2;
      if (rc != 0) status = -1;
    }
  }
  return status;
}

/* ------------------------------------------------------------------------
 * Verification pass of speculative decoding ([M23] 23.5: the large model
 * checks all drafted tokens in one pass; [SLS] "Speculative decoding";
 * [DSS] "Speculative decoding"). Each sequence brings q_len query tokens:
 * the last q_len of its ctx cached tokens (their keys and values are
 * already in the pool). Query token i sits at position ctx - q_len + i and,
 * as in any decode step, attends to every cached token up to and including
 * its own position, i.e. to the first ctx - q_len + i + 1 tokens: each row
 * is oracle_decode_row over the sequence cut at that length.
 * q and out: [num_seqs][q_len][n_q][d]. A sequence with ctx < q_len (or ctx
 * past its table) is invalid: its rows are NaN. Returns 0, -1 if any
 * sequence was invalid, -2 on allocation failure, -3 on bad heads. */
int oracle_verify(double* out, const uint16_t* q, const uint16_t* k_pool,
                  const uint16_t* v_pool, const int32_t* block_tables,
                  const int32_t* context_lens, int num_seqs, int q_len,
                  int max_blocks_per_seq, int num_blocks, int n_q, int n_kv,
                  int d, double scale) {
  if (n_kv <= 0 || n_q % n_kv != 0 || q_len < 1) return -3;
  int group = n_q / n_kv;
  int status = 0;
  for (int s = 0; s < num_seqs; ++s) {
    int ctx = context_lens[s];
    int bad_ctx = ctx < q_len || ctx > ORACLE_BLOCK * max_blocks_per_seq;
    for (int i = 0; i < q_len; ++i) {
      int seen = ctx - q_len + i + 1; /* tokens up to query i's own position */
      for (int j = 0; j < n_q; ++j) {
        size_t row_index = ((size_t)s * q_len + i) * n_q + j;
        double* row = out + row_index * d;
        if (bad_ctx) {
          for (int e = 0; e < d; ++e) row[e] = NAN;
          status = -1;
          continue;
        }
        int rc = oracle_decode_row(row, q + row_index * d, k_pool, v_pool,
                                   block_tables + (size_t)s * max_blocks_per_seq,
                                   seen, num_blocks, n_kv, j / group, d, scale);
        if (rc == -2) return -2;
        if (rc != 0) status = -1;
      }
    }
  }
  return status;
}
