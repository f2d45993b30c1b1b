/*
 * pkv.h -- C ABI of libpkv: decode-phase attention over a paged KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources. Three web pages describe the method:
 *   [SLS]  "Scaling LLM serving" (jayaprakash.net), sections "The KV cache",
 *          "Managing the cache: PagedAttention", "Reuse shared prefixes".
 *   [M23]  "Module 23: Serving" (Transformers & Math), section 23.1 "The Memory
 *          Wall" (KV-size equation), 23.2 "Prefill and Decode", 23.4 "Paged
 *          Attention", and the closing Exercises.
 *   [DSS]  "Designing an LLM serving system" (clio.skatech.org), sections
 *          "What it must do, and at what size", "The KV cache", "Continuous
 *          batching" (scheduler flowchart) and "Paged attention".
 *
 * Everything here is plain C: pointers, sizes, status codes. No C++ or torch
 * type crosses the boundary. Device pointers are HIP device addresses on the
 * current device; `stream` is a hipStream_t passed as void* (NULL = the
 * legacy default stream). All device entry points only enqueue work: they
 * return after the launch, with no implicit synchronisation.
 *
 * ---------------------------------------------------------------------------
 * Memory layout (one K pool and one V pool per layer; the block tables are
 * one per sequence and shared by all layers)
 *
 *   PKV_BLOCK_TOKENS = 16 tokens per block (the block size [M23] 23.4 uses as its example).
 *
 *   k_pool  bf16  [num_blocks][n_kv_heads][16][head_dim]        (token-major)
 *           element (blk, h, t, i) at  ((blk*n_kv_heads + h)*16 + t)*head_dim + i
 *   v_pool  bf16  [num_blocks][n_kv_heads][head_dim][16]        (dim-major)
 *           element (blk, h, t, i) at  ((blk*n_kv_heads + h)*head_dim + i)*16 + t
 *
 *   So one (block, head) tile of K and of V is 16*head_dim*2 bytes of
 *   contiguous memory each (4 KiB at head_dim 128). V is stored dim-major so
 *   that the 16 tokens of one head dimension are adjacent: that is the
 *   operand order the matrix cores need for the probability-times-V product.
 *   All offsets are computed in 64-bit arithmetic.
 *
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entry (s, b) is the
 *                 physical block holding positions 16b .. 16b+15 of sequence
 *                 s ([M23] 23.4: a per-sequence table maps positions to
 *                 blocks; [DSS] "Paged attention": the blocks need not be
 *                 contiguous). Entries at b >= ceil(ctx_s/16) are ignored.
 *   context_lens  int32 [num_seqs]; ctx_s counts every cached token of
 *                 sequence s INCLUDING the one appended in this step, which
 *                 sits at position ctx_s - 1. Valid range 1 .. max_context_len.
 *
 *   q      bf16  [num_seqs][n_q_heads][head_dim]
 *   k_new  bf16  [num_seqs][n_kv_heads][head_dim]   (same for v_new)
 *   out    fp32  [num_seqs][n_q_heads][head_dim]
 *
 *   Grouped-query attention ([SLS] "The KV cache": fewer KV heads than query
 *   heads, every KV head serving several query heads): G = n_q_heads / n_kv_heads, and query
 *   head j reads KV head j / G (consecutive groups). G = 1 is multi-head
 *   attention, n_kv_heads = 1 is multi-query attention.
 *
 * What the decode computes, for each sequence s and query head j with
 * h = j / G (softmax attention of the one new query token over the whole
 * cached context, [M23] 23.2: every decode step streams a sequence's entire
 * cache to produce its single new token):
 *
 *   z_t       = scale * sum_i q[s,j,i] * K(bt[s][t/16], h, t%16, i),  0 <= t < ctx_s
 *   out[s,j,:] = sum_t softmax(z)_t * V(bt[s][t/16], h, t%16, :)
 *
 * Arithmetic: bf16 inputs widened exactly to fp32; scores, the online
 * softmax and the accumulation in fp32; output fp32.
 *
 * ---------------------------------------------------------------------------
 * Errors
 *
 *   Every entry point returns PKV_OK (0) or a negative PKV_E* code. Host-side
 *   checks happen before any launch; on an error nothing is enqueued.
 *   Device-side checks (values that live in device memory: block ids,
 *   context lengths) cannot return a status: the kernel ORs a PKV_DEVERR_*
 *   bit into *err_flag (an int32 in device memory the caller zeroes; NULL
 *   disables reporting), never reads or writes out of bounds, and writes NaN
 *   to the outputs that depended on the bad value.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_BLOCK_TOKENS 16
#define PKV_DEFAULT_PARTITION_TOKENS 0 /* pass 0 to let the library choose */

enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* null pointer, negative size, inconsistent shape */
  PKV_EUNSUPPORTED = -2,  /* head_dim not in {64, 128} */
  PKV_ENOMEM = -3,        /* allocator: no free block */
  PKV_EWORKSPACE = -4,    /* workspace smaller than pkv_decode_workspace_bytes */
  PKV_EHIP = -5           /* the HIP runtime reported a launch error */
};

/* Device error bits, ORed into *err_flag by the kernels. */
#define PKV_DEVERR_BLOCK_ID 1   /* a needed block-table entry outside [0, num_blocks) */
#define PKV_DEVERR_CONTEXT 2    /* a context length outside [1, max_context_len] */
#define PKV_DEVERR_COPY_PAIR 4  /* a copy_blocks id outside [0, num_blocks) */
#define PKV_DEVERR_TOKEN 8      /* pkv_spec_accept: a drafted token outside [0, vocab) */
#define PKV_DEVERR_PREFIX 16    /* pkv_decode_step_prefix: a member's table does not start with the prefix */

/* Static string for a status code; never NULL. */
const char* pkv_strerror(int status);

/* ------------------------------------------------------------------------
 * KV-cache size closed form ([M23] 23.1, the KV-memory equation; [SLS] "The
 * KV cache" gives the same product per token).
 *   bytes per token = 2 * n_layers * n_kv_heads * head_dim * bytes_per_value
 *   bytes           = bytes per token * context_len * batch
 * Pure host arithmetic, exact in 64 bits. Returns 0 if any argument is < 0. */
uint64_t pkv_kv_bytes_per_token(int32_t n_layers, int32_t n_kv_heads,
                                int32_t head_dim, int32_t bytes_per_value);
uint64_t pkv_kv_cache_bytes(int32_t n_layers, int32_t n_kv_heads,
                            int32_t head_dim, int64_t context_len,
                            int64_t batch, int32_t bytes_per_value);
/* Bytes of ONE pool (K or V) of one layer in the layout above:
 * num_blocks * n_kv_heads * 16 * head_dim * 2. */
uint64_t pkv_pool_bytes(int32_t num_blocks, int32_t n_kv_heads, int32_t head_dim);

/* ------------------------------------------------------------------------
 * kv_append: scatter this step's new key and value of every sequence into
 * its pool slot ([M23] 23.4 and [DSS] "Paged attention": positions reach
 * physical blocks through the per-sequence table; a sequence gains blocks
 * only as its context lengthens, so the caller has already made bt[s][(ctx_s-1)/16]
 * valid and private, e.g. with pkv_seq_grow).
 *
 * For each s: p = ctx_s - 1, blk = bt[s][p/16], slot = p % 16, and for every
 * KV head h and dimension i the 16-bit patterns k_new[s,h,i] / v_new[s,h,i]
 * are stored at K/V element (blk, h, slot, i). Pure bit copy: bit-exact.
 *
 * k_pool, v_pool : device, bf16 pools of one layer, num_blocks blocks.
 * k_new, v_new   : device, bf16 [num_seqs][n_kv_heads][head_dim].
 * block_tables, context_lens : device int32, as above.
 * Device errors: bt entry outside [0, num_blocks) or ctx_s outside
 * [1, 16*max_blocks_per_seq] -> the sequence is skipped and the matching
 * PKV_DEVERR bit set. num_seqs == 0 is a no-op. */
int pkv_kv_append(void* k_pool, void* v_pool, const void* k_new,
                  const void* v_new, const int32_t* block_tables,
                  const int32_t* context_lens, int32_t num_seqs,
                  int32_t max_blocks_per_seq, int32_t num_blocks,
                  int32_t n_kv_heads, int32_t head_dim, int32_t* err_flag,
                  void* stream);

/* ------------------------------------------------------------------------
 * kv_write: scatter arbitrary tokens' keys and values into the pools
 * ([M23] 23.4: a position selects its block through the sequence's table).
 * Token t of k_src / v_src goes to row seq_rows[t] at position positions[t]:
 * K/V element (bt[row][pos/16], h, pos%16, i). For the keys and values a
 * prefill computed for a newly admitted request, or recomputed for a
 * preempted one ([DSS] "Continuous batching": admit it, run its prefill;
 * "Scheduling": preemption by recompute). Pure bit copy.
 *
 * k_src, v_src : device bf16 [n_tokens][n_kv_heads][head_dim].
 * seq_rows, positions : device int32 [n_tokens].
 * block_tables : device int32 [num_seqs][max_blocks_per_seq].
 * The blocks written must not be shared with another sequence. Two tokens
 * for the same (row, position) leave one of them, unspecified which. The
 * pools and k_src / v_src must be 16-byte aligned (PKV_EINVAL otherwise;
 * every torch allocation is). Fastest when runs of 16 consecutive tokens
 * are consecutive positions of one sequence, as a prompt is. Device
 * errors: a row outside [0, num_seqs) or a position outside
 * [0, 16*max_blocks_per_seq) -> PKV_DEVERR_CONTEXT; a table entry outside
 * [0, num_blocks) -> PKV_DEVERR_BLOCK_ID; that token is skipped. */
int pkv_kv_write(void* k_pool, void* v_pool, const void* k_src,
                 const void* v_src, const int32_t* block_tables,
                 const int32_t* seq_rows, const int32_t* positions,
                 int32_t n_tokens, int32_t num_seqs, int32_t max_blocks_per_seq,
                 int32_t num_blocks, int32_t n_kv_heads, int32_t head_dim,
                 int32_t* err_flag, void* stream);

/* ------------------------------------------------------------------------
 * paged_attn_decode: the attention above, for every sequence and query head.
 *
 * Work split. A unit is one (sequence, KV head, group of up to 16 of its
 * query heads); one wavefront serves all query heads of the group from the
 * same K/V tiles, so each KV byte is read once for G <= 16 (larger groups
 * take ceil(G/16) passes). A wavefront processes a run of consecutive
 * 16-token tiles of a unit:
 *   partition_tokens == 0 (default): balanced split. All tiles of the call,
 *     ordered by (KV head, group, sequence, tile), are cut into
 *     pkv_decode_split_waves(...) equal ranges, one per wavefront, so every
 *     wavefront streams the same bytes whatever the context lengths. The
 *     split depends on the context lengths only.
 *   partition_tokens = P (a multiple of 16 in [16, 1024]): fixed
 *     partitions, one wavefront per P tokens of each unit.
 * A unit processed by one wavefront is written to out directly; otherwise
 * each wavefront leaves a partial (reference max, sum, accumulator) in the
 * workspace and a second kernel merges them (log-sum-exp rescaling).
 * Loads: a sequence whose first block is also the first block of a
 * neighbouring sequence (a shared prefix) is read through the caches; any
 * other is streamed with non-temporal loads. This only affects speed.
 *
 * out        : device fp32 [num_seqs][n_q_heads][head_dim], written fully.
 * q          : device bf16 [num_seqs][n_q_heads][head_dim].
 * k_pool, v_pool, block_tables, context_lens : as above.
 * n_q_heads % n_kv_heads must be 0. head_dim in {64, 128}.
 * scale      : multiplies the q.k dot product (1/sqrt(head_dim) usually).
 * max_context_len : host-side upper bound of every ctx_s, at most
 *              16*max_blocks_per_seq; sizes the grid and the workspace.
 * workspace  : device scratch of at least pkv_decode_workspace_bytes(...)
 *              bytes (may be NULL when that is 0); caller-owned.
 * Device errors: ctx_s outside [1, max_context_len], or a needed table
 * entry outside [0, num_blocks): out[s,:,:] becomes NaN for that sequence
 * and the PKV_DEVERR bit is set. num_seqs == 0 is a no-op. Host-side
 * limits: num_seqs * ceil(max_context_len / 16) < 2^30.
 *
 * Workspace bytes: 4 * (head_dim + 2) * min(G, 16) * slots, with slots =
 * units * ceil(max_context_len / P) for fixed partitions (0 if that is one
 * partition) and units + min(8192, ceil(units * ceil(max_context_len/16) / 16))
 * for the balanced split; units = num_seqs * n_kv_heads * ceil(G / 16). The
 * balanced split's workspace starts with 8 * units bytes (rounded up to a
 * multiple of 256) of per-unit bookkeeping the partition kernel writes for
 * the merge kernel. No initialisation is needed. One workspace serves one
 * call at a time. */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim,
                                  int32_t max_context_len,
                                  int32_t partition_tokens);
int pkv_paged_attn_decode(float* out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_blocks_per_seq, int32_t num_blocks,
                          int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, float scale,
                          int32_t max_context_len, int32_t partition_tokens,
                          void* workspace, size_t workspace_bytes,
                          int32_t* err_flag, void* stream);
/* The two kernels of pkv_paged_attn_decode as separate calls, with the
 * same arguments and checks; calling partition then merge on one stream is
 * exactly pkv_paged_attn_decode. pkv_paged_attn_partition writes the units
 * one wavefront covers to out, and the partials of the others into the
 * workspace; pkv_paged_attn_merge combines those into out and writes the
 * NaN rows of sequences with an invalid context length. Separate calls let
 * a caller time the two kernels. */
int pkv_paged_attn_partition(float* out, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_tables,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_blocks_per_seq, int32_t num_blocks,
                             int32_t n_q_heads, int32_t n_kv_heads,
                             int32_t head_dim, float scale,
                             int32_t max_context_len, int32_t partition_tokens,
                             void* workspace, size_t workspace_bytes,
                             int32_t* err_flag, void* stream);
int pkv_paged_attn_merge(float* out, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t num_seqs,
                         int32_t max_blocks_per_seq, int32_t num_blocks,
                         int32_t n_q_heads, int32_t n_kv_heads,
                         int32_t head_dim, float scale,
                         int32_t max_context_len, int32_t partition_tokens,
                         void* workspace, size_t workspace_bytes,
                         int32_t* err_flag, void* stream);
/* One layer's decode step: pkv_kv_append of (k_new, v_new), then
 * pkv_paged_attn_decode, with the same arguments as those two calls (k_pool
 * and v_pool are written). Results, pools included, are bit for bit those of
 * the two calls. With the balanced split the append runs inside the
 * attention's partition kernel (two launches instead of three): the
 * wavefront that holds a sequence's last tile takes the new token's key and
 * value from k_new / v_new and stores them into the pools (for the first
 * query group of each KV head) during the attention. The block holding
 * position ctx - 1
 * must not be shared with another sequence (copy on write first, as
 * pkv_seq_grow arranges). Invalid context lengths (outside
 * [1, max_context_len]) and bad block ids are reported as for the two calls;
 * such a sequence is not appended. k_new / v_new: device bf16
 * [num_seqs][n_kv_heads][head_dim]. */
int pkv_decode_step(float* out, const void* q, const void* k_new,
                    const void* v_new, void* k_pool, void* v_pool,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t num_seqs, int32_t max_blocks_per_seq,
                    int32_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
                    int32_t head_dim, float scale, int32_t max_context_len,
                    int32_t partition_tokens, void* workspace,
                    size_t workspace_bytes, int32_t* err_flag, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * pkv_decode_step with the balanced split (partition_tokens = 0) and no
 * workspace argument. Its workspace is a device array of
 * PKV_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it
 * runs on, from the first call made with that GPU current until the process
 * ends. The call allocates nothing: no hipMalloc, no allocating library
 * routine. Results, pools included, are bit for bit those of
 * pkv_decode_step with partition_tokens = 0 on the same arguments.
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents (the kernels need no initialisation: every value the
 * merge reads is written by the same call's partition kernel). Calls on one
 * stream are ordered; calls on one GPU that can overlap (different
 * streams, or other processes' threads sharing the library's state) race
 * on the array. Arguments, layouts and device errors as for pkv_decode_step.
 * Host-checked errors: those of pkv_decode_step, and PKV_EWORKSPACE when the
 * call needs more than PKV_NOALLOC_SCRATCH_BYTES
 * (pkv_decode_workspace_bytes(num_seqs, n_q_heads, n_kv_heads, head_dim,
 * max_context_len, 0) is the need), before anything is launched; PKV_EHIP if
 * the array's device address cannot be looked up. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pkv_decode_step_noalloc(float* out, const void* q, const void* k_new,
                            const void* v_new, void* k_pool, void* v_pool,
                            const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t num_blocks,
                            int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, float scale,
                            int32_t max_context_len, int32_t* err_flag,
                            void* stream);

/* The first half of pkv_decode_step: the append and the partition kernel
 * (with the balanced split one launch, the append inside it). Same arguments
 * as pkv_decode_step; pkv_paged_attn_merge with the same arguments then
 * finishes the step. Together the two calls are pkv_decode_step, bit for
 * bit; apart, each kernel can be timed or scheduled on its own. */
int pkv_decode_step_partition(float* out, const void* q, const void* k_new,
                              const void* v_new, void* k_pool, void* v_pool,
                              const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_blocks_per_seq, int32_t num_blocks,
                              int32_t n_q_heads, int32_t n_kv_heads,
                              int32_t head_dim, float scale,
                              int32_t max_context_len, int32_t partition_tokens,
                              void* workspace, size_t workspace_bytes,
                              int32_t* err_flag, void* stream);

/* pkv_decode_step_partition with the balanced split (partition_tokens must
 * be 0) and the attention's two products on the vector ALUs instead of the
 * matrix cores: packed bf16 dot products with fp32 accumulation for both
 * the scores and the weighted sum of the values (the weights split into
 * bf16 hi + lo, as the matrix path splits them); the same split, loads,
 * append and partials, so pkv_paged_attn_merge with the same arguments
 * finishes the step. The unit's query rows are staged in at most 8 KiB of
 * LDS per workgroup. Kept to measure what the matrix cores buy on
 * this memory-bound path (the pages call the decode a streaming read of the
 * cache: [M23] 23.2; [SLS] "Why decoding is limited by memory"). Results
 * within 1e-3 of the oracle, not bit-identical to the matrix path (another
 * summation order). n_q_heads / n_kv_heads at most 8, else
 * PKV_EUNSUPPORTED; partition_tokens other than 0: PKV_EINVAL; other errors
 * as for pkv_decode_step_partition. */
int pkv_decode_step_partition_valu(float* out, const void* q, const void* k_new,
                                   const void* v_new, void* k_pool, void* v_pool,
                                   const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t max_blocks_per_seq, int32_t num_blocks,
                                   int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, float scale,
                                   int32_t max_context_len, int32_t partition_tokens,
                                   void* workspace, size_t workspace_bytes,
                                   int32_t* err_flag, void* stream);

/* A decode step whose batch shares a prompt prefix held once in the pools
 * ([SLS] "Reuse shared prefixes": requests that begin with the same prompt
 * share its cached blocks; [DSS] "Paged attention": shared blocks are
 * reference-counted and written only after a copy). The result is that of
 * pkv_decode_step on the same arguments, to fp32 rounding (the softmax is
 * merged in another order); the pools are bitwise the same.
 *
 * Sequences prefix_first_seq .. prefix_first_seq + prefix_num_seqs - 1 are
 * the members. A member whose context extends past the prefix
 * (context_lens[s] > 16 * prefix_blocks) must hold prefix_table's ids as
 * its first prefix_blocks table entries. The partition kernel then reads
 * the prefix's tiles once for all members, as prefix units of its balanced
 * split that serve 32 member rows per K/V tile (the decode serves
 * n_q/n_kv), and each member's own unit covers only its later tiles; the
 * merge kernel combines both. The merge checks every such member's table
 * at each call: one whose table differs there gets NaN rows and sets
 * PKV_DEVERR_PREFIX (never a wrong finite result). A member whose context
 * ends inside the prefix, and every sequence outside the range, runs as in
 * pkv_decode_step.
 *   prefix_table    : device int32 [prefix_blocks], the prefix's block ids
 *   prefix_blocks   : whole 16-token blocks of the prefix, in
 *                     [0, max_blocks_per_seq]; 0 (or prefix_num_seqs = 0)
 *                     is pkv_decode_step with the balanced split
 *   workspace       : at least pkv_decode_prefix_workspace_bytes(...) bytes
 *                     (the decode's workspace, then the prefix units'
 *                     bookkeeping and partials); no initialisation needed
 * Other arguments as for pkv_decode_step with partition_tokens = 0. Two
 * launches on `stream`: the partition kernel (prefix units, the members'
 * own tiles and the append), then the merge kernel. Host-checked errors:
 * PKV_EINVAL for a member range outside [0, num_seqs), a negative count or
 * prefix_blocks > max_blocks_per_seq, a null prefix_table with a non-empty
 * prefix, and everything pkv_decode_step checks; PKV_EWORKSPACE. Device errors as for
 * pkv_decode_step; an id in prefix_table outside the pool sets
 * PKV_DEVERR_BLOCK_ID and makes the rows of every member that reads the
 * prefix NaN (never read out of bounds). */
size_t pkv_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t n_q_heads,
                                         int32_t n_kv_heads, int32_t head_dim,
                                         int32_t max_context_len,
                                         int32_t prefix_blocks,
                                         int32_t prefix_num_seqs);
int pkv_decode_step_prefix(float* out, const void* q, const void* k_new,
                           const void* v_new, void* k_pool, void* v_pool,
                           const int32_t* block_tables,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t max_blocks_per_seq, int32_t num_blocks,
                           int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, float scale,
                           int32_t max_context_len,
                           const int32_t* prefix_table, int32_t prefix_blocks,
                           int32_t prefix_first_seq, int32_t prefix_num_seqs,
                           void* workspace, size_t workspace_bytes,
                           int32_t* err_flag, void* stream);

/* ------------------------------------------------------------------------
 * Verification pass of speculative decoding ([M23] 23.5: the target model
 * checks all drafted tokens in one pass, at about the cost of one decode
 * step since the pass is bound by memory reads; [SLS] "Speculative
 * decoding"; [DSS] "Speculative decoding").
 *
 * Each sequence brings q_len query tokens (the last accepted token and the
 * drafts): the last q_len of its context_lens[s] cached tokens, whose keys
 * and values the caller has already written into the pools (pkv_kv_write).
 * Query token i sits at position ctx - q_len + i and attends to positions
 * 0 .. ctx - q_len + i (causal among the new tokens). Every K/V byte is read
 * once for all q_len * (n_q/n_kv) rows of a KV head (up to 32 rows per read;
 * more rows read the cache once per 32).
 *   q:   device bf16 [num_seqs][q_len][n_q_heads][head_dim]
 *   out: device fp32 [num_seqs][q_len][n_q_heads][head_dim]
 * q_len in [1, 64]; q_len == 1 is pkv_paged_attn_decode (same kernels, same
 * bits). Other arguments as for pkv_paged_attn_decode with the balanced
 * split; workspace of at least pkv_verify_workspace_bytes, no initialisation
 * needed. Device errors: a context length outside [q_len, max_context_len]
 * sets PKV_DEVERR_CONTEXT, a bad block id PKV_DEVERR_BLOCK_ID; that
 * sequence's rows are NaN. After the pass the caller keeps the accepted
 * tokens by setting the context length; slots past it are overwritten by
 * later appends. */
size_t pkv_verify_workspace_bytes(int32_t num_seqs, int32_t q_len,
                                  int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int32_t max_context_len);
int pkv_paged_attn_verify(float* out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t q_len, int32_t max_blocks_per_seq,
                          int32_t num_blocks, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t head_dim, float scale,
                          int32_t max_context_len, void* workspace,
                          size_t workspace_bytes, int32_t* err_flag,
                          void* stream);

/* The verification pass for a batch whose member sequences share a prompt
 * prefix held once in the pools ([SLS] "Reuse shared prefixes"; [M23] 23.5;
 * [DSS] "Paged attention": shared blocks are reference-counted). The result
 * is that of pkv_paged_attn_verify on the same arguments, to fp32 rounding
 * (the softmax is merged in another order). Sequences prefix_first_seq ..
 * prefix_first_seq + prefix_num_seqs - 1 are the members. A member whose
 * query tokens all lie after the prefix (context_lens[s] - q_len >=
 * 16 * prefix_blocks) must hold prefix_table's ids as its first
 * prefix_blocks table entries: the prefix's tiles are then read once for
 * all such members, as prefix units of the balanced split that serve 32
 * member rows (query token, head) per K/V tile, and each member's own unit
 * covers only its later tiles; the merge kernel combines both and checks
 * every such member's table at each call (one whose table differs there
 * gets NaN rows and PKV_DEVERR_PREFIX). Any other member, and every
 * sequence outside the range, runs as in pkv_paged_attn_verify.
 *   prefix_table : device int32 [prefix_blocks], the prefix's block ids
 *   workspace    : at least pkv_verify_prefix_workspace_bytes(...) bytes (the
 *                  verification pass's workspace, then the prefix units'
 *                  bookkeeping and partials); no initialisation needed
 * q_len in [1, 64]. Other arguments, host-checked errors and device errors
 * as for pkv_paged_attn_verify and pkv_decode_step_prefix; prefix_blocks = 0
 * or prefix_num_seqs = 0 runs pkv_paged_attn_verify's computation. Two
 * launches on `stream`. */
size_t pkv_verify_prefix_workspace_bytes(int32_t num_seqs, int32_t q_len,
                                         int32_t n_q_heads, int32_t n_kv_heads,
                                         int32_t head_dim,
                                         int32_t max_context_len,
                                         int32_t prefix_blocks,
                                         int32_t prefix_num_seqs);
int pkv_paged_attn_verify_prefix(float* out, const void* q, const void* k_pool,
                                 const void* v_pool,
                                 const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t q_len, int32_t max_blocks_per_seq,
                                 int32_t num_blocks, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim,
                                 float scale, int32_t max_context_len,
                                 const int32_t* prefix_table,
                                 int32_t prefix_blocks,
                                 int32_t prefix_first_seq,
                                 int32_t prefix_num_seqs, void* workspace,
                                 size_t workspace_bytes, int32_t* err_flag,
                                 void* stream);

/* ------------------------------------------------------------------------
 * Chunked prefill against the paged cache ([SLS] "Split long prefills into
 * chunks": a long prompt is taken a chunk per step beside the ongoing
 * decodes; [DSS] "Scheduling: when prefill meets decode"; [M23] 23.2:
 * prefill reuses every weight across all the prompt's tokens, which makes it
 * compute-bound).
 *
 * Each sequence's chunk is its last chunk_len cached tokens (the chunk's
 * keys and values already written, pkv_kv_write); chunk token i, at position
 * ctx - chunk_len + i, attends to positions 0 .. ctx - chunk_len + i: the
 * earlier chunks and the prompt's cached prefix through the block table,
 * and the chunk itself causally. The same computation as
 * pkv_paged_attn_verify with q_len = chunk_len, organised for long chunks:
 * a workgroup of 8 wavefronts per (sequence, KV head, 256 query rows)
 * stages 64-token K/V tiles in LDS for all its rows; scores and values on
 * 32x32x16 MFMAs; no workspace. The workgroups take the (sequence, KV head)
 * pairs longest context first (the ranking reads context_lens on the
 * device, so a captured launch follows the lengths at each replay). For
 * chunks of a few tokens, whose rows fill a small part of a workgroup,
 * pkv_paged_attn_verify is the faster call.
 *   q:   device bf16 [num_seqs][chunk_len][n_q_heads][head_dim]
 *   out: device fp32 [num_seqs][chunk_len][n_q_heads][head_dim]
 * chunk_len in [1, 16384]. Other arguments as for pkv_paged_attn_decode.
 * Device errors: a context length outside [chunk_len, max_context_len] sets
 * PKV_DEVERR_CONTEXT, a bad block id PKV_DEVERR_BLOCK_ID; that sequence's
 * rows are NaN. */
int pkv_paged_prefill(float* out, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t num_seqs,
                      int32_t chunk_len, int32_t max_blocks_per_seq,
                      int32_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
                      int32_t head_dim, float scale, int32_t max_context_len,
                      int32_t* err_flag, void* stream);

/* The acceptance rule of speculative decoding ([M23] 23.5 and Exercises;
 * [SLS] "Speculative decoding"): for each sequence the gamma drafted tokens
 * are checked in order, draft i kept with probability
 * min(1, p_i(x_i) / q_i(x_i)), taken as the float32 decision
 * u_i * q_i(x_i) < p_i(x_i). At the first rejection (draft n) the rest are
 * discarded and one token is drawn from the leftover max(0, p_n - q_n)
 * (from p_n itself if the leftover has no weight, which exact arithmetic
 * rules out); with every draft kept, one token is drawn from p_gamma. A draw
 * with weights w returns the smallest x whose running sum exceeds
 * u_gamma * sum(w), sums in float64 (so a uniform within rounding of a
 * boundary may land on either neighbour).
 *   p_target:     device fp32 [num_seqs][gamma + 1][vocab] target probabilities
 *   q_draft:      device fp32 [num_seqs][gamma][vocab] draft probabilities
 *   draft_tokens: device int32 [num_seqs][gamma]
 *   uniforms:     device fp32 [num_seqs][gamma + 1] in [0, 1): u_0 .. u_{gamma-1}
 *                 for the keep tests, u_gamma for the draw (random numbers are
 *                 the caller's)
 *   n_accepted:   device int32 [num_seqs] out: drafts kept (0 .. gamma)
 *   next_token:   device int32 [num_seqs] out: the drawn token
 *   workspace:    device scratch of at least
 *                 pkv_spec_accept_workspace_bytes(num_seqs, vocab) bytes
 *                 (caller-owned, no initialisation needed; one call at a time)
 * A pass yields n_accepted + 1 tokens. gamma in [0, 64] (0: a plain draw
 * from p_0; q_draft and draft_tokens may then be null); vocab in
 * [1, 2097152]. A row with no positive weight draws token 0. Two launches
 * on `stream`: the weight sums of 2,048-entry tiles of the chosen rows,
 * spread over 4-tile workgroups, into the workspace; then one workgroup per
 * sequence for the draw. Host-checked errors: PKV_EINVAL for bad sizes or
 * null pointers, PKV_EWORKSPACE. Device errors: a draft outside [0, vocab)
 * sets PKV_DEVERR_TOKEN and that sequence's outputs are -1. Workspace
 * bytes: 16 * num_seqs * ceil(vocab / 2048) (two float64 sums per tile). */
size_t pkv_spec_accept_workspace_bytes(int32_t num_seqs, int32_t vocab);
int pkv_spec_accept(const float* p_target, const float* q_draft,
                    const int32_t* draft_tokens, const float* uniforms,
                    int32_t num_seqs, int32_t gamma, int32_t vocab,
                    int32_t* n_accepted, int32_t* next_token, void* workspace,
                    size_t workspace_bytes, int32_t* err_flag, void* stream);

/* Wavefronts of the decode's balanced split on the current device for this
 * shape: one per SIMD for head_dim 128 and two for head_dim 64 (fewer if the
 * kernel's occupancy were lower), at most 8192, and at most one per 16 tiles of
 * units * ceil(max_context_len / 16). (The verification pass puts two per
 * SIMD at both head sizes.) Queries the HIP runtime; returns
 * PKV_EINVAL / PKV_EUNSUPPORTED for bad shapes, PKV_EHIP without a device. */
int32_t pkv_decode_split_waves(int32_t num_seqs, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim,
                               int32_t max_context_len);

/* ------------------------------------------------------------------------
 * copy_blocks: copy-on-write support ([DSS] "Paged attention": a block
 * held by several sequences is duplicated before one of them writes to it).
 * For each pair p: the whole K and V block src[p] (all heads, all 16 slots)
 * is copied to block dst[p] of the given layer's pools. src/dst are device
 * int32 arrays of n_pairs entries; the dst blocks must be distinct and must
 * not be any src block. Device errors: an id outside [0, num_blocks) skips
 * the pair and sets PKV_DEVERR_COPY_PAIR. */
int pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src,
                    const int32_t* dst, int32_t n_pairs, int32_t num_blocks,
                    int32_t n_kv_heads, int32_t head_dim, int32_t* err_flag,
                    void* stream);

/* ------------------------------------------------------------------------
 * Host block allocator with reference counts ([SLS] "Managing the cache":
 * blocks allocated as the sequence grows, requests can share blocks; [DSS]
 * "Paged attention": shared prefix blocks, copy on write at divergence;
 * [DSS] "Continuous batching": a finished sequence releases its blocks;
 * [DSS] "Autoscaling": cache occupancy is the capacity signal).
 *
 * Host memory only, no device calls, not thread-safe (one scheduler thread
 * owns it). Free blocks form a LIFO stack: a freed block is the next one
 * handed out; a new allocator hands out 0, 1, 2, ... in order. Block ids are
 * otherwise opaque: results never depend on which ids are used.
 *
 * Tables passed to the seq functions are host int32 arrays of capacity
 * max_blocks entries, n_blocks of which are in use. */
typedef struct pkv_allocator pkv_allocator;

int pkv_allocator_create(int32_t num_blocks, pkv_allocator** out); /* num_blocks >= 1 */
void pkv_allocator_destroy(pkv_allocator* a);                      /* NULL ok */
int pkv_block_alloc(pkv_allocator* a, int32_t* id); /* refcount 1; PKV_ENOMEM if none */
int pkv_block_incref(pkv_allocator* a, int32_t id); /* EINVAL if id free/out of range */
int pkv_block_decref(pkv_allocator* a, int32_t id); /* at 0 the block is freed */
int32_t pkv_block_refcount(const pkv_allocator* a, int32_t id); /* -1 if out of range */
int32_t pkv_num_free(const pkv_allocator* a);
int32_t pkv_num_blocks(const pkv_allocator* a);

/* Make the table ready for writing position new_context_len - 1:
 *  1. allocate blocks until n_blocks >= ceil(new_context_len / 16), so a
 *     sequence holds exactly the blocks its context needs, of which only
 *     the last can be partly filled ([M23] Exercises: paging wastes less
 *     than one block per request);
 *  2. if the block holding position new_context_len - 1 has refcount > 1,
 *     copy on write: allocate a fresh block, decref the shared one, put the
 *     fresh one in the table and report the pair in (*cow_src, *cow_dst);
 *     otherwise both are set to -1. The caller must then run
 *     pkv_copy_blocks(src, dst) on every layer before the next kv_append.
 * new_context_len in [1, 16*max_blocks]. On PKV_ENOMEM the blocks already
 * added stay in the table (n_blocks says how many) and no copy-on-write was
 * done; the state is consistent and the call can be retried after a
 * release. */
int pkv_seq_grow(pkv_allocator* a, int32_t* table, int32_t* n_blocks,
                 int32_t max_blocks, int32_t new_context_len,
                 int32_t* cow_src, int32_t* cow_dst);
/* Share the first n_blocks entries of table with a new sequence: increfs
 * each (the caller copies those entries into the new sequence's table).
 * All-or-nothing: on an invalid id nothing is changed. */
int pkv_seq_fork(pkv_allocator* a, const int32_t* table, int32_t n_blocks);
/* A finished sequence: decref each of its n_blocks blocks.
 * All-or-nothing: on an invalid id nothing is changed. */
int pkv_seq_release(pkv_allocator* a, const int32_t* table, int32_t n_blocks);

/* ------------------------------------------------------------------------
 * Prefix cache ([SLS] "Reuse shared prefixes": requests that begin the
 * same way share the KV cache of that start, kept in a tree so a new
 * request picks it up instead of recomputing it; [SLS] "Caching and
 * shortcuts": with paged attention this is block sharing; [DSS] "Paged
 * attention").
 *
 * Host only, not thread-safe, over a caller's allocator (which must
 * outlive the cache). A radix tree from token prefixes (int32 token ids) to
 * the blocks holding their keys and values, at whole-block granularity:
 * only full 16-token blocks are cached (their contents never change). The
 * tree holds one reference to every block it caches.
 *
 * pkv_prefix_match: the longest cached prefix of tokens[0 .. n_tokens) of
 *   whole blocks, at most max_blocks: writes its block ids to table[0 .. m)
 *   and gives the caller one reference to each (release them with the
 *   table, pkv_seq_release). Returns m (tokens matched: 16 m). A request
 *   computes at least its last prompt token, so callers usually match
 *   n_tokens - 1 tokens.
 * pkv_prefix_insert: caches the first min(n_tokens / 16, n_blocks) blocks
 *   of a sequence (table[i] holds tokens 16i .. 16i+15): prefixes already
 *   cached keep their blocks; each newly cached block gets a reference
 *   owned by the tree. Returns the number newly cached. Every table entry
 *   used must be a live block (EINVAL otherwise).
 * pkv_prefix_evict: frees up to n_blocks, one at a time, choosing the
 *   block reached least recently (by match or insert) among the cached
 *   blocks with no cached extension whose only reference is the tree's.
 *   Returns the number freed (fewer if nothing else is evictable).
 * Negative returns are PKV_E* codes. */
typedef struct pkv_prefix_cache pkv_prefix_cache;

int pkv_prefix_cache_create(pkv_allocator* alloc, pkv_prefix_cache** out);
void pkv_prefix_cache_destroy(pkv_prefix_cache* pc); /* drops the tree's references */
int32_t pkv_prefix_match(pkv_prefix_cache* pc, const int32_t* tokens,
                         int32_t n_tokens, int32_t* table, int32_t max_blocks);
int32_t pkv_prefix_insert(pkv_prefix_cache* pc, const int32_t* tokens,
                          int32_t n_tokens, const int32_t* table,
                          int32_t n_blocks);
int32_t pkv_prefix_evict(pkv_prefix_cache* pc, int32_t n_blocks);
int32_t pkv_prefix_cached_blocks(const pkv_prefix_cache* pc);

/* ------------------------------------------------------------------------
 * Continuous batching ([DSS] "Continuous batching": each step first frees
 * the blocks of sequences that are done, then brings queued requests in
 * while room remains, then decodes the batch that results; [M23] 23.3;
 * [SLS] "Batching: static to continuous"; [DSS] "Scheduling: when prefill
 * meets decode": a sequence that runs out of memory gives up its blocks
 * and is recomputed when it comes back).
 *
 * Host only, not thread-safe. The batcher owns a block allocator of
 * num_blocks blocks and, if prefix_tokens > 0, the blocks of a shared prefix
 * (a system prompt) that requests submitted with shares_prefix begin with.
 *
 * pkv_batcher_step, in order:
 *  1. every request resident in the previous plan has produced one token;
 *     those that have produced gen_len are finished and release their
 *     blocks (finished_ids);
 *  2. every other resident request grows by this step's token
 *     (pkv_seq_grow: a block at each 16-token boundary, copy on write of a
 *     shared last block). With no free block, the most recently admitted
 *     resident request is preempted (preempted_ids): its blocks are
 *     released and it returns to the front of the queue with everything it
 *     has so far as its prompt (recomputed on re-admission);
 *  3. waiting requests are admitted in submission order while the batch
 *     holds fewer than max_batch requests and the free blocks cover the
 *     request's prompt plus its first token plus one block per resident
 *     request. A prefix-sharing request forks the prefix's blocks; the
 *     prefix's partly filled last block is copied on write before its own
 *     tokens go there.
 * The caller then, on the device and for every layer: copies the cow pairs
 * (pkv_copy_blocks), writes the fill tokens' keys and values (pkv_kv_write;
 * a prompt's prefill output, or a preempted request's recomputed tokens),
 * uploads the tables and context lengths, and runs pkv_decode_step for the
 * plan's rows. The plan's arrays stay valid until the next step. */
typedef struct pkv_batcher pkv_batcher;

typedef struct {
  int32_t num_seqs;              /* resident requests, rows 0 .. num_seqs-1 (admission order) */
  int32_t max_blocks_per_seq;    /* row stride of block_tables */
  const int32_t* block_tables;   /* [num_seqs][max_blocks_per_seq], -1 padded */
  const int32_t* context_lens;   /* [num_seqs], each including this step's token */
  const int64_t* request_ids;    /* [num_seqs] */
  int32_t n_cow;                 /* copy-on-write pairs, to copy before any write */
  const int32_t* cow_src;
  const int32_t* cow_dst;
  int32_t n_fill;                /* prompt tokens to write this step */
  const int32_t* fill_rows;      /* [n_fill] row of this plan */
  const int32_t* fill_positions; /* [n_fill] position within that row's sequence */
  int32_t n_finished;            /* requests finished and released in this step */
  const int64_t* finished_ids;
  int32_t n_preempted;           /* requests preempted in this step */
  const int64_t* preempted_ids;
  int32_t num_free_blocks;       /* after this step's allocations (occupancy) */
  int32_t num_waiting;
  int32_t n_cached_tokens;       /* prompt tokens admitted this step taken from the prefix cache */
} pkv_step_plan;

/* max_blocks_per_seq: the table width (longest request / 16, rounded up). */
int pkv_batcher_create(int32_t num_blocks, int32_t max_batch,
                       int32_t max_blocks_per_seq, int32_t prefix_tokens,
                       pkv_batcher** out);
void pkv_batcher_destroy(pkv_batcher* b); /* NULL ok */
/* The prefix's table (*table, max_blocks_per_seq entries) and its number of
 * blocks; the caller writes the prefix's keys and values through it once. */
int32_t pkv_batcher_prefix_table(const pkv_batcher* b, const int32_t** table);
/* Queue a request: prompt_len >= 1 tokens (at least the prefix if
 * shares_prefix), then gen_len >= 1 decode steps. EINVAL for a bad shape or
 * more than 16*max_blocks_per_seq tokens in all; ENOMEM if it could never
 * fit in the pool beside the prefix. */
int pkv_batcher_submit(pkv_batcher* b, int64_t request_id, int32_t prompt_len,
                       int32_t gen_len, int32_t shares_prefix);
int pkv_batcher_step(pkv_batcher* b, pkv_step_plan* plan);

/* Prefix caching in the batcher ([SLS] "Reuse shared prefixes"): after
 * pkv_batcher_enable_prefix_cache, requests submitted with their prompt's
 * token ids (pkv_batcher_submit_tokens) are matched at admission against
 * a prefix cache over the batcher's blocks (pkv_prefix_match on all but
 * the last prompt token): the cached whole blocks are forked into the
 * request's table and only the positions after them are in the plan's
 * fill list. The prompt's full blocks join the cache at admission (this
 * step's writes precede every read of them in each layer). Blocks only the
 * cache holds are evicted (least recently used leaf first) before an
 * admission is refused and before a resident request is preempted. A
 * preempted request is matched again on its prompt tokens when it
 * returns. pkv_batcher_cached_blocks: blocks the cache holds. */
int pkv_batcher_enable_prefix_cache(pkv_batcher* b);
int pkv_batcher_submit_tokens(pkv_batcher* b, int64_t request_id,
                              const int32_t* tokens, int32_t prompt_len,
                              int32_t gen_len);
int32_t pkv_batcher_cached_blocks(const pkv_batcher* b);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
