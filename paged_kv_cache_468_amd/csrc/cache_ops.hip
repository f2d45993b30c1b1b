// Writes into the paged pools: append of the step's new K/V, a write of
// arbitrary tokens (a prompt's K/V after its prefill), and whole-block
// copies for copy-on-write. Layouts are the ones include/pkv.h documents.
//
// Append ("Module 23: Serving", 23.4; "Designing an LLM serving system",
// "Paged attention"): position p = ctx - 1 of sequence s lives in block
// table[s][p / 16] at slot p % 16. One wave per (sequence, KV head); the K
// row (head_dim contiguous values) is written with 4-byte stores, the V
// column (head_dim values 32 bytes apart in the dim-major tile) with 2-byte
// stores.
//
// Copy ("Designing an LLM serving system", "Paged attention": a shared block
// is copied when a sequence that shares it writes to it): one workgroup per
// (src, dst) pair copies the K and V block, all heads, in 16-byte chunks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kXcds = 8;   // XCDs of the device; workgroups are dealt to them in turn

__global__ __launch_bounds__(256) void kv_append_kernel(
    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int num_seqs, int max_blocks, int num_blocks, int n_kv, int d, int32_t* err_flag) {
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= num_seqs * n_kv) return;
  const int s = unit / n_kv;
  const int h = unit % n_kv;
  const int ctx = context_lens[s];
  if (ctx < 1 || ctx > 16 * max_blocks) {
    if (h == 0 && lane == 0 && err_flag) atomicOr(err_flag, PKV_DEVERR_CONTEXT);
    return;
  }
  const int pos = ctx - 1;
  const int blk = block_tables[(int64_t)s * max_blocks + pos / 16];
  if (blk < 0 || blk >= num_blocks) {
    if (h == 0 && lane == 0 && err_flag) atomicOr(err_flag, PKV_DEVERR_BLOCK_ID);
    return;
  }
  const int slot = pos % 16;
  const int64_t tile = ((int64_t)blk * n_kv + h) * 16 * d;
  const uint16_t* kn = k_new + ((int64_t)s * n_kv + h) * d;
  const uint16_t* vn = v_new + ((int64_t)s * n_kv + h) * d;
  // K: row `slot` of the token-major tile, d contiguous values
  uint32_t* kdst = (uint32_t*)(k_pool + tile + (int64_t)slot * d);
  const uint32_t* ksrc = (const uint32_t*)kn;
  for (int i = lane; i < d / 2; i += 64) kdst[i] = ksrc[i];
  // V: column `slot` of the dim-major tile
  uint16_t* vdst = v_pool + tile + slot;
  for (int i = lane; i < d; i += 64) vdst[(int64_t)i * 16] = vn[i];
}

// Write of arbitrary tokens: token t goes to row seq_rows[t] at position
// positions[t]. One wave per (16 consecutive input tokens, KV head); lane
// (j, q) = (lane % 16, lane / 16) moves token j's dims 32k + 8q .. +7 with
// 16-byte loads. K rows go out as 16-byte stores. The V tile is dim-major,
// so for each of the 8 dims a store instruction writes, per q, the 16 tokens'
// values of one dim: when the tokens are consecutive positions of one block
// (a prompt written in order) that is a whole 32-byte row of the tile, and
// the wave writes every row once, instead of 16 waves each writing 2 bytes
// of it. A run of 16 that starts inside a block shares its first and last
// block's rows with the neighbouring runs: units are ordered (head, run) and
// consecutive workgroups are placed on one XCD (workgroups are dealt to the
// 8 XCDs in turn), so those halves meet in the same L2 and leave it as whole
// lines.
template <int D>
__global__ __launch_bounds__(256) void kv_write_kernel(
    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_rows,
    const int32_t* __restrict__ positions, int n_tokens, int num_seqs, int max_blocks,
    int num_blocks, int n_kv, int wg_per_xcd, int32_t* err_flag) {
  const int lane = threadIdx.x & 63;
  const int64_t wg = (int64_t)(blockIdx.x % kXcds) * wg_per_xcd + blockIdx.x / kXcds;
  const int64_t unit = wg * 4 + (threadIdx.x >> 6);
  const int64_t n_seg = ((int64_t)n_tokens + 15) / 16;
  if (unit >= n_seg * n_kv) return;
  const int h = (int)(unit / n_seg);
  const int64_t seg = unit % n_seg;
  const int j = lane & 15;
  const int q = lane >> 4;
  const int64_t tok = seg * 16 + j;
  if (tok >= n_tokens) return;
  const int row = seq_rows[tok];
  const int pos = positions[tok];
  if (row < 0 || row >= num_seqs || pos < 0 || pos >= 16 * max_blocks) {
    if (h == 0 && q == 0 && err_flag) atomicOr(err_flag, PKV_DEVERR_CONTEXT);
    return;
  }
  const int blk = block_tables[(int64_t)row * max_blocks + pos / 16];
  if (blk < 0 || blk >= num_blocks) {
    if (h == 0 && q == 0 && err_flag) atomicOr(err_flag, PKV_DEVERR_BLOCK_ID);
    return;
  }
  const int slot = pos % 16;
  const int64_t tile = ((int64_t)blk * n_kv + h) * 16 * D;
  const uint16_t* ks = k_src + (tok * n_kv + h) * D + 8 * q;
  const uint16_t* vs = v_src + (tok * n_kv + h) * D + 8 * q;
  uint16_t* kd = k_pool + tile + (int64_t)slot * D + 8 * q;
  uint16_t* vd = v_pool + tile + (int64_t)(8 * q) * 16 + slot;
  uint4 kv[D / 32], vv[D / 32];
#pragma unroll
  for (int k = 0; k < D / 32; ++k) {
    kv[k] = *(const uint4*)(ks + 32 * k);
    vv[k] = *(const uint4*)(vs + 32 * k);
  }
#pragma unroll
  for (int k = 0; k < D / 32; ++k) {
    *(uint4*)(kd + 32 * k) = kv[k];
    const uint32_t w[4] = {vv[k].x, vv[k].y, vv[k].z, vv[k].w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vd[(32 * k + e) * 16] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
  }
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool, const int32_t* __restrict__ src,
    const int32_t* __restrict__ dst, int num_blocks, int64_t chunks_per_block, int32_t* err_flag) {
  const int pair = blockIdx.x;
  const int sb = src[pair];
  const int db = dst[pair];
  if (sb < 0 || sb >= num_blocks || db < 0 || db >= num_blocks) {
    if (threadIdx.x == 0 && err_flag) atomicOr(err_flag, PKV_DEVERR_COPY_PAIR);
    return;
  }
  const uint4* ks = k_pool + (int64_t)sb * chunks_per_block;
  const uint4* vs = v_pool + (int64_t)sb * chunks_per_block;
  uint4* kd = k_pool + (int64_t)db * chunks_per_block;
  uint4* vd = v_pool + (int64_t)db * chunks_per_block;
  for (int64_t i = threadIdx.x; i < chunks_per_block; i += blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                             int32_t n_kv_heads, int32_t head_dim, int32_t* err_flag,
                             void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 1 || num_blocks < 1 || n_kv_heads < 1)
    return PKV_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !block_tables || !context_lens) return PKV_EINVAL;
  if ((int64_t)num_seqs * n_kv_heads > INT32_MAX / 2) return PKV_EINVAL;
  const unsigned grid = (unsigned)(((int64_t)num_seqs * n_kv_heads + 3) / 4);
  hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)k_pool, (uint16_t*)v_pool, (const uint16_t*)k_new,
                     (const uint16_t*)v_new, block_tables, context_lens, num_seqs,
                     max_blocks_per_seq, num_blocks, n_kv_heads, head_dim, err_flag);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

extern "C" int pkv_kv_write(void* k_pool, void* v_pool, const void* k_src, const void* v_src,
                            const int32_t* block_tables, const int32_t* seq_rows,
                            const int32_t* positions, int32_t n_tokens, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t num_blocks, int32_t n_kv_heads,
                            int32_t head_dim, int32_t* err_flag, void* stream) {
  if (n_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 1 || num_blocks < 1 || n_kv_heads < 1)
    return PKV_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if (n_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_src || !v_src || !block_tables || !seq_rows || !positions)
    return PKV_EINVAL;
  if ((int64_t)n_tokens * n_kv_heads > INT32_MAX / 2) return PKV_EINVAL;
  if (((uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)k_src | (uintptr_t)v_src) % 16)
    return PKV_EINVAL;
  const int64_t units = ((int64_t)n_tokens + 15) / 16 * n_kv_heads;
  const int wg_per_xcd = (int)(((units + 3) / 4 + kXcds - 1) / kXcds);
  const unsigned grid = (unsigned)(wg_per_xcd * kXcds);
  auto kernel = head_dim == 128 ? kv_write_kernel<128> : kv_write_kernel<64>;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (uint16_t*)k_pool,
                     (uint16_t*)v_pool, (const uint16_t*)k_src, (const uint16_t*)v_src,
                     block_tables, seq_rows, positions, n_tokens, num_seqs, max_blocks_per_seq,
                     num_blocks, n_kv_heads, wg_per_xcd, err_flag);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

extern "C" int pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src,
                               const int32_t* dst, int32_t n_pairs, int32_t num_blocks,
                               int32_t n_kv_heads, int32_t head_dim, int32_t* err_flag,
                               void* stream) {
  if (n_pairs < 0 || num_blocks < 1 || n_kv_heads < 1) return PKV_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if (n_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src || !dst) return PKV_EINVAL;
  const int64_t chunks = (int64_t)n_kv_heads * 16 * head_dim * 2 / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n_pairs), dim3(256), 0,
                     (hipStream_t)stream, (uint4*)k_pool, (uint4*)v_pool, src, dst, num_blocks,
                     chunks, err_flag);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}
