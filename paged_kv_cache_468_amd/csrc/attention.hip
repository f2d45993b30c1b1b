// Decode-phase attention over a paged KV cache, for gfx950 (MI355X).
//
// What is computed (see include/pkv.h for the layouts): for every sequence
// s and query head j, the softmax-weighted sum of the values of every cached
// token of s, weights from the scaled dot products of q[s, j] with the keys,
// keys and values reached through the sequence's block table. Sources:
// "Module 23: Serving", 23.2 (decode reads the whole KV cache for one new
// token per sequence) and 23.4 (16-token blocks behind a per-sequence
// table); "Scaling LLM serving", "The KV cache" (grouped-query heads) and
// "Make attention itself cheaper" (attention in on-chip tiles without
// materialising the score matrix, which is what the running-max softmax
// below does); "Designing an LLM serving system", "Paged attention"
// (logical to physical block indirection).
//
// Work decomposition
//   One wavefront = one (KV head h, query group, sequence s, partition).
//   A partition is P consecutive tokens (P a multiple of 16); the wave walks
//   its 16-token blocks. For each block it loads the K tile (16 x D bf16,
//   token-major) and the V tile (D x 16 bf16, dim-major), both contiguous,
//   and serves all (up to 16) query rows of the group from them, so every
//   KV byte is read from HBM once.
//
//   Scores:  S^T[t][g] = sum_k K[t][k] * Q[g][k]    16x16x32 bf16 MFMA, D/32 of them
//   Values:  O^T[n][g] += sum_t V^T[n][t] * P^T[t][g] 16x16x16 bf16 MFMA, 2 per 16 dims
//   The probabilities P (fp32) are split as P = hi + lo with hi, lo bf16, so
//   the bf16 products keep ~16 bits of P; both halves go through the MFMA.
//
//   Lane (c = lane % 16, r = lane / 16) holds, after the score MFMA, the
//   scores of tokens 4r..4r+3 for query row g = c. That is exactly the
//   B-operand layout of the value MFMA, and the value MFMA's result puts
//   dims 4r..4r+3 (+16m) of row g = c in the same lane, so the online
//   softmax (running max m, running sum l, rescale of the accumulator) needs
//   no data movement beyond a max over the four lanes of one column.
//
//   Softmax runs in the base-2 domain: x = score * scale * log2(e), weights
//   exp2(x - m). The merge kernel uses the same convention.
//
//   Grid: workgroups of 4 waves; the workgroup index is remapped so that
//   consecutive work (same KV head, neighbouring sequences) lands on the
//   same XCD (the hardware deals workgroups to the 8 XCDs round-robin), so
//   blocks shared between sequences (a common prefix) are re-read from that
//   XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef short bf16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kXcds = 8;           // XCDs of an MI355X
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  float* out;
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_ml;      // [B][n_q][p_max][2]  (m in log2 units, l)
  float* ws_acc;     // [B][n_q][p_max][D]  unnormalised accumulators
  int32_t* err_flag;
  int num_seqs, max_blocks, num_blocks;
  int n_q, n_kv, group, n_qgroups;
  int max_ctx, part_tokens, p_max;
  int total_units, wg_per_xcd;
  float scale_log2;  // scale * log2(e)
};

__device__ inline float wave_max_across_rows(float x) {
  // max over lanes c, c+16, c+32, c+48
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ inline float wave_sum_across_rows(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ inline void flag_error(int32_t* err_flag, int bit) {
  if (err_flag) atomicOr(err_flag, bit);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ inline uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int D>
__global__ __launch_bounds__(256) void paged_attn_partition_kernel(DecodeArgs a) {
  constexpr int KM = D / 32;   // score MFMAs per tile (k = 32 dims each)
  constexpr int VM = D / 16;   // value MFMA column chunks (16 dims each)

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;     // query row in the group / token row of K
  const int r = lane >> 4;     // quad: tokens 4r..4r+3 after the score MFMA

  const int logical_wg = (blockIdx.x % kXcds) * a.wg_per_xcd + blockIdx.x / kXcds;
  const int unit = logical_wg * kWaves + wave;
  if (unit >= a.total_units) return;
  const int part = unit % a.p_max;
  const int rest = unit / a.p_max;
  const int s = rest % a.num_seqs;
  const int hq = rest / a.num_seqs;
  const int h = hq / a.n_qgroups;
  const int qg = hq % a.n_qgroups;

  const int g_in_group = qg * 16 + c;
  const bool row_valid = g_in_group < a.group;
  const int j = h * a.group + g_in_group;           // query head of this lane's row
  const bool direct = a.p_max == 1;

  const int ctx = a.context_lens[s];
  if (ctx < 1 || ctx > a.max_ctx) {
    if (part == 0) {
      if (hq == 0 && lane == 0) flag_error(a.err_flag, PKV_DEVERR_CONTEXT);
      if (direct && row_valid) {
        float* o = a.out + ((int64_t)s * a.n_q + j) * D;
        for (int m = 0; m < VM; ++m)
          *(f32x4_t*)(o + 16 * m + 4 * r) = f32x4_t{__builtin_nanf(""), __builtin_nanf(""),
                                                   __builtin_nanf(""), __builtin_nanf("")};
      }
    }
    return;   // multi-partition: the merge kernel writes NaN for this sequence
  }
  const int t0 = part * a.part_tokens;
  if (t0 >= ctx) return;
  const int t1 = min(t0 + a.part_tokens, ctx);
  const int b0 = t0 >> 4;
  const int nb = ((t1 + 15) >> 4) - b0;            // <= 64 (part_tokens <= 1024)

  // Physical block ids of this partition: lane i holds entry b0 + i.
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks + b0;
  const int my_id = lane < nb ? bt_row[lane] : 0;
  const bool bad_id = lane < nb && (my_id < 0 || my_id >= a.num_blocks);
  const bool any_bad = __ballot(bad_id) != 0;

  f32x4_t acc[VM];
#pragma unroll
  for (int m = 0; m < VM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  if (!any_bad) {
    // Q as the B operand of the score MFMA: lane (c, r) holds row g = c,
    // dims 32m + 8r .. +8. Rows past the group are zero.
    bf16x8_t qv[KM];
    const uint16_t* q_row = a.q + ((int64_t)s * a.n_q + (row_valid ? j : 0)) * D;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      bf16x8_t v = *(const bf16x8_t*)(q_row + 32 * m + 8 * r);
      qv[m] = row_valid ? v : bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }

    const int64_t tile_elems = 16 * D;
    const int64_t head_off = (int64_t)h * tile_elems;
    const int64_t block_stride = (int64_t)a.n_kv * tile_elems;
    const int k_lane_off = c * D + 8 * r;          // + 32m
    const int v_lane_off = c * 16 + 4 * r;         // + 256m (16 dims x 16 tokens)

    bf16x8_t kA[KM], kB[KM];
    bf16x4_t vA[VM], vB[VM];

    auto load_tile = [&](int i, bf16x8_t* kr, bf16x4_t* vr) {
      const int blk = __builtin_amdgcn_readlane(my_id, i);
      const int64_t base = (int64_t)blk * block_stride + head_off;
      const uint16_t* kt = a.k_pool + base;
      const uint16_t* vt = a.v_pool + base;
#pragma unroll
      for (int m = 0; m < KM; ++m) kr[m] = *(const bf16x8_t*)(kt + k_lane_off + 32 * m);
#pragma unroll
      for (int m = 0; m < VM; ++m) vr[m] = *(const bf16x4_t*)(vt + v_lane_off + 256 * m);
    };

    auto compute_tile = [&](int i, const bf16x8_t* kr, bf16x4_t* vr) {
      f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KM; ++m)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[m], qv[m], sc, 0, 0, 0);
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = sc[e] * a.scale_log2;
      const int tok0 = (b0 + i) * 16;
      if (tok0 + 16 > ctx) {   // the sequence's last, partly filled block
        const int valid = ctx - tok0 - 4 * r;      // tokens of this quad still inside
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e >= valid) x[e] = -__builtin_inff();
        // masked slots may hold anything (NaN included): zero their values
        const uint32_t keep0 = (valid > 0 ? 0xFFFFu : 0u) | (valid > 1 ? 0xFFFF0000u : 0u);
        const uint32_t keep1 = (valid > 2 ? 0xFFFFu : 0u) | (valid > 3 ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int m = 0; m < VM; ++m) {
          typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));
          u32x2_t w = __builtin_bit_cast(u32x2_t, vr[m]);
          w[0] &= keep0;
          w[1] &= keep1;
          vr[m] = __builtin_bit_cast(bf16x4_t, w);
        }
      }
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = wave_max_across_rows(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(x[e] - m_new);
      l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
      for (int m = 0; m < VM; ++m) {
        acc[m][0] *= alpha; acc[m][1] *= alpha; acc[m][2] *= alpha; acc[m][3] *= alpha;
      }
      // P = hi + lo, both bf16: hi by truncation (exact remainder), lo rounded.
      uint32_t pu[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pu[e] = __float_as_uint(p[e]) & 0xFFFF0000u;
        lo[e] = bf16_rne_bits(p[e] - __uint_as_float(pu[e]));
      }
      typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));
      u32x2_t hi2 = u32x2_t{(pu[0] >> 16) | pu[1], (pu[2] >> 16) | pu[3]};
      u32x2_t lo2 = u32x2_t{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
      const bf16x4_t phi = __builtin_bit_cast(bf16x4_t, hi2);
      const bf16x4_t plo = __builtin_bit_cast(bf16x4_t, lo2);
#pragma unroll
      for (int m = 0; m < VM; ++m) {
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vr[m], phi, acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vr[m], plo, acc[m], 0, 0, 0);
      }
    };

    // Two register sets: the next tile's loads are in flight while the
    // current one is computed.
    load_tile(0, kA, vA);
    int i = 0;
    for (; i + 1 < nb; i += 2) {
      load_tile(i + 1, kB, vB);
      compute_tile(i, kA, vA);
      if (i + 2 < nb) load_tile(i + 2, kA, vA);
      compute_tile(i + 1, kB, vB);
    }
    if (i < nb) compute_tile(i, kA, vA);
  } else if (lane == 0) {
    flag_error(a.err_flag, PKV_DEVERR_BLOCK_ID);
  }

  const float l_tot = wave_sum_across_rows(l_run);
  if (!row_valid) return;
  const float nan = __builtin_nanf("");
  if (direct) {
    const float inv = any_bad ? nan : 1.0f / l_tot;
    float* o = a.out + ((int64_t)s * a.n_q + j) * D + 4 * r;
#pragma unroll
    for (int m = 0; m < VM; ++m)
      *(f32x4_t*)(o + 16 * m) = acc[m] * inv;
  } else {
    const int64_t slot = ((int64_t)s * a.n_q + j) * a.p_max + part;
    if (r == 0) {
      a.ws_ml[2 * slot] = any_bad ? nan : m_run;
      a.ws_ml[2 * slot + 1] = any_bad ? nan : l_tot;
    }
    float* w = a.ws_acc + slot * D + 4 * r;
#pragma unroll
    for (int m = 0; m < VM; ++m) *(f32x4_t*)(w + 16 * m) = acc[m];
  }
}

// Merge of the partitions of one (sequence, query head) row: with per
// partition maxima m_p, sums l_p and accumulators a_p (all relative to
// exp2(x - m_p)), out = sum_p 2^(m_p - M) a_p / sum_p 2^(m_p - M) l_p,
// M = max_p m_p. One wave per row; lane i owns dims 2i, 2i+1 (D = 128) or i.
template <int D>
__global__ __launch_bounds__(256) void paged_attn_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= a.num_seqs * a.n_q) return;
  const int s = row / a.n_q;
  const int ctx = a.context_lens[s];
  float* o = a.out + (int64_t)row * D + lane * PER;
  const float nan = __builtin_nanf("");
  if (ctx < 1 || ctx > a.max_ctx) {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = nan;
    return;
  }
  const int n_parts = (ctx + a.part_tokens - 1) / a.part_tokens;
  const float* ml = a.ws_ml + (int64_t)row * a.p_max * 2;
  float mx = -__builtin_inff();
  bool bad = false;
  for (int p = lane; p < n_parts; p += 64) {
    const float mp = ml[2 * p];
    bad |= mp != mp;
    mx = fmaxf(mx, mp);
  }
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (__ballot(bad) != 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = nan;
    return;
  }
  float lsum = 0.f;
  for (int p = lane; p < n_parts; p += 64)
    lsum += ml[2 * p + 1] * __builtin_amdgcn_exp2f(ml[2 * p] - mx);
  for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
  float res[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) res[e] = 0.f;
  const float* acc = a.ws_acc + (int64_t)row * a.p_max * D + lane * PER;
  for (int p = 0; p < n_parts; ++p) {
    const float wgt = __builtin_amdgcn_exp2f(ml[2 * p] - mx);
#pragma unroll
    for (int e = 0; e < PER; ++e) res[e] += wgt * acc[(int64_t)p * D + e];
  }
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = res[e] * inv;
}

int32_t default_partition_tokens(int num_seqs, int n_q, int n_kv, int max_ctx) {
  const int64_t qgroups = (n_q / n_kv + 15) / 16;
  int p = 512;
  while (p > 64 && (int64_t)num_seqs * n_kv * qgroups * ((max_ctx + p - 1) / p) < 8192) p >>= 1;
  return p;
}

static int resolve_partition(int partition_tokens, int num_seqs, int n_q, int n_kv, int max_ctx) {
  if (partition_tokens == 0) return default_partition_tokens(num_seqs, n_q, n_kv, max_ctx);
  return partition_tokens;
}

size_t workspace_bytes(int num_seqs, int n_q, int n_kv, int d, int max_ctx, int part) {
  const int p_max = (max_ctx + part - 1) / part;
  if (p_max <= 1) return 0;
  return (size_t)num_seqs * n_q * p_max * (2 + d) * sizeof(float);
}

}  // namespace pkv

using namespace pkv;

extern "C" int32_t pkv_default_partition_tokens(int32_t num_seqs, int32_t n_q_heads,
                                                int32_t n_kv_heads, int32_t head_dim,
                                                int32_t max_context_len) {
  (void)head_dim;
  if (num_seqs <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || max_context_len <= 0) return 512;
  return default_partition_tokens(num_seqs, n_q_heads, n_kv_heads, max_context_len);
}

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t n_q_heads,
                                             int32_t n_kv_heads, int32_t head_dim,
                                             int32_t max_context_len,
                                             int32_t partition_tokens) {
  if (num_seqs <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || max_context_len <= 0)
    return 0;
  if (partition_tokens < 0 || partition_tokens % 16 != 0 || partition_tokens > 1024) return 0;
  const int part = resolve_partition(partition_tokens, num_seqs, n_q_heads, n_kv_heads, max_context_len);
  return workspace_bytes(num_seqs, n_q_heads, n_kv_heads, head_dim, max_context_len, part);
}

// Host-side checks and launch geometry shared by the three entry points.
static int prepare(DecodeArgs& a, int& head_dim_out, float* out, const void* q, const void* k_pool,
                   const void* v_pool, const int32_t* block_tables, const int32_t* context_lens,
                   int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                   int32_t max_context_len, int32_t partition_tokens, void* workspace,
                   size_t workspace_bytes_given, int32_t* err_flag) {
  if (num_seqs < 0 || max_blocks_per_seq < 1 || num_blocks < 1 || n_q_heads < 1 ||
      n_kv_heads < 1 || max_context_len < 1)
    return PKV_EINVAL;
  if (n_q_heads % n_kv_heads != 0) return PKV_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if ((int64_t)max_context_len > 16 * (int64_t)max_blocks_per_seq) return PKV_EINVAL;
  if (partition_tokens < 0 || partition_tokens % 16 != 0 || partition_tokens > 1024)
    return PKV_EINVAL;
  if (!(scale == scale)) return PKV_EINVAL;
  if (num_seqs > 0 && (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens))
    return PKV_EINVAL;

  a.out = out;
  a.q = (const uint16_t*)q;
  a.k_pool = (const uint16_t*)k_pool;
  a.v_pool = (const uint16_t*)v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.err_flag = err_flag;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.n_q = n_q_heads;
  a.n_kv = n_kv_heads;
  a.group = n_q_heads / n_kv_heads;
  a.n_qgroups = (a.group + 15) / 16;
  a.max_ctx = max_context_len;
  a.part_tokens = resolve_partition(partition_tokens, num_seqs, n_q_heads, n_kv_heads, max_context_len);
  a.p_max = (max_context_len + a.part_tokens - 1) / a.part_tokens;
  a.scale_log2 = scale * kLog2e;
  head_dim_out = head_dim;

  const size_t need = workspace_bytes(num_seqs, n_q_heads, n_kv_heads, head_dim, max_context_len, a.part_tokens);
  if (num_seqs > 0 && need > 0 && (workspace == nullptr || workspace_bytes_given < need))
    return PKV_EWORKSPACE;
  const int64_t rows_part = (int64_t)num_seqs * n_q_heads * a.p_max;
  a.ws_ml = (float*)workspace;
  a.ws_acc = need > 0 ? (float*)workspace + 2 * rows_part : nullptr;

  const int64_t units = (int64_t)n_kv_heads * a.n_qgroups * num_seqs * a.p_max;
  if (units > (int64_t)INT32_MAX / 2) return PKV_EINVAL;
  a.total_units = (int)units;
  const int64_t wgs = (units + kWaves - 1) / kWaves;
  a.wg_per_xcd = (int)((wgs + kXcds - 1) / kXcds);
  return PKV_OK;
}

static int launch_partition(const DecodeArgs& a, int head_dim, hipStream_t st) {
  const unsigned grid = (unsigned)a.wg_per_xcd * kXcds;
  if (head_dim == 128)
    hipLaunchKernelGGL(paged_attn_partition_kernel<128>, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(paged_attn_partition_kernel<64>, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

static int launch_merge(const DecodeArgs& a, int head_dim, hipStream_t st) {
  if (a.p_max <= 1) return PKV_OK;
  const unsigned mgrid = (unsigned)(((int64_t)a.num_seqs * a.n_q + kWaves - 1) / kWaves);
  if (head_dim == 128)
    hipLaunchKernelGGL(paged_attn_merge_kernel<128>, dim3(mgrid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(paged_attn_merge_kernel<64>, dim3(mgrid), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

#define PKV_DECODE_PARAMS                                                                    \
  float *out, const void *q, const void *k_pool, const void *v_pool,                         \
      const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,            \
      int32_t max_blocks_per_seq, int32_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads, \
      int32_t head_dim, float scale, int32_t max_context_len, int32_t partition_tokens,      \
      void *workspace, size_t workspace_bytes_given, int32_t *err_flag, void *stream
#define PKV_DECODE_ARGS                                                                      \
  out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, max_blocks_per_seq,          \
      num_blocks, n_q_heads, n_kv_heads, head_dim, scale, max_context_len, partition_tokens, \
      workspace, workspace_bytes_given, err_flag

extern "C" int pkv_paged_attn_partition(PKV_DECODE_PARAMS) {
  DecodeArgs a;
  int d = 0;
  const int rc = prepare(a, d, PKV_DECODE_ARGS);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  return launch_partition(a, d, (hipStream_t)stream);
}

extern "C" int pkv_paged_attn_merge(PKV_DECODE_PARAMS) {
  DecodeArgs a;
  int d = 0;
  const int rc = prepare(a, d, PKV_DECODE_ARGS);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  return launch_merge(a, d, (hipStream_t)stream);
}

extern "C" int pkv_paged_attn_decode(PKV_DECODE_PARAMS) {
  DecodeArgs a;
  int d = 0;
  int rc = prepare(a, d, PKV_DECODE_ARGS);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  rc = launch_partition(a, d, (hipStream_t)stream);
  if (rc != PKV_OK) return rc;
  return launch_merge(a, d, (hipStream_t)stream);
}
