// The acceptance rule of speculative decoding, on the device, for gfx950.
//
// From "Module 23: Serving", 23.5 and "Scaling LLM serving", "Speculative
// decoding": the drafted tokens x_0 .. x_{gamma-1} are checked in order,
// x_i kept with probability min(1, p_i(x_i) / q_i(x_i)); at the first
// rejection the rest are discarded and one token is drawn from the leftover
// distribution max(0, p_i - q_i) (normalised); if every draft is kept, one
// more token is drawn from p_gamma. The uniforms are inputs (u_i for the
// test of draft i, u_gamma for the draw).
//
// One workgroup of 256 threads per sequence:
//   * lanes 0 .. gamma-1 of the first wave take the keep test of their draft
//     as the float32 decision u * q(x) < p(x) (a product and a comparison,
//     the same decision as u < p/q without a divide); a ballot gives the
//     first rejection;
//   * the draw, in two passes over the chosen row: (A) sums of the weights
//     per tile of 2048 entries, coalesced loads, float64, then the tiles'
//     prefix sums in order; (B) the tile holding u * total staged in LDS,
//     prefix sums of its 256 threads' runs of 8 entries in order, and the
//     thread whose run holds the target walks it to the first running sum
//     above the target. Prefix sums formed in order never decrease, so at
//     each level exactly one range holds the target (or, by rounding, the
//     target lies past the last one, and the last entry with weight is
//     taken).
// The row is read once in full and one tile a second time: V * 4 bytes (8
// for a leftover, p and q) per sequence.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv_spec {

constexpr int kThreads = 512;
constexpr int kWavesPerSeq = kThreads / 64;
constexpr int kPer = 4;                   // entries per thread in a tile
constexpr int kTile = kThreads * kPer;    // 2048 vocabulary entries per tile
constexpr int kUnroll = 4;                // tiles whose loads are in flight together
constexpr int kMaxTiles = 1024;           // vocabularies up to 2M entries
constexpr int kMaxGamma = 64;

struct AcceptArgs {
  const float* p;        // [B][gamma + 1][V]
  const float* q;        // [B][gamma][V]
  const int32_t* draft;  // [B][gamma]
  const float* u;        // [B][gamma + 1]
  int32_t* n_accepted;   // [B]
  int32_t* next_token;   // [B]
  int32_t* err_flag;
  int num_seqs, gamma, vocab;
};

// Weight of entry x for the draw: the leftover max(0, p - q) after a
// rejection at draft n < gamma (or p_n itself when the leftover is empty),
// p_gamma when every draft was kept. Entries past the vocabulary weigh 0.
// The loads are unconditional (the index clamped into the row) and the
// kind of weight is a compile-time choice, so a thread's loads of several
// entries are all in flight together.
template <bool LEFTOVER>
__device__ inline float draw_weight(const float* prow, const float* qrow, int x, int V) {
  const int xc = x < V ? x : V - 1;
  float w = prow[xc];
  if (LEFTOVER) w = fmaxf(w - qrow[xc], 0.f);
  return x < V ? w : 0.f;
}

__device__ inline double wave_sum_f64(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Pass A: per tile of kTile entries, the sum of the weights (each thread
// takes kPer entries, kThreads apart, so every load is coalesced; kUnroll
// tiles are loaded before any is reduced; each wave reduces its lanes and
// leaves its share in LDS). Then one thread turns the tile sums into prefix
// sums in order, tile_start[k] = sum of tiles < k (non-decreasing: the
// tiles' ranges [tile_start[k], tile_start[k+1]) cover [0, total) with no
// gap or overlap).
template <bool LEFTOVER>
__device__ inline void tile_sums(const float* prow, const float* qrow, int V,
                                 int n_tiles, double (*wave_part)[kWavesPerSeq],
                                 double* tile_start) {
  const int t = threadIdx.x;
  for (int k0 = 0; k0 < n_tiles; k0 += kUnroll) {
    float wv[kUnroll][kPer];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        wv[u][j] = draw_weight<LEFTOVER>(prow, qrow, (k0 + u) * kTile + j * kThreads + t, V);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      double s = 0.0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) s += (double)wv[u][j];
      s = wave_sum_f64(s);
      if ((t & 63) == 0 && k0 + u < n_tiles) wave_part[k0 + u][t >> 6] = s;
    }
  }
  __syncthreads();
  if (t == 0) {
    double c = 0.0;
    for (int k = 0; k < n_tiles; ++k) {
      tile_start[k] = c;
      double ts = 0.0;
#pragma unroll
      for (int w = 0; w < kWavesPerSeq; ++w) ts += wave_part[k][w];
      c += ts;
    }
    tile_start[n_tiles] = c;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void spec_accept_kernel(AcceptArgs a) {
  __shared__ double wave_part[kMaxTiles][kWavesPerSeq];
  __shared__ double tile_start[kMaxTiles + 1];
  __shared__ float w_tile[kTile];
  __shared__ double thread_start[kThreads + 1];
  __shared__ double wave_start[kWavesPerSeq + 1];
  __shared__ int wave_last[kWavesPerSeq];
  __shared__ int shared_n, shared_bad, shared_tile, shared_last;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int V = a.vocab;
  const int G = a.gamma;

  if (t < 64) {
    // keep test of draft t
    bool reject = false, bad = false;
    if (t < G) {
      const int x = a.draft[(int64_t)b * G + t];
      bad = x < 0 || x >= V;
      if (!bad) {
        const float px = a.p[((int64_t)b * (G + 1) + t) * V + x];
        const float qx = a.q[((int64_t)b * G + t) * V + x];
        const float ut = a.u[(int64_t)b * (G + 1) + t];
        reject = !(ut * qx < px);
      }
    }
    const uint64_t rej = __ballot(reject);
    const uint64_t badm = __ballot(bad);
    if (t == 0) {
      shared_n = rej ? __builtin_ctzll(rej) : G;
      shared_bad = badm != 0;
    }
  }
  __syncthreads();
  if (shared_bad) {
    if (t == 0) {
      a.n_accepted[b] = -1;
      a.next_token[b] = -1;
      if (a.err_flag) atomicOr(a.err_flag, PKV_DEVERR_TOKEN);
    }
    return;
  }
  const int n = shared_n;
  const float* prow = a.p + ((int64_t)b * (G + 1) + n) * V;
  const float* qrow = n < G ? a.q + ((int64_t)b * G + n) * V : prow;
  const int n_tiles = (V + kTile - 1) / kTile;

  bool leftover = n < G;
  if (leftover) {
    tile_sums<true>(prow, qrow, V, n_tiles, wave_part, tile_start);
    // nothing is left (p = q up to rounding): draw from p_n instead
    if (!(tile_start[n_tiles] > 0.0)) leftover = false;
  }
  if (!leftover) tile_sums<false>(prow, qrow, V, n_tiles, wave_part, tile_start);
  const double total = tile_start[n_tiles];
  const double target = (double)a.u[(int64_t)b * (G + 1) + G] * total;

  // the tile whose range holds the target; past the total (u >= 1, or
  // rounding), the last tile with weight
  if (t == 0) {
    shared_tile = -1;
    int last = -1;
    for (int k = 0; k < n_tiles; ++k) {
      if (tile_start[k + 1] > tile_start[k]) last = k;
      if (tile_start[k] <= target && target < tile_start[k + 1]) shared_tile = k;
    }
    if (shared_tile < 0) shared_tile = last;
  }
  __syncthreads();
  const int k = shared_tile;
  if (k < 0) {   // no weight anywhere
    if (t == 0) {
      a.n_accepted[b] = n;
      a.next_token[b] = 0;
    }
    return;
  }
  // Pass B, inside tile k: its weights staged in LDS (coalesced loads),
  // thread t owns the kPer consecutive entries kPer*t .. kPer*t + kPer - 1.
  // Starting sums of the threads, in order at two levels: lane 0 of each
  // wave sums its 64 threads' runs one after another (P_i), one thread sums
  // the waves' totals one after another from tile_start[k] (O_w), and
  // thread i starts at O_w + P_i. Rounding is monotonic, so the starts never
  // decrease, also across waves (O_w + P_64 = O_{w+1}): exactly one thread's
  // range holds the target, or the target lies at or past the end, and that
  // thread walks its entries.
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int x = k * kTile + j * kThreads + t;
    w_tile[j * kThreads + t] = leftover ? draw_weight<true>(prow, qrow, x, V)
                                        : draw_weight<false>(prow, qrow, x, V);
  }
  __syncthreads();
  double mine = 0.0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) mine += (double)w_tile[kPer * t + e];
  thread_start[t] = mine;
  __syncthreads();
  const int wave = t >> 6;
  if ((t & 63) == 0) {
    double c = 0.0;
    for (int i = t; i < t + 64; ++i) {
      const double y = thread_start[i];
      thread_start[i] = c;   // P_i, relative to the wave's start
      c += y;
    }
    wave_start[wave + 1] = c;   // the wave's total, for now
  }
  __syncthreads();
  // the last thread with weight, for a target at or past the end
  const uint64_t pos = __ballot(mine > 0.0);
  if ((t & 63) == 0) wave_last[wave] = pos ? t + 63 - __builtin_clzll(pos) : -1;
  if (t == 0) {
    double c = tile_start[k];
    for (int w = 0; w < kWavesPerSeq; ++w) {
      const double y = wave_start[w + 1];
      wave_start[w] = c;
      c += y;
    }
    wave_start[kWavesPerSeq] = c;
  }
  __syncthreads();
  if (t == 0) {
    int last = -1;
    for (int w = 0; w < kWavesPerSeq; ++w)
      if (wave_last[w] >= 0) last = wave_last[w];
    shared_last = last;
  }
  const double my_start = wave_start[wave] + thread_start[t];
  __syncthreads();
  thread_start[t] = my_start;
  if (t == 0) thread_start[kThreads] = wave_start[kWavesPerSeq];
  __syncthreads();
  const bool holds = thread_start[t] <= target && target < thread_start[t + 1];
  const bool past_end = !(target < thread_start[kThreads]) && t == shared_last;
  if (holds || past_end) {
    double c = thread_start[t];
    int tok = -1, last_pos = -1;
    for (int e = 0; e < kPer; ++e) {
      const float wx = w_tile[kPer * t + e];
      if (wx > 0.f) last_pos = e;
      c += (double)wx;
      if (holds && c > target) {
        tok = e;
        break;
      }
    }
    a.n_accepted[b] = n;
    a.next_token[b] = k * kTile + kPer * t + (tok >= 0 ? tok : last_pos);
  }
}

}  // namespace pkv_spec

using namespace pkv_spec;

extern "C" int pkv_spec_accept(const float* p_target, const float* q_draft,
                               const int32_t* draft_tokens, const float* uniforms,
                               int32_t num_seqs, int32_t gamma, int32_t vocab,
                               int32_t* n_accepted, int32_t* next_token, int32_t* err_flag,
                               void* stream) {
  if (num_seqs < 0 || gamma < 0 || gamma > kMaxGamma || vocab < 1 || vocab > kMaxTiles * kTile)
    return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!p_target || !uniforms || !n_accepted || !next_token) return PKV_EINVAL;
  if (gamma > 0 && (!q_draft || !draft_tokens)) return PKV_EINVAL;
  AcceptArgs a{p_target, q_draft, draft_tokens, uniforms, n_accepted, next_token, err_flag,
               num_seqs, gamma, vocab};
  hipLaunchKernelGGL(spec_accept_kernel, dim3((unsigned)num_seqs), dim3(kThreads), 0,
                     (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}
