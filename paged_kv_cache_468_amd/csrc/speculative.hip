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
// Two kernels, so that the sweep over the vocabulary uses the whole GPU:
//   * spec_sums_kernel, kPartTiles tiles of kTile entries per workgroup
//     (kThreads threads, each taking kPer entries kThreads apart, so every
//     load is coalesced; all the workgroup's tiles in flight together):
//     lanes 0 .. gamma-1 of its first wave take the keep tests of the drafts
//     as the float32 decision u * q(x) < p(x) (a product and a comparison,
//     the same decision as u < p/q without a divide), and a ballot gives the
//     first rejection n; then each tile's sum of the draw's weights in
//     float64 (per thread, then per wave, then the waves in order) goes to
//     the workspace: the leftover max(0, p_n - q_n) and p_n itself after a
//     rejection, p_gamma otherwise (both from the same loads).
//   * spec_draw_kernel, one workgroup per sequence: the same keep tests, the
//     tiles' prefix sums in order (tile_start[k] = sum of tiles < k,
//     non-decreasing, so the tiles' ranges cover [0, total) with no gap or
//     overlap), the leftover replaced by p_n if it has no weight, and the
//     tile holding u_gamma * total. That tile is staged in LDS; its threads'
//     starting sums are formed in order at two levels (within each wave,
//     then across waves), and the one thread whose run of kPer entries holds
//     the target walks it to the first running sum above the target. Sums
//     formed in order never decrease, so at each level exactly one range
//     holds the target (or, by rounding, the target lies past the last one,
//     and the last entry with weight is taken).
// The row is read once in full and one tile a second time: V * 4 bytes (8
// for a leftover, p and q) per sequence, plus 16 bytes per tile of sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv_spec {

constexpr int kThreads = 512;
constexpr int kWavesPerSeq = kThreads / 64;
constexpr int kPer = 4;                   // entries per thread in a tile
constexpr int kTile = kThreads * kPer;    // 2048 vocabulary entries per tile
constexpr int kPartTiles = 4;             // tiles per workgroup of the sums pass (loads in flight together)
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
  double* sums;          // [B][2][n_tiles]: per tile, the leftover's sum and p_n's
  int num_seqs, gamma, vocab, n_tiles, parts;
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

// The keep tests of sequence b (threads 0 .. 63 take them, draft t by
// thread t): the first rejection (gamma if none) and whether a draft lies
// outside the vocabulary, left in *n and *bad for the whole workgroup.
__device__ inline void keep_tests(const AcceptArgs& a, int b, int* n, int* bad) {
  const int t = threadIdx.x;
  const int G = a.gamma;
  const int V = a.vocab;
  if (t < 64) {
    bool reject = false, out_of_range = false;
    if (t < G) {
      const int x = a.draft[(int64_t)b * G + t];
      out_of_range = x < 0 || x >= V;
      if (!out_of_range) {
        const float px = a.p[((int64_t)b * (G + 1) + t) * V + x];
        const float qx = a.q[((int64_t)b * G + t) * V + x];
        const float ut = a.u[(int64_t)b * (G + 1) + t];
        reject = !(ut * qx < px);
      }
    }
    const uint64_t rej = __ballot(reject);
    const uint64_t badm = __ballot(out_of_range);
    if (t == 0) {
      *n = rej ? __builtin_ctzll(rej) : G;
      *bad = badm != 0;
    }
  }
  __syncthreads();
}

// Pass A: workgroup (sequence b, part) sums the weights of tiles
// [part * kPartTiles, ..) of the chosen row. Per tile: each thread sums its
// kPer entries in float64, each wave reduces its lanes, and the waves'
// shares are added in wave order; the same order whatever the part count.
// After a rejection both the leftover's and p_n's sums come from one set of
// loads (the draw takes p_n when the leftover has no weight).
__global__ __launch_bounds__(kThreads) void spec_sums_kernel(AcceptArgs a) {
  __shared__ double wave_part[2][kPartTiles][kWavesPerSeq];
  __shared__ int shared_n, shared_bad;
  const int b = blockIdx.x / a.parts;
  const int part = blockIdx.x - b * a.parts;
  const int t = threadIdx.x;
  const int V = a.vocab;
  const int G = a.gamma;
  keep_tests(a, b, &shared_n, &shared_bad);
  if (shared_bad) return;   // the draw kernel reports it
  const int n = shared_n;
  const float* prow = a.p + ((int64_t)b * (G + 1) + n) * V;
  const float* qrow = n < G ? a.q + ((int64_t)b * G + n) * V : prow;
  const int k0 = part * kPartTiles;

  float pv[kPartTiles][kPer], qv[kPartTiles][kPer];
#pragma unroll
  for (int u = 0; u < kPartTiles; ++u)
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int x = (k0 + u) * kTile + j * kThreads + t;
      pv[u][j] = draw_weight<false>(prow, qrow, x, V);
      qv[u][j] = n < G ? qrow[x < V ? x : V - 1] : 0.f;
    }
#pragma unroll
  for (int u = 0; u < kPartTiles; ++u) {
    double s_left = 0.0, s_plain = 0.0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int x = (k0 + u) * kTile + j * kThreads + t;
      // max(0, p - q) as draw_weight<true> forms it (0 past the vocabulary)
      const float left = x < V ? fmaxf(pv[u][j] - qv[u][j], 0.f) : 0.f;
      s_left += (double)left;
      s_plain += (double)pv[u][j];
    }
    s_left = wave_sum_f64(s_left);
    s_plain = wave_sum_f64(s_plain);
    if ((t & 63) == 0) {
      wave_part[0][u][t >> 6] = s_left;
      wave_part[1][u][t >> 6] = s_plain;
    }
  }
  __syncthreads();
  if (t < 2 * kPartTiles) {
    const int kind = t / kPartTiles;   // 0: leftover, 1: plain
    const int u = t % kPartTiles;
    if (k0 + u < a.n_tiles) {
      double ts = 0.0;
#pragma unroll
      for (int w = 0; w < kWavesPerSeq; ++w) ts += wave_part[kind][u][w];
      a.sums[((int64_t)b * 2 + kind) * a.n_tiles + k0 + u] = ts;
    }
  }
}

// A float64 value of lane i (i wave-uniform).
__device__ inline double lane_f64(double x, int i) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)bits, i);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(bits >> 32), i);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Running sums in order over one wave's values: every lane forms the same
// sums c_0 = base, c_{i+1} = c_i + x_i (one addition after another, the
// same operations as a serial loop) and lane i keeps its starting sum c_i.
// Returns lane i's start; *end gets c_64.
__device__ inline double ordered_starts(double x, double base, double* end) {
  const int lane = threadIdx.x & 63;
  double c = base, mine = 0.0;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (lane == i) mine = c;
    c += lane_f64(x, i);
  }
  *end = c;
  return mine;
}

// Pass B and the outputs, one workgroup per sequence (see the top of the
// file). The first wave forms the tiles' prefix sums in order and finds
// the target's tile; then every thread stages the tile's weights.
__global__ __launch_bounds__(kThreads) void spec_draw_kernel(AcceptArgs a) {
  __shared__ float w_tile[kTile];
  __shared__ double wave_total[kWavesPerSeq];
  __shared__ int wave_last[kWavesPerSeq];
  __shared__ double shared_base, shared_target;
  __shared__ int shared_n, shared_bad, shared_tile, shared_leftover;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int V = a.vocab;
  const int G = a.gamma;
  const int n_tiles = a.n_tiles;

  // The first round of tile sums (both kinds) is loaded together with the
  // keep tests: it does not depend on their outcome.
  const double* sums = a.sums + (int64_t)b * 2 * n_tiles;
  double ts_first_left = 0.0, ts_first_plain = 0.0;
  if (wave == 0 && lane < n_tiles) {
    ts_first_left = sums[lane];
    ts_first_plain = sums[n_tiles + lane];
  }
  const float u_draw = a.u[(int64_t)b * (G + 1) + G];   // independent of the keep tests too
  keep_tests(a, b, &shared_n, &shared_bad);
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

  if (wave == 0) {
    // Prefix sums of the tiles in order, 64 tiles per round (lane l: tile
    // 64 r + l): tile_start[k] = sum of tiles < k. The leftover's; if it has
    // no weight (p = q up to rounding), p_n's instead; p_gamma's if every
    // draft was kept.
    bool leftover = n < G;
    double total = 0.0;
    // one round (at most 64 tiles, as for vocabularies up to 131,072): the
    // round's starts stay in registers for the search below
    double start1 = 0.0, next1 = 0.0;
    for (int kind = leftover ? 0 : 1; kind < 2; ++kind) {
      double c = 0.0;
      for (int r0 = 0; r0 < n_tiles; r0 += 64) {
        const double first = kind == 0 ? ts_first_left : ts_first_plain;
        const double ts = r0 == 0 ? first
                                  : (r0 + lane < n_tiles ? sums[kind * n_tiles + r0 + lane] : 0.0);
        double end_c;
        const double start = ordered_starts(ts, c, &end_c);
        // the next lane's start (every lane takes part in the shuffle, so
        // no lane reads an inactive one); the last lane's next is the end
        const double from_next = __shfl_down(start, 1);
        start1 = start;
        next1 = lane < 63 ? from_next : end_c;
        c = end_c;
      }
      total = c;
      if (kind == 0 && c > 0.0) break;
      leftover = false;
    }
    const int kind = leftover ? 0 : 1;
    const double target = (double)u_draw * total;
    // The tile whose range [tile_start[k], tile_start[k+1]) holds the
    // target; past the total (u >= 1, or rounding), the last tile with
    // weight. Each lane checks its tile of a round (with more than 64
    // tiles, the rounds' sums are formed again).
    int hit = -1, last = -1;
    double hit_base = 0.0, last_base = 0.0;
    double c = 0.0;
    for (int r0 = 0; r0 < n_tiles; r0 += 64) {
      const bool in = r0 + lane < n_tiles;
      double start = start1, next = next1;
      if (n_tiles > 64) {
        const double ts = in ? sums[kind * n_tiles + r0 + lane] : 0.0;
        double end_c;
        start = ordered_starts(ts, c, &end_c);
        const double from_next = __shfl_down(start, 1);
        next = lane < 63 ? from_next : end_c;
        c = end_c;
      }
      const uint64_t holds = __ballot(in && start <= target && target < next);
      const uint64_t has = __ballot(in && next > start);
      if (holds && hit < 0) {
        const int l = __builtin_ctzll(holds);
        hit = r0 + l;
        hit_base = lane_f64(start, l);
      }
      if (has) {
        const int l = 63 - __builtin_clzll(has);
        last = r0 + l;
        last_base = lane_f64(start, l);
      }
    }
    if (lane == 0) {
      shared_tile = hit >= 0 ? hit : last;
      shared_base = hit >= 0 ? hit_base : last_base;
      shared_target = target;
      shared_leftover = leftover;
    }
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
  const bool leftover = shared_leftover;
  const double target = shared_target;
  // Pass B, inside tile k: its weights staged in LDS (coalesced loads),
  // thread t owns the kPer consecutive entries kPer*t .. kPer*t + kPer - 1.
  // Starting sums of the threads, in order at two levels: within each wave
  // its 64 threads' runs one after another (P_i), across waves their
  // totals one after another from tile_start[k] (O_w); thread i starts at
  // O_w + P_i. Rounding is monotonic, so the starts never decrease, also
  // across waves (O_w + P_64 = O_{w+1}): exactly one thread's range holds
  // the target, or the target lies at or past the end, and that thread
  // walks its entries.
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
  double wave_sum_c;
  const double p_rel = ordered_starts(mine, 0.0, &wave_sum_c);   // P_i
  // the last thread with weight, for a target at or past the end
  const uint64_t pos = __ballot(mine > 0.0);
  if (lane == 0) {
    wave_total[wave] = wave_sum_c;
    wave_last[wave] = pos ? t + 63 - __builtin_clzll(pos) : -1;
  }
  __syncthreads();
  double o_w = shared_base, o_next = 0.0, o_end = 0.0;
  int last = -1;
  {
    double c = shared_base;
#pragma unroll
    for (int v = 0; v < kWavesPerSeq; ++v) {
      if (v == wave) o_w = c;
      c += wave_total[v];
      if (v == wave) o_next = c;
      if (wave_last[v] >= 0) last = wave_last[v];
    }
    o_end = c;
  }
  const double my_start = o_w + p_rel;
  const double from_next = __shfl_down(my_start, 1);   // all lanes take part
  const double next_start = lane < 63 ? from_next : o_next;
  const bool holds = my_start <= target && target < next_start;
  const bool past_end = !(target < o_end) && t == last;
  if (holds || past_end) {
    double c = my_start;
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

static int n_tiles_of(int32_t vocab) { return (vocab + kTile - 1) / kTile; }

}  // namespace pkv_spec

using namespace pkv_spec;

extern "C" size_t pkv_spec_accept_workspace_bytes(int32_t num_seqs, int32_t vocab) {
  if (num_seqs < 0 || vocab < 1 || vocab > kMaxTiles * kTile) return 0;
  return (size_t)num_seqs * 2 * (size_t)n_tiles_of(vocab) * sizeof(double);
}

extern "C" int pkv_spec_accept(const float* p_target, const float* q_draft,
                               const int32_t* draft_tokens, const float* uniforms,
                               int32_t num_seqs, int32_t gamma, int32_t vocab,
                               int32_t* n_accepted, int32_t* next_token, void* workspace,
                               size_t workspace_bytes, int32_t* err_flag, void* stream) {
  if (num_seqs < 0 || gamma < 0 || gamma > kMaxGamma || vocab < 1 || vocab > kMaxTiles * kTile)
    return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!p_target || !uniforms || !n_accepted || !next_token) return PKV_EINVAL;
  if (gamma > 0 && (!q_draft || !draft_tokens)) return PKV_EINVAL;
  if (!workspace || workspace_bytes < pkv_spec_accept_workspace_bytes(num_seqs, vocab))
    return PKV_EWORKSPACE;
  const int n_tiles = n_tiles_of(vocab);
  const int parts = (n_tiles + kPartTiles - 1) / kPartTiles;
  if ((int64_t)num_seqs * parts > INT32_MAX) return PKV_EINVAL;
  AcceptArgs a{p_target,   q_draft,  draft_tokens, uniforms, n_accepted, next_token, err_flag,
               (double*)workspace, num_seqs, gamma, vocab, n_tiles, parts};
  const hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(spec_sums_kernel, dim3((unsigned)(num_seqs * parts)), dim3(kThreads), 0, st, a);
  if (hipGetLastError() != hipSuccess) return PKV_EHIP;
  hipLaunchKernelGGL(spec_draw_kernel, dim3((unsigned)num_seqs), dim3(kThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}
