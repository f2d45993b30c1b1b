// Decode-phase attention over a paged KV cache, for gfx950 (MI355X), the
// verification pass of speculative decoding ("Module 23: Serving", 23.5:
// the target model checks several drafted tokens in one pass) and chunked
// prefill ("Scaling LLM serving", "Split long prefills into chunks": a chunk
// of query tokens per sequence over its cached context; its own kernel, near
// the end of this file).
//
// What is computed (include/pkv.h has the layouts): for every sequence s and
// query head j, the softmax-weighted sum of the values of every cached token
// of s, weights from the scaled dot products of q[s, j] with the keys, keys
// and values reached through the sequence's block table. Sources:
// "Module 23: Serving", 23.2 (decode reads the whole KV cache for one new
// token per sequence) and 23.4 (16-token blocks behind a per-sequence
// table); "Scaling LLM serving", "The KV cache" (grouped-query heads) and
// "Make attention itself cheaper" (attention in on-chip tiles without
// materialising the score matrix, which is what the running-max softmax
// below does); "Designing an LLM serving system", "Paged attention"
// (logical to physical block indirection).
//
// Work decomposition
//   The query rows of KV head h are the q_len * G pairs (query token i,
//   head jj of h's group), row i*G + jj (decode: q_len = 1, the G heads).
//   A unit is one (KV head h, row group qg, sequence s): rows
//   qg*16*NG .. qg*16*NG + 16*NG - 1 (NG = 1 for the decode; the
//   verification pass of speculative decoding takes NG = 2 when a head has
//   more than 16 rows) over the ceil(ctx/16) tiles of s. A segment is a run
//   of consecutive tiles of one unit, and one wavefront processes a segment:
//   for each 16-token block it loads the K tile (16 x D bf16, token-major)
//   and the V tile (D x 16 bf16, dim-major), both contiguous, and serves all
//   rows of the unit from them, so every KV byte is read from HBM once per
//   unit. In the verification pass row i sees positions up to
//   ctx - q_len + i only (causal among the new tokens).
//
//   Balanced split (partition_tokens == 0): all tiles of the launch, in
//   (KV head, query group, sequence, tile) order, are cut into n_waves equal
//   ranges, one per wave; a wave walks its range, which may cross unit
//   boundaries, and processes one segment per unit it touches. Every wave
//   streams the same number of bytes, whatever the mix of context lengths.
//   The split depends only on the context lengths, never on block ids.
//   Fixed partitions (partition_tokens = P > 0): one wave per (unit,
//   partition of P tokens).
//
//   A segment that covers its whole unit writes out directly. Otherwise it
//   writes a partial (reference max m, sum l, unnormalised accumulator) to a
//   workspace slot and the merge kernel combines the slots of the unit.
//   Slot of a segment: balanced, wave + unit (unique: along the tile order
//   both indices only grow, and each new segment starts a new wave or a new
//   unit); fixed, unit * p_max + partition.
//
//   Per tile, with lane (c = lane % 16, r = lane / 16):
//   Scores   S^T[t][g] = sum_k K[t][k] Q[g][k]   v_mfma_f32_16x16x32_bf16, D/32 of them;
//            lane (c, r) then holds tokens 4r..4r+3 of query row g = c.
//   Values   O^T[n][g] += sum_t V^T[n][t] P^T[t][g]  one v_mfma_f32_16x16x32_bf16
//            per 16 dims: P (fp32) is split into bf16 hi + lo, and the MFMA's
//            32-long k dimension holds (token, hi) and (token, lo) pairs, the
//            V operand repeating each token's value for both, so the product
//            carries ~16 bits of P. Lane (c, r) holds dims 4r..4r+3 (+16m) of
//            row c: the same lanes as its scores, so the online softmax needs
//            no data movement beyond a max over the four lanes of a column.
//   Softmax  base 2: x = score * scale * log2(e), weights 2^(x - m). m is a
//            reference maximum: it is raised (and l, acc rescaled) only when
//            some row's tile maximum exceeds it by more than 8, so weights
//            stay below 2^8 and most tiles skip the rescale. Any reference
//            gives the same softmax, since it cancels between sum and
//            accumulator; the merge kernel uses the same convention.
//
//   Shared prefix (pkv_decode_step_prefix): the prefix's tiles become
//   prefix units, one per (KV head, 32 member rows), placed after every
//   sequence's tiles in the split; a prefix unit serves the rows of several
//   member sequences from each tile (the decode serves group rows), and a
//   member's own unit covers only its tiles after the prefix. The merge
//   kernel takes both partial lists.
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
typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kXcds = 8;             // XCDs of an MI355X
constexpr int kMaxSplitWaves = 8192; // cap of the balanced split's wave count
constexpr int kMinTilesPerWave = 16; // balanced split: at least this much work per wave
constexpr int kMaxQueryTokens = 64;  // verification pass: query tokens per sequence
constexpr int kMaxChunkTokens = 16384;  // chunked prefill: tokens per chunk
constexpr float kLog2e = 1.4426950408889634f;
// Register sets of the tile ring (tiles in flight + 1): the decode at
// head_dim 128 runs one wave per SIMD and has the registers for three; the
// other kernels run two waves per SIMD and keep two.
constexpr int kDecodeRing128 = 3;
constexpr int kRing = 2;
// Shared prefix: member rows served per prefix tile, in groups of 16.
constexpr int kPrefixNG = 2;
constexpr int kPrefixRows = 16 * kPrefixNG;
// Time per tile of a wave that reads only a shared prefix's tiles (from
// L2), relative to a wave streaming tiles from HBM: the prefix's share of
// the waves (see balanced_body). Measured best: 2/3 for the decode (4
// rows per member tile, 32 per prefix tile); 1/2 for the verification pass
// (its member tiles carry q_len times the rows, so they cost relatively
// more): 192.0 us per LLaMA-3-8B layer at 5 query tokens, against 194.9
// at 2/3 and 203.6 at 1.
constexpr int kPrefixCostNum = 2;
constexpr int kPrefixCostDen = 3;
constexpr int kVerifyPrefixCostNum = 1;
constexpr int kVerifyPrefixCostDen = 2;
constexpr float kRescaleSlack = 8.0f; // log2 units a tile max may exceed the reference

struct DecodeArgs {
  float* out;
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const uint16_t* k_new;   // append fused into the attention: [B][n_kv][D], or null
  const uint16_t* v_new;
  float* ws_ml;      // [slots][rows][2]  (reference max in log2 units, sum)
  float* ws_acc;     // [slots][rows][D]  unnormalised accumulators
  int32_t* unit_info; // balanced split: per unit, first partial slot and partial count
  int32_t* err_flag;
  int num_seqs, max_blocks, num_blocks;
  int n_q, n_kv, group;
  int q_len;         // query tokens per sequence (1: decode)
  int qrows;         // query rows per KV head: q_len * group
  int group_rows;    // rows one wave serves per unit: 16 * NG
  int n_qgroups;     // units per (KV head, sequence): ceil(qrows / group_rows)
  int rows;          // rows per partial slot: min(qrows, group_rows)
  int max_ctx;
  int part_tokens;   // 0: balanced split
  int p_max;         // fixed partitions: partitions per unit
  int n_units;       // n_kv * n_qgroups * num_seqs
  int n_waves;       // waves launched by the partition kernel
  int wg_per_xcd;
  float scale_log2;  // scale * log2(e)
  // Shared prefix (pkv_decode_step_prefix): sequences pre_first ..
  // pre_first + pre_count - 1 whose last tile lies after the prefix read its
  // pre_tiles tiles (blocks pre_table[0 .. pre_tiles - 1]) through prefix
  // units: one per (KV head, 32 member rows), pre_tiles tiles each, placed
  // after every sequence's tiles in the split. A prefix unit serves 32
  // rows of several members from each tile, and its partials (32 rows per
  // slot) go to pre_ml / pre_acc; pre_info holds each prefix unit's first
  // slot and partial count. pre_tiles = 0: no prefix.
  const int32_t* pre_table;
  int pre_first, pre_count, pre_tiles;
  int pre_qgroups;   // row groups per KV head: ceil(pre_count * qrows / kPrefixRows)
  int pre_units;     // n_kv * pre_qgroups
  int32_t* pre_info; // [pre_units][2]
  int pre_cost_num, pre_cost_den;   // relative time per prefix tile (see kPrefixCostNum)
  float* pre_ml;     // [slots][kPrefixRows][2]
  float* pre_acc;    // [slots][kPrefixRows][D]
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

__device__ inline int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ inline int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ inline void flag_error(int32_t* err_flag, int bit) {
  if (err_flag) atomicOr(err_flag, bit);
}

// Tiles of a sequence for the work split: 0 for an invalid context length,
// outside [q_len, max_ctx] (the merge kernel reports those and writes NaN
// rows).
__device__ inline int seq_tiles(int ctx, int q_len, int max_ctx) {
  return (ctx >= q_len && ctx <= max_ctx) ? (ctx + 15) >> 4 : 0;
}

// Tiles of sequence s read through the shared prefix (the prefix units'
// partials): all of them for a member whose query tokens (positions
// ctx - q_len .. ctx - 1; the decode's one new token) all lie after the
// prefix, so that every query row sees the whole prefix and no token it
// writes is in a prefix block (such a member holds the prefix's blocks as
// its first table entries; the merge checks that, and turns a member that
// does not into NaN rows); none otherwise.
__device__ inline int prefix_skip(const DecodeArgs& a, int s, int ctx) {
  return (a.pre_tiles > 0 && (unsigned)(s - a.pre_first) < (unsigned)a.pre_count &&
          ctx - a.q_len >= 16 * a.pre_tiles)
             ? a.pre_tiles
             : 0;
}

// Tiles of sequence s in the partition kernel's split: its tiles after the
// prefix (0 for an invalid context length). PREFIX = false: a kernel that
// never runs with a shared prefix (the verification pass).
template <bool PREFIX = true>
__device__ inline int unit_tiles(const DecodeArgs& a, int s, int ctx) {
  const int nt = seq_tiles(ctx, a.q_len, a.max_ctx);
  if (!PREFIX) return nt;
  return nt > 0 ? nt - prefix_skip(a, s, ctx) : 0;
}

// A compile-time flag passed as a value (to a generic lambda).
template <bool B>
struct Flag {
  constexpr operator bool() const { return B; }
};

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ inline uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline int logical_workgroup(const DecodeArgs& a) {
  return (blockIdx.x % kXcds) * a.wg_per_xcd + blockIdx.x / kXcds;
}

// Sum over all sequences of unit_tiles (identical in every lane).
template <bool PREFIX>
__device__ inline int total_seq_tiles(const DecodeArgs& a, int lane) {
  int sum = 0;
  for (int base = 0; base < a.num_seqs; base += 64) {
    const int i = base + lane;
    sum += wave_sum(i < a.num_seqs ? unit_tiles<PREFIX>(a, i, a.context_lens[i]) : 0);
  }
  return sum;
}

// The sequence holding tile r (0 <= r < total) of the per-unit-row tile
// order, and the number of tiles of the sequences before it.
template <bool PREFIX>
__device__ inline void locate_tile(const DecodeArgs& a, int lane, int r, int& s_out,
                                   int& before_out) {
  int carry = 0;
  for (int base = 0; base < a.num_seqs; base += 64) {
    const int i = base + lane;
    const int n = i < a.num_seqs ? unit_tiles<PREFIX>(a, i, a.context_lens[i]) : 0;
    const int incl = wave_inclusive_scan(n, lane) + carry;
    const uint64_t hit = __ballot(i < a.num_seqs && incl > r);
    if (hit) {
      const int ln = __builtin_ctzll(hit);
      s_out = base + ln;
      before_out = __builtin_amdgcn_readlane(incl, ln) - __builtin_amdgcn_readlane(n, ln);
      return;
    }
    carry = __builtin_amdgcn_readlane(incl, 63);
  }
  s_out = a.num_seqs;   // not reached for r < total
  before_out = carry;
}

// Load policy of a sequence: if its first block is also the first block of
// a neighbouring sequence in the batch, the sequences share a prefix and its
// blocks are read again by others, so they are loaded through the caches;
// otherwise every tile is read once and is streamed past them. Only the
// speed depends on this guess, never the result.
__device__ inline bool shares_first_block(const DecodeArgs& a, int s) {
  const int32_t* row = a.block_tables + (int64_t)s * a.max_blocks;
  const int first = row[0];
  return (s > 0 && row[-a.max_blocks] == first) ||
         (s + 1 < a.num_seqs && row[a.max_blocks] == first);
}

// The context lengths read once per wave: for up to 256 sequences each
// lane loads its (at most four) lengths, and the first table entries of
// the same sequences, together, and keeps them and the tile counts in
// registers. The total, the location of a tile, a sequence's context length
// and its load policy then follow without another round trip to memory;
// longer batches use the chunked loops above and read memory each time.
struct TileScan {
  int n[4];       // tiles of sequences lane, lane + 64, lane + 128, lane + 192
  int ctx[4];     // their context lengths
  int first[4];   // their first table entries
};

// Sequence s's value of a per-lane quadruple (s wave-uniform, s < 256).
__device__ inline int scan_value(const int (&v)[4], int s) {
  const int k = s >> 6;
  const int x = k == 0 ? v[0] : (k == 1 ? v[1] : (k == 2 ? v[2] : v[3]));
  return __builtin_amdgcn_readlane(x, s & 63);
}

// KEEP: keep the context lengths and first table entries in registers (the
// decode kernels); without it only the tile counts are kept (the
// verification pass, whose registers are spoken for).
template <bool PREFIX, bool KEEP>
__device__ inline int tile_scan_total(const DecodeArgs& a, int lane, TileScan& ts) {
  if (a.num_seqs > 256) return total_seq_tiles<PREFIX>(a, lane);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = lane + 64 * k;
    ts.ctx[k] = i < a.num_seqs ? a.context_lens[i] : 0;
    ts.first[k] = KEEP && i < a.num_seqs ? a.block_tables[(int64_t)i * a.max_blocks] : 0;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = lane + 64 * k;
    ts.n[k] = i < a.num_seqs ? unit_tiles<PREFIX>(a, i, ts.ctx[k]) : 0;
  }
  int total = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) total += wave_sum(ts.n[k]);
  return total;
}

// Context length of sequence s (from the scan's registers when it holds
// them).
template <bool KEEP>
__device__ inline int scan_ctx(const DecodeArgs& a, const TileScan& ts, int s) {
  return KEEP && a.num_seqs <= 256 ? scan_value(ts.ctx, s) : a.context_lens[s];
}

// shares_first_block from the scan's registers when it holds them.
template <bool KEEP>
__device__ inline bool scan_shares_first(const DecodeArgs& a, const TileScan& ts, int s) {
  if (!KEEP || a.num_seqs > 256) return shares_first_block(a, s);
  const int f = scan_value(ts.first, s);
  const bool prev = s > 0 && scan_value(ts.first, s > 0 ? s - 1 : 0) == f;
  const bool next = s + 1 < a.num_seqs && scan_value(ts.first, s + 1 < a.num_seqs ? s + 1 : s) == f;
  return prev || next;
}

template <bool PREFIX>
__device__ inline void tile_scan_locate(const DecodeArgs& a, int lane, const TileScan& ts, int r,
                                        int& s_out, int& before_out) {
  if (a.num_seqs > 256) {
    locate_tile<PREFIX>(a, lane, r, s_out, before_out);
    return;
  }
  int carry = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int incl = wave_inclusive_scan(ts.n[k], lane) + carry;
    const uint64_t hit = __ballot(lane + 64 * k < a.num_seqs && incl > r);
    if (hit) {
      const int ln = __builtin_ctzll(hit);
      s_out = 64 * k + ln;
      before_out = __builtin_amdgcn_readlane(incl, ln) - __builtin_amdgcn_readlane(ts.n[k], ln);
      return;
    }
    carry = __builtin_amdgcn_readlane(incl, 63);
  }
  s_out = a.num_seqs;   // not reached for r < total
  before_out = carry;
}

// The query rows one wave serves in a unit: NG groups of 16 lanes' rows,
// row c of group g being row qg * 16 * NG + 16 * g + c of the unit's KV head.
// A row stands for (query token i, head within the group jj) with
// i = row / group, jj = row % group (decode: one token, i = 0). For each
// group the lane keeps whether its row exists, the row's index into q and
// out ([num_seqs][q_len][n_q] rows of D values), and with the causal mask
// the last position the row may see (ctx - q_len + i).
template <int NG>
struct Rows {
  bool valid[NG];
  int64_t index[NG];
  int lim[NG];
};

template <int NG, bool CAUSAL>
__device__ inline Rows<NG> rows_of(const DecodeArgs& a, int lane, int s, int h, int qg, int ctx) {
  Rows<NG> rw;
  const int c = lane & 15;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int gr = qg * 16 * NG + 16 * g + c;
    rw.valid[g] = gr < a.qrows;
    if (CAUSAL) {
      const int i = gr / a.group;
      const int jj = gr - i * a.group;
      rw.index[g] = ((int64_t)s * a.q_len + i) * a.n_q + h * a.group + jj;
      rw.lim[g] = rw.valid[g] ? ctx - a.q_len + i : 0x7fffffff;
    } else {
      rw.index[g] = (int64_t)s * a.n_q + h * a.group + gr;
      rw.lim[g] = 0x7fffffff;
    }
  }
  return rw;
}

// What a segment needs loaded before its first tile: its query rows (the B
// operand of the score MFMA: lane (c, r) holds row c, dims 32m + 8r .. +8,
// zero for rows past the group) and its first block ids (lane l: the id of
// tile l, and of tile NBUF - 1 + l, clamped to the segment's last). The
// decode loop issues these loads one segment ahead, so that a wave moving
// to its next unit finds them in registers instead of waiting two memory
// round trips with its loads drained.
template <int D, int NG>
struct SegPre {
  bf16x8_t qv[NG][D / 32];
  int id0, idw;
};

template <int D, int NG, int NBUF, bool IDS = true>
__device__ inline void segment_preload(const DecodeArgs& a, int lane, int s, const Rows<NG>& rw,
                                       int ta, int tb, SegPre<D, NG>& p) {
  constexpr int KM = D / 32;
  const int r = lane >> 4;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint16_t* q_row = a.q + (rw.valid[g] ? rw.index[g] : 0) * D;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      const bf16x8_t v = *(const bf16x8_t*)(q_row + 32 * m + 8 * r);
      p.qv[g][m] = rw.valid[g] ? v : bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  if (!IDS) {   // the verification pass loads its ids in chunks of its own
    p.id0 = p.idw = 0;
    return;
  }
  const int n = tb - ta;
  const int32_t* ids = a.block_tables + (int64_t)s * a.max_blocks + ta;
  p.id0 = ids[min(lane, n - 1)];
  p.idw = ids[min(NBUF - 1 + lane, n - 1)];
}

// One segment: tiles [ta, tb) of unit (h, qg, s). Leaves, per row group g,
// the running reference max m_run[g] (log2 units, per query row c,
// identical in the 4 lanes of a column), the column's partial sum l_run[g]
// (this lane's tokens only) and the accumulator acc[g] (dims 16m + 4r .. +3
// of row c). Returns false if a block id was out of range (nothing else is
// then meaningful).
//
// With a.k_new set and the segment ending at the unit's last tile, the token
// at position ctx - 1 is this step's new one: its key and value come from
// k_new / v_new (substituted into the tile's registers, so the result never
// depends on the order of this wave's own store and load), and when
// store_new is set (the unit of the head's first query group) they are also
// written into the pools.
//
// STREAM selects non-temporal K/V loads (the tile is used once, so it is not
// kept in cache at the expense of other data); without it the loads are
// ordinary, for blocks that other sequences read too. NG row groups share
// every K/V tile. CAUSAL masks, per row, the positions after the row's own
// (the verification pass); a row may then see nothing in a whole tile, so
// its weights and rescale factors are guarded against -inf - (-inf).
// NBUF register sets hold tiles in flight (NBUF - 1 ahead of the one
// being computed).
template <int D, bool STREAM, int NG, bool CAUSAL, int NBUF>
__device__ inline bool process_segment(const DecodeArgs& a, int lane, int s, int h,
                                       const Rows<NG>& rw, int ctx, int ta, int tb, bool store_new,
                                       const SegPre<D, NG>& pre, f32x4_t (&acc)[NG][D / 16],
                                       float (&m_run)[NG], float (&l_run)[NG]) {
  constexpr int KM = D / 32;   // score MFMAs per tile (k = 32 dims each)
  constexpr int VM = D / 16;   // value MFMAs per tile (16 dims each)
  const int c = lane & 15;
  const int r = lane >> 4;

#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int m = 0; m < VM; ++m) acc[g][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[g] = -__builtin_inff();
    l_run[g] = 0.f;
  }

  const auto& qv = pre.qv;   // the query rows, loaded by segment_preload

  const int64_t tile_elems = 16 * D;
  const int64_t head_off = (int64_t)h * tile_elems;
  const int64_t block_stride = (int64_t)a.n_kv * tile_elems;
  const int k_lane_off = c * D + 8 * r;          // + 32m
  const int v_lane_off = c * 16 + 4 * r;         // + 256m (16 dims x 16 tokens)
  const int last_tile = (ctx - 1) >> 4;
  const int last_valid = ctx - last_tile * 16;   // tokens in the sequence's last tile
  const int new_slot = last_valid - 1;           // slot of position ctx - 1
  const bool has_new = !CAUSAL && a.k_new != nullptr && tb > last_tile;   // decode only
  const int first_masked = ctx - a.q_len + 1;    // causal: first position some row may not see

  bf16x8_t kn[KM];   // new token: key dims 32m + 8r .. +7
  short vn[VM];      // new token: value dim 16m + c
  if (has_new) {
    const int64_t row = ((int64_t)s * a.n_kv + h) * D;
#pragma unroll
    for (int m = 0; m < KM; ++m) kn[m] = *(const bf16x8_t*)(a.k_new + row + 32 * m + 8 * r);
#pragma unroll
    for (int m = 0; m < VM; ++m) vn[m] = (short)a.v_new[row + 16 * m + c];
  }

  // Block ids: idw holds in lane l the id of tile j0 + NBUF - 1 + l of the
  // segment (clamped to its last tile), the tiles whose loads iteration j0
  // issues; it is loaded one iteration ahead, so no id waits on a round
  // trip. An id outside the pool is never dereferenced: block 0 is read in
  // its place, and the segment reports failure (its rows become NaN) and
  // stores nothing.
  const int n = tb - ta;
  const int32_t* ids = a.block_tables + (int64_t)s * a.max_blocks + ta;
  auto ids_from = [&](int j) { return ids[min(j + lane, n - 1)]; };
  bool bad = false;

  // NBUF register sets in a ring: tile j of the segment lives in set
  // j % NBUF, and the loads of the next NBUF - 1 tiles are in flight while
  // one is computed. blk_of[b]: the (checked) block id of set b's tile.
  bf16x8_t kb[NBUF][KM];
  bf16x4_t vb[NBUF][VM];
  int blk_of[NBUF];

  // Issue the loads of the tile in block blk into set b.
  auto issue = [&](int blk, int b) {
    if ((unsigned)blk >= (unsigned)a.num_blocks) {
      bad = true;
      blk = 0;
    }
    blk_of[b] = blk;
    const int64_t base = (int64_t)blk * block_stride + head_off;
    const uint16_t* kt = a.k_pool + base;
    const uint16_t* vt = a.v_pool + base;
    if (STREAM) {
#pragma unroll
      for (int m = 0; m < KM; ++m)
        kb[b][m] = __builtin_nontemporal_load((const bf16x8_t*)(kt + k_lane_off + 32 * m));
#pragma unroll
      for (int m = 0; m < VM; ++m)
        vb[b][m] = __builtin_nontemporal_load((const bf16x4_t*)(vt + v_lane_off + 256 * m));
    } else {
#pragma unroll
      for (int m = 0; m < KM; ++m) kb[b][m] = *(const bf16x8_t*)(kt + k_lane_off + 32 * m);
#pragma unroll
      for (int m = 0; m < VM; ++m) vb[b][m] = *(const bf16x4_t*)(vt + v_lane_off + 256 * m);
    }
  };

  // Tile j of the segment, in set b. maybe_last: the tile may be the
  // unit's last (new token, partly filled block); the steady loop below
  // never computes the segment's last tile, so it passes false.
  auto compute_tile = [&](int j, int b, auto maybe_last) {
    bf16x8_t* kr = kb[b];
    bf16x4_t* vr = vb[b];
    const int tile = ta + j;
    if (maybe_last && has_new && tile == last_tile) {
      if (c == new_slot) {
#pragma unroll
        for (int m = 0; m < KM; ++m) kr[m] = kn[m];
      }
      if (r == (new_slot >> 2)) {
#pragma unroll
        for (int m = 0; m < VM; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e)   // static indices keep the ring in registers
            if (e == (new_slot & 3)) vr[m][e] = vn[m];
      }
      // stored only while every id of the segment so far was valid
      if (store_new && !bad) {
        const int blk = blk_of[b];
        const int64_t base = (int64_t)blk * block_stride + head_off;
        uint16_t* kt = (uint16_t*)a.k_pool + base;
        uint16_t* vt = (uint16_t*)a.v_pool + base;
        if (c == new_slot) {
#pragma unroll
          for (int m = 0; m < KM; ++m) *(bf16x8_t*)(kt + new_slot * D + 32 * m + 8 * r) = kn[m];
        }
        if (r == 0) {
#pragma unroll
          for (int m = 0; m < VM; ++m) vt[(16 * m + c) * 16 + new_slot] = (uint16_t)vn[m];
        }
      }
    }
    float x[NG][4];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KM; ++m)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[m], qv[g][m], sc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[g][e] = sc[e] * a.scale_log2;
    }
    if (maybe_last && tile == last_tile && last_valid < 16) {   // the partly filled last block
      const int valid = last_valid - 4 * r;         // tokens of this quad still inside
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e >= valid) x[g][e] = -__builtin_inff();
      // masked slots may hold anything (NaN included): zero their values
      const uint32_t keep0 = (valid > 0 ? 0xFFFFu : 0u) | (valid > 1 ? 0xFFFF0000u : 0u);
      const uint32_t keep1 = (valid > 2 ? 0xFFFFu : 0u) | (valid > 3 ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int m = 0; m < VM; ++m) {
        u32x2_t wv = __builtin_bit_cast(u32x2_t, vr[m]);
        wv[0] &= keep0;
        wv[1] &= keep1;
        vr[m] = __builtin_bit_cast(bf16x4_t, wv);
      }
    }
    if (CAUSAL && tile * 16 + 15 >= first_masked) {
      const int p0 = tile * 16 + 4 * r;   // position of this lane's first token
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (p0 + e > rw.lim[g]) x[g][e] = -__builtin_inff();
    }
    bf16x8_t pb[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float mx = fmaxf(fmaxf(x[g][0], x[g][1]), fmaxf(x[g][2], x[g][3]));
      mx = wave_max_across_rows(mx);
      if (__ballot(mx > m_run[g] + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_run[g], mx);
        float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
        if (CAUSAL && m_new == -__builtin_inff()) alpha = 1.f;   // row still sees nothing
        m_run[g] = m_new;
        l_run[g] *= alpha;
#pragma unroll
        for (int m = 0; m < VM; ++m) acc[g][m] *= alpha;
      }
      const float m_use = (CAUSAL && m_run[g] == -__builtin_inff()) ? 0.f : m_run[g];
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(x[g][e] - m_use);
      l_run[g] += (p[0] + p[1]) + (p[2] + p[3]);
      // P = hi + lo, both bf16: hi by truncation (exact remainder), lo rounded.
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = __float_as_uint(p[e]) & 0xFFFF0000u;
        lo[e] = bf16_rne_bits(p[e] - __uint_as_float(hi[e]));
      }
      const u32x4_t pw = u32x4_t{(hi[0] >> 16) | hi[1], (hi[2] >> 16) | hi[3],
                                 lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
      pb[g] = __builtin_bit_cast(bf16x8_t, pw);
    }
#pragma unroll
    for (int m = 0; m < VM; ++m) {
      const bf16x8_t vv = __builtin_shufflevector(vr[m], vr[m], 0, 1, 2, 3, 0, 1, 2, 3);
#pragma unroll
      for (int g = 0; g < NG; ++g)
        acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb[g], acc[g][m], 0, 0, 0);
    }
  };

  if constexpr (CAUSAL) {
    // The verification pass (two row groups, two waves per SIMD): chunks of
    // 64 tiles, two register sets, the next tile's loads in flight. The
    // ring below keeps more values live, and at this kernel's register
    // budget they spill (measured 3 % slower per call).
    for (int cb = 0; cb < n; cb += 64) {
      const int nb = min(64, n - cb);
      const int my_id = lane < nb ? ids[cb + lane] : 0;
      issue(__builtin_amdgcn_readlane(my_id, 0), 0);
      int i = 0;
      for (; i + 1 < nb; i += 2) {
        issue(__builtin_amdgcn_readlane(my_id, i + 1), 1);
        compute_tile(cb + i, 0, Flag<true>{});
        if (i + 2 < nb) issue(__builtin_amdgcn_readlane(my_id, i + 2), 0);
        compute_tile(cb + i + 1, 1, Flag<true>{});
      }
      if (i < nb) compute_tile(cb + i, 0, Flag<true>{});
    }
    return !bad;
  }
  // The steady loop runs while every load it issues is inside the segment,
  // so its loads are unconditional and the compiler's waits on them stay
  // exact; the last (at most 2 NBUF - 2) tiles are computed after it.
  const int id0 = pre.id0;   // ids of tiles 0 .. and NBUF - 1 .., from segment_preload
  int idw = pre.idw;
  int j0 = 0;
  if (n >= 2 * NBUF - 1) {
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b) issue(__builtin_amdgcn_readlane(id0, b), b);
    do {
      const int idnext = ids_from(j0 + 2 * NBUF - 1);
#pragma unroll
      for (int b = 0; b < NBUF; ++b) {
        issue(__builtin_amdgcn_readlane(idw, b), (b + NBUF - 1) % NBUF);
        compute_tile(j0 + b, b, Flag<false>{});
      }
      idw = idnext;
      j0 += NBUF;
    } while (j0 + 2 * NBUF - 2 < n);
  } else {
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b)
      if (b < n) issue(__builtin_amdgcn_readlane(id0, b), b);
  }
#pragma unroll
  for (int b = 0; b < 2 * NBUF - 2; ++b) {
    if (j0 + b + NBUF - 1 < n) issue(__builtin_amdgcn_readlane(idw, b), (b + NBUF - 1) % NBUF);
    if (j0 + b < n) compute_tile(j0 + b, b % NBUF, Flag<true>{});
  }
  return !bad;
}

// ---------------------------------------------------------------------------
// The decode's scores and P.V on the vector ALUs instead of the matrix
// cores, for comparison (pkv_decode_step_partition_valu): the same split,
// ring of register sets, append and partials as process_segment, its own
// lane layout for the tiles.
//   K: each quad of lanes holds one token, lane (c, r) token 4r + c/4, dims
//      32m + 8(c%4) .. +7 (the same 16-byte loads per lane as the matrix
//      path). The token's score is four packed bf16 dot-product chains, one
//      per lane, summed across the quad by two DPP moves.
//   q: the unit's rows staged in LDS once per segment and read per tile
//      (every lane of a quad position reads the same 16 bytes).
//   V: as in the matrix path, lane (c, r) dim 16m + c of tokens 4r .. 4r+3;
//      the weights of those four tokens are the first lanes of the row's
//      four quads, broadcast within the row by DPP (row_newbcast).
//   Softmax: base 2, reference maximum with the same slack as the matrix
//      path; a ballot finds whether any token exceeds it before any
//      reduction is taken.
// The rows per KV head are a compile-time count VG (1, 2, 4, 5 or 8; a
// group size in between takes the next, its extra rows computed on zero
// queries and dropped), so a tile is straight-line code: every row's
// scores, one ballot over all rows for the rare rescale, then every row's
// weights and P.V.
constexpr int kVecMaxG = 8;
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int kDppRowBcast = 0x150;   // + n: lane n of each row of 16 to the whole row

typedef __bf16 bf16x8v_t __attribute__((ext_vector_type(8)));
// LDS-qualified views, so volatile accesses stay LDS instructions
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

template <int CTRL>
__device__ inline float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// acc + the dot product of 8 bf16 values of k and q, in fp32, as four
// packed pair products. The pairs are taken with shufflevector: taking them
// as the dwords of a bit-cast vector has compiled to the first dword read
// four times.
__device__ inline float dot8_bf16(const bf16x8_t& k, const bf16x8_t& q, float acc) {
  const bf16x8v_t a = __builtin_bit_cast(bf16x8v_t, k);
  const bf16x8v_t b = __builtin_bit_cast(bf16x8v_t, q);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1),
                                        __builtin_shufflevector(b, b, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3),
                                        __builtin_shufflevector(b, b, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5),
                                        __builtin_shufflevector(b, b, 4, 5), acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7),
                                         __builtin_shufflevector(b, b, 6, 7), acc, false);
}

// One vector-ALU segment, tiles [ta, tb) of unit (h, qg = 0, s). Leaves per
// row g: m_run[g] (identical in every lane), l_run[g] (this lane's token's
// weights: every token is counted by the four lanes of its quad) and
// acc[g][m] (dim 16m + c over this lane's tokens 4r .. 4r+3).
template <int D, bool STREAM, int NBUF, int VG>
__device__ inline bool process_segment_valu(const DecodeArgs& a, int lane, int s, int h, int ctx,
                                            int ta, int tb, bool store_new,
                                            const SegPre<D, 1>& pre, float (&acc)[VG][D / 16],
                                            float (&m_run)[VG], float (&l_run)[VG]) {
  constexpr int KM = D / 32;
  constexpr int VM = D / 16;
  const int c = lane & 15;
  const int r = lane >> 4;
  const int tok = 4 * r + (c >> 2);   // this lane's token within a tile
  const int quarter = 8 * (c & 3);    // its first dim within each 32

#pragma unroll
  for (int g = 0; g < VG; ++g) {
#pragma unroll
    for (int m = 0; m < VM; ++m) acc[g][m] = 0.f;
    m_run[g] = -__builtin_inff();
    l_run[g] = 0.f;
  }
  // The unit's query rows into this wave's LDS slice: lane (c, r) holds row
  // c's dims 32m + 8r .. +7 (rows past the group are zeros). Reads and
  // writes of the slice are volatile, so they stay in program order (one
  // wave's LDS operations complete in order) and the per-tile reads are not
  // hoisted into registers.
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[kWaves][VG * D];
  volatile lds_u16_t* qs = (volatile lds_u16_t*)q_lds[threadIdx.x >> 6];
  if (c < VG) {
#pragma unroll
    for (int m = 0; m < KM; ++m)
      *(volatile lds_bf16x8_t*)(qs + c * D + 32 * m + 8 * r) = pre.qv[0][m];
  }

  const int64_t tile_elems = 16 * D;
  const int64_t head_off = (int64_t)h * tile_elems;
  const int64_t block_stride = (int64_t)a.n_kv * tile_elems;
  const int k_lane_off = tok * D + quarter;
  const int v_lane_off = c * 16 + 4 * r;
  const int last_tile = (ctx - 1) >> 4;
  const int last_valid = ctx - last_tile * 16;
  const int new_slot = last_valid - 1;
  const bool has_new = a.k_new != nullptr && tb > last_tile;

  bf16x8_t kn[KM];   // new token: key dims 32m + quarter .. +7
  short vn[VM];      // new token: value dim 16m + c
  if (has_new) {
    const int64_t row = ((int64_t)s * a.n_kv + h) * D;
#pragma unroll
    for (int m = 0; m < KM; ++m) kn[m] = *(const bf16x8_t*)(a.k_new + row + 32 * m + quarter);
#pragma unroll
    for (int m = 0; m < VM; ++m) vn[m] = (short)a.v_new[row + 16 * m + c];
  }

  const int n = tb - ta;
  const int32_t* ids = a.block_tables + (int64_t)s * a.max_blocks + ta;
  auto ids_from = [&](int j) { return ids[min(j + lane, n - 1)]; };
  bool bad = false;
  bf16x8_t kb[NBUF][KM];
  bf16x4_t vb[NBUF][VM];
  int blk_of[NBUF];

  auto issue = [&](int blk, int b) {
    if ((unsigned)blk >= (unsigned)a.num_blocks) {
      bad = true;
      blk = 0;
    }
    blk_of[b] = blk;
    const int64_t base = (int64_t)blk * block_stride + head_off;
    const uint16_t* kt = a.k_pool + base;
    const uint16_t* vt = a.v_pool + base;
    if (STREAM) {
#pragma unroll
      for (int m = 0; m < KM; ++m)
        kb[b][m] = __builtin_nontemporal_load((const bf16x8_t*)(kt + k_lane_off + 32 * m));
#pragma unroll
      for (int m = 0; m < VM; ++m)
        vb[b][m] = __builtin_nontemporal_load((const bf16x4_t*)(vt + v_lane_off + 256 * m));
    } else {
#pragma unroll
      for (int m = 0; m < KM; ++m) kb[b][m] = *(const bf16x8_t*)(kt + k_lane_off + 32 * m);
#pragma unroll
      for (int m = 0; m < VM; ++m) vb[b][m] = *(const bf16x4_t*)(vt + v_lane_off + 256 * m);
    }
  };

  auto compute_tile = [&](int j, int b, auto maybe_last) {
    bf16x8_t* kr = kb[b];
    bf16x4_t* vr = vb[b];
    const int tile = ta + j;
    if (maybe_last && has_new && tile == last_tile) {
      if (tok == new_slot) {
#pragma unroll
        for (int m = 0; m < KM; ++m) kr[m] = kn[m];
      }
      if (r == (new_slot >> 2)) {
#pragma unroll
        for (int m = 0; m < VM; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e == (new_slot & 3)) vr[m][e] = vn[m];
      }
      if (store_new && !bad) {
        const int64_t base = (int64_t)blk_of[b] * block_stride + head_off;
        uint16_t* kt = (uint16_t*)a.k_pool + base;
        uint16_t* vt = (uint16_t*)a.v_pool + base;
        if (tok == new_slot) {
#pragma unroll
          for (int m = 0; m < KM; ++m) *(bf16x8_t*)(kt + new_slot * D + 32 * m + quarter) = kn[m];
        }
        if (r == 0) {
#pragma unroll
          for (int m = 0; m < VM; ++m) vt[(16 * m + c) * 16 + new_slot] = (uint16_t)vn[m];
        }
      }
    }
    const bool partly = maybe_last && tile == last_tile && last_valid < 16;
    if (partly) {   // values past the context may hold anything (NaN included): zeroed
      const int valid = last_valid - 4 * r;
      const uint32_t keep0 = (valid > 0 ? 0xFFFFu : 0u) | (valid > 1 ? 0xFFFF0000u : 0u);
      const uint32_t keep1 = (valid > 2 ? 0xFFFFu : 0u) | (valid > 3 ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int m = 0; m < VM; ++m) {
        u32x2_t wv = __builtin_bit_cast(u32x2_t, vr[m]);
        wv[0] &= keep0;
        wv[1] &= keep1;
        vr[m] = __builtin_bit_cast(bf16x4_t, wv);
      }
    }
    // every row's score of this lane's token
    float x[VG];
#pragma unroll
    for (int g = 0; g < VG; ++g) {
      float sc = 0.f;
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const bf16x8_t qv = *(const volatile lds_bf16x8_t*)(qs + g * D + 32 * m + quarter);
        sc = dot8_bf16(kr[m], qv, sc);
      }
      sc += dpp_f32<kDppQuadXor1>(sc);
      sc += dpp_f32<kDppQuadXor2>(sc);   // the token's whole score, in all four lanes
      x[g] = (partly && tok >= last_valid) ? -__builtin_inff() : sc * a.scale_log2;
    }
    // one ballot for all rows; the reductions and rescales only when some
    // token exceeds its row's reference maximum (rare after a row's first
    // tile)
    bool over = false;
#pragma unroll
    for (int g = 0; g < VG; ++g) over = over || x[g] > m_run[g] + kRescaleSlack;
    if (__ballot(over) != 0) {
#pragma unroll
      for (int g = 0; g < VG; ++g) {
        float mx = x[g];
#pragma unroll
        for (int off = 4; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if (mx > m_run[g] + kRescaleSlack) {   // the same in every lane
          const float m_new = fmaxf(m_run[g], mx);
          const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
          m_run[g] = m_new;
          l_run[g] *= alpha;
#pragma unroll
          for (int m = 0; m < VM; ++m) acc[g][m] *= alpha;
        }
      }
    }
    bf16x8_t vv[VM];   // tokens 4r .. 4r+3 twice, the hi and the lo half of the pairs
#pragma unroll
    for (int m = 0; m < VM; ++m) vv[m] = __builtin_shufflevector(vr[m], vr[m], 0, 1, 2, 3, 0, 1, 2, 3);
#pragma unroll
    for (int g = 0; g < VG; ++g) {
      const float p = __builtin_amdgcn_exp2f(x[g] - m_run[g]);
      l_run[g] += p;
      // weights of tokens 4r .. 4r+3, each as bf16 hi (truncated: exact
      // remainder) + lo (rounded), paired for the packed dot products
      const float pt[4] = {dpp_f32<kDppRowBcast + 0>(p), dpp_f32<kDppRowBcast + 4>(p),
                           dpp_f32<kDppRowBcast + 8>(p), dpp_f32<kDppRowBcast + 12>(p)};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = __float_as_uint(pt[e]) & 0xFFFF0000u;
        lo[e] = bf16_rne_bits(pt[e] - __uint_as_float(hi[e]));
      }
      const bf16x8_t pw = __builtin_bit_cast(
          bf16x8_t, u32x4_t{(hi[0] >> 16) | hi[1], (hi[2] >> 16) | hi[3], lo[0] | (lo[1] << 16),
                            lo[2] | (lo[3] << 16)});
#pragma unroll
      for (int m = 0; m < VM; ++m) acc[g][m] = dot8_bf16(vv[m], pw, acc[g][m]);
    }
  };

  // the ring and loop of process_segment
  const int id0 = pre.id0;
  int idw = pre.idw;
  int j0 = 0;
  if (n >= 2 * NBUF - 1) {
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b) issue(__builtin_amdgcn_readlane(id0, b), b);
    do {
      const int idnext = ids_from(j0 + 2 * NBUF - 1);
#pragma unroll
      for (int b = 0; b < NBUF; ++b) {
        issue(__builtin_amdgcn_readlane(idw, b), (b + NBUF - 1) % NBUF);
        compute_tile(j0 + b, b, Flag<false>{});
      }
      idw = idnext;
      j0 += NBUF;
    } while (j0 + 2 * NBUF - 2 < n);
  } else {
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b)
      if (b < n) issue(__builtin_amdgcn_readlane(id0, b), b);
  }
#pragma unroll
  for (int b = 0; b < 2 * NBUF - 2; ++b) {
    if (j0 + b + NBUF - 1 < n) issue(__builtin_amdgcn_readlane(idw, b), (b + NBUF - 1) % NBUF);
    if (j0 + b < n) compute_tile(j0 + b, b % NBUF, Flag<true>{});
  }
  return !bad;
}

// A finished vector-ALU segment: per row, l summed over the wave (each
// token counted four times, so a quarter of it: exact in binary) and the
// accumulators over the four lanes r of a dim; then, as finish_rows does,
// out directly or a partial. Lane (c, r) writes dims 16m + c for
// m = r, r + 4, ... of every row.
template <int D, int VG>
__device__ inline void finish_rows_valu(const DecodeArgs& a, int lane, bool ok, bool whole,
                                        int64_t slot, int s, int h, float (&acc)[VG][D / 16],
                                        const float (&m_run)[VG], const float (&l_run)[VG]) {
  constexpr int VM = D / 16;
  const int c = lane & 15;
  const int r = lane >> 4;
  if (!ok && lane == 0) flag_error(a.err_flag, PKV_DEVERR_BLOCK_ID);
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int g = 0; g < VG; ++g) {
    if (g >= a.group) break;
    float l = l_run[g];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) l += __shfl_xor(l, off);
    l *= 0.25f;
#pragma unroll
    for (int m = 0; m < VM; ++m) {
      acc[g][m] += __shfl_xor(acc[g][m], 16);
      acc[g][m] += __shfl_xor(acc[g][m], 32);
    }
    const int64_t out_row = (int64_t)s * a.n_q + h * a.group + g;
    if (whole) {
      const float inv = ok ? 1.0f / l : nan;
#pragma unroll
      for (int m = 0; m < VM; ++m)
        if ((m & 3) == r) a.out[out_row * D + 16 * m + c] = acc[g][m] * inv;
    } else {
      const int64_t row = slot * a.rows + g;
      if (lane == 0) {
        a.ws_ml[2 * row] = ok ? m_run[g] : nan;
        a.ws_ml[2 * row + 1] = ok ? l : nan;
      }
#pragma unroll
      for (int m = 0; m < VM; ++m)
        if ((m & 3) == r) a.ws_acc[row * D + 16 * m + c] = acc[g][m];
    }
  }
}

// Write a finished segment's row: out directly when the segment covers its
// whole unit, else a partial into its workspace slot (row g_in_slot of the
// slot). Rows past the group write nothing.
template <int D>
__device__ inline void finish_segment(const DecodeArgs& a, int lane, bool ok, bool whole,
                                      int64_t slot, int64_t out_row, int g_in_slot,
                                      bool row_valid, const f32x4_t* acc, float m_run,
                                      float l_run) {
  constexpr int VM = D / 16;
  const int r = lane >> 4;
  const float l_tot = wave_sum_across_rows(l_run);
  if (!row_valid) return;
  const float nan = __builtin_nanf("");
  if (whole) {
    const float inv = ok ? 1.0f / l_tot : nan;
    float* o = a.out + out_row * D + 4 * r;
#pragma unroll
    for (int m = 0; m < VM; ++m) *(f32x4_t*)(o + 16 * m) = acc[m] * inv;
  } else {
    const int64_t row = slot * a.rows + g_in_slot;
    if (r == 0) {
      a.ws_ml[2 * row] = ok ? m_run : nan;
      a.ws_ml[2 * row + 1] = ok ? l_tot : nan;
    }
    float* w = a.ws_acc + row * D + 4 * r;
#pragma unroll
    for (int m = 0; m < VM; ++m) *(f32x4_t*)(w + 16 * m) = acc[m];
  }
}

template <int D, int NG>
__device__ inline void finish_rows(const DecodeArgs& a, int lane, bool ok, bool whole,
                                   int64_t slot, const Rows<NG>& rw,
                                   const f32x4_t (&acc)[NG][D / 16], const float (&m_run)[NG],
                                   const float (&l_run)[NG]) {
  if (!ok && lane == 0) flag_error(a.err_flag, PKV_DEVERR_BLOCK_ID);
#pragma unroll
  for (int g = 0; g < NG; ++g)
    finish_segment<D>(a, lane, ok, whole, slot, rw.index[g], 16 * g + (lane & 15), rw.valid[g],
                      acc[g], m_run[g], l_run[g]);
}

// First wave and last wave (inclusive) of the balanced split that touch
// tiles [t0, t1) of the launch order, t1 > t0.
__device__ inline void waves_of_range(int64_t t0, int64_t t1, int64_t total, int n_waves,
                                      int& w0, int& w1) {
  // wave of tile x: the largest w with floor(w*total/W) <= x
  w0 = (int)(((t0 + 1) * n_waves - 1) / total);
  w1 = (int)((t1 * n_waves - 1) / total);
}

// Fixed partitions: one wave per (unit, partition). Decode only.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void paged_attn_fixed_kernel(DecodeArgs a) {
  constexpr int VM = D / 16;
  const int lane = threadIdx.x & 63;
  const int unit_part = logical_workgroup(a) * kWaves + (threadIdx.x >> 6);
  if (unit_part >= a.n_units * a.p_max) return;
  const int part = unit_part % a.p_max;
  const int u = unit_part / a.p_max;
  const int s = u % a.num_seqs;
  const int hq = u / a.num_seqs;
  const int h = hq / a.n_qgroups;
  const int qg = hq % a.n_qgroups;

  const int ctx = a.context_lens[s];
  const int nt = seq_tiles(ctx, a.q_len, a.max_ctx);   // invalid: 0, reported by the merge
  const int tiles_per_part = a.part_tokens >> 4;
  const int ta = part * tiles_per_part;
  if (ta >= nt) return;
  const int tb = min(ta + tiles_per_part, nt);

  const Rows<1> rw = rows_of<1, false>(a, lane, s, h, qg, ctx);
  SegPre<D, 1> pre;
  segment_preload<D, 1, kRing>(a, lane, s, rw, ta, tb, pre);
  f32x4_t acc[1][VM];
  float m_run[1], l_run[1];
  const bool ok =
      shares_first_block(a, s)
          ? process_segment<D, false, 1, false, kRing>(a, lane, s, h, rw, ctx, ta, tb, false, pre,
                                                       acc, m_run, l_run)
          : process_segment<D, true, 1, false, kRing>(a, lane, s, h, rw, ctx, ta, tb, false, pre,
                                                      acc, m_run, l_run);
  finish_rows<D, 1>(a, lane, ok, ta == 0 && tb == nt, (int64_t)u * a.p_max + part, rw, acc, m_run,
                    l_run);
}

// A prefix unit's partial (kPrefixRows rows per slot; row group g):
// reference max, sum and accumulator of the rows this wave served, NaN
// after a bad block id.
template <int D>
__device__ inline void write_prefix_partial(const DecodeArgs& a, int lane, bool ok, int64_t slot,
                                            int g, bool valid, const f32x4_t* acc, float m_run,
                                            float l_run) {
  constexpr int VM = D / 16;
  const int r = lane >> 4;
  const float l_tot = wave_sum_across_rows(l_run);
  if (!valid) return;
  const float nan = __builtin_nanf("");
  const int64_t row = slot * kPrefixRows + 16 * g + (lane & 15);
  if (r == 0) {
    a.pre_ml[2 * row] = ok ? m_run : nan;
    a.pre_ml[2 * row + 1] = ok ? l_tot : nan;
  }
  float* o = a.pre_acc + row * D + 4 * r;
#pragma unroll
  for (int m = 0; m < VM; ++m) *(f32x4_t*)(o + 16 * m) = acc[m];
}

// The rows of prefix unit pu: a member's qrows rows (query token i, head
// jj of KV head h's group; the decode's one token), row
// member * qrows + i * group + jj, rows qg * 32 .. qg * 32 + 31 of KV head h
// (two groups of 16). Every prefix position is visible to all of them.
__device__ inline Rows<kPrefixNG> prefix_rows(const DecodeArgs& a, int lane, int h, int qg) {
  Rows<kPrefixNG> rw;
#pragma unroll
  for (int g = 0; g < kPrefixNG; ++g) {
    const int gr = qg * kPrefixRows + 16 * g + (lane & 15);
    rw.valid[g] = gr < a.pre_count * a.qrows;
    const int member = gr / a.qrows;
    const int rem = gr - member * a.qrows;
    const int i = rem / a.group;
    rw.index[g] = ((int64_t)(a.pre_first + member) * a.q_len + i) * a.n_q + h * a.group +
                  (rem - i * a.group);
    rw.lim[g] = 0x7fffffff;
  }
  return rw;
}

// Tiles [ta, tb) of prefix unit pu, through the prefix's own table: every
// block is full, none is written, and the tiles are read by the other
// prefix units of the KV head too (so through the caches).
template <int D, int NBUF>
__device__ inline void prefix_segment(const DecodeArgs& a, int lane, int pu, int ta, int tb,
                                      int64_t slot) {
  constexpr int VM = D / 16;
  const int h = pu / a.pre_qgroups;
  const Rows<kPrefixNG> rw = prefix_rows(a, lane, h, pu % a.pre_qgroups);
  DecodeArgs pa = a;
  pa.block_tables = a.pre_table;
  pa.max_blocks = a.pre_tiles;
  pa.k_new = nullptr;
  pa.v_new = nullptr;
  SegPre<D, kPrefixNG> pre;
  segment_preload<D, kPrefixNG, NBUF>(pa, lane, 0, rw, ta, tb, pre);
  f32x4_t acc[kPrefixNG][VM];
  float m_run[kPrefixNG], l_run[kPrefixNG];
  const bool ok = process_segment<D, false, kPrefixNG, false, NBUF>(
      pa, lane, 0, h, rw, a.pre_tiles * 16, ta, tb, false, pre, acc, m_run, l_run);
  if (!ok && lane == 0) flag_error(a.err_flag, PKV_DEVERR_BLOCK_ID);
#pragma unroll
  for (int g = 0; g < kPrefixNG; ++g)
    write_prefix_partial<D>(a, lane, ok, slot, g, rw.valid[g], acc[g], m_run[g], l_run[g]);
}

// Balanced split: wave w processes tiles [w*T/W, (w+1)*T/W) of the
// (head, group, sequence, tile) order, T = all tiles of the launch. With a
// shared prefix the waves form two classes: waves [0, W - Wp) split the
// sequences' tiles that way, and the last Wp waves split the prefix units'
// tiles, in (KV head, row group, tile) order. Wp follows from the tile
// counts and the relative cost of a prefix tile (a wave that reads only
// L2-resident prefix tiles takes about pre_cost_num / pre_cost_den of
// the time per tile of a wave streaming from HBM), so both classes end
// together. (With a single wave, one order holds both.) The wave holding
// a unit's first tile records, for the merge kernel, the unit's first
// partial slot and its number of partials (1: written here).
template <int D, int NG, bool CAUSAL, int NBUF, bool PREFIX, int VG = 0>
__device__ inline void balanced_body(const DecodeArgs& a) {
  static_assert(VG == 0 || (!PREFIX && !CAUSAL && NG == 1), "vector-ALU path: the plain decode only");
  constexpr int VM = D / 16;
  const int lane = threadIdx.x & 63;
  const int w = logical_workgroup(a) * kWaves + (threadIdx.x >> 6);
  if (w >= a.n_waves) return;

  TileScan ts;
  constexpr bool KEEP = !CAUSAL;
  const int per_row = tile_scan_total<PREFIX, KEEP>(a, lane, ts);   // tiles of one (head, group)
  const int n_hq = a.n_kv * a.n_qgroups;
  const int64_t t_seq = (int64_t)n_hq * per_row;
  const int64_t t_pre = PREFIX ? (int64_t)a.pre_units * a.pre_tiles : 0;
  int w_pre = 0;   // waves of the prefix class (0: one order for all tiles)
  if (PREFIX && t_pre > 0 && a.n_waves >= 2) {
    if (t_seq == 0) {
      w_pre = a.n_waves;
    } else {
      const int64_t num = (int64_t)a.n_waves * a.pre_cost_num * t_pre;
      const int64_t den = t_seq * a.pre_cost_den + (int64_t)a.pre_cost_num * t_pre;
      w_pre = (int)max((int64_t)1, min((int64_t)a.n_waves - 1, (num + den / 2) / den));
    }
  }
  // This wave's span: its tiles, waves and first wave, and where in it the
  // prefix units begin.
  const bool pre_class = w_pre > 0 && w >= a.n_waves - w_pre;
  const int64_t total = w_pre == 0 ? t_seq + t_pre : (pre_class ? t_pre : t_seq);
  const int span_waves = w_pre == 0 ? a.n_waves : (pre_class ? w_pre : a.n_waves - w_pre);
  const int wave_base = pre_class ? a.n_waves - w_pre : 0;
  const int64_t pre_origin = pre_class ? 0 : t_seq;
  int64_t cur = total * (w - wave_base) / span_waves;
  const int64_t end = total * (w - wave_base + 1) / span_waves;

  // Prefix segments from tile c (at or after pre_origin) up to end.
  auto prefix_walk = [&](int64_t c) {
    int pu = (int)((c - pre_origin) / a.pre_tiles);
    int pos = (int)((c - pre_origin) - (int64_t)pu * a.pre_tiles);
    while (c < end) {
      const int tb = (int)min((int64_t)a.pre_tiles, pos + (end - c));
      if (pos == 0 && lane == 0) {
        int w0, w1;
        waves_of_range(c, c + a.pre_tiles, total, span_waves, w0, w1);
        a.pre_info[2 * pu] = wave_base + w0 + pu;
        a.pre_info[2 * pu + 1] = w1 - w0 + 1;
      }
      prefix_segment<D, NBUF>(a, lane, pu, pos, tb, (int64_t)w + pu);
      c += tb - pos;
      pos = 0;
      ++pu;
    }
  };

  if (cur >= end) {
    // An empty range (fewer tiles than waves). If it sits strictly inside a
    // unit (after the unit's first tile), the merge of that unit counts
    // this wave: leave a neutral partial (weight 2^-inf, sum 0, accumulator
    // 0) in its slot. At a unit's first tile it belongs to no unit.
    f32x4_t zero[NG][VM];
    float m0[NG], l0[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int m = 0; m < VM; ++m) zero[g][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m0[g] = -__builtin_inff();
      l0[g] = 0.f;
    }
    if (cur < pre_origin) {
      const int hq = (int)(cur / per_row);
      int s, before;
      tile_scan_locate<PREFIX>(a, lane, ts, (int)(cur - (int64_t)hq * per_row), s, before);
      if (s >= a.num_seqs || (int)(cur - (int64_t)hq * per_row) == before) return;
      const int u = hq * a.num_seqs + s;
      const Rows<NG> rw = rows_of<NG, CAUSAL>(a, lane, s, hq / a.n_qgroups, hq % a.n_qgroups,
                                              scan_ctx<KEEP>(a, ts, s));
      finish_rows<D, NG>(a, lane, true, false, (int64_t)w + u, rw, zero, m0, l0);
    } else if (PREFIX && cur < total) {
      const int pu = (int)((cur - pre_origin) / a.pre_tiles);
      if (cur - pre_origin == (int64_t)pu * a.pre_tiles) return;
      const Rows<kPrefixNG> rw = prefix_rows(a, lane, pu / a.pre_qgroups, pu % a.pre_qgroups);
#pragma unroll
      for (int g = 0; g < kPrefixNG; ++g)
        write_prefix_partial<D>(a, lane, true, (int64_t)w + pu, g, rw.valid[g], zero[0], m0[0],
                                l0[0]);
    }
    return;
  }
  if (PREFIX && cur >= pre_origin) {
    prefix_walk(cur);
    return;
  }

  int hq = (int)(cur / per_row);
  int s, before;
  tile_scan_locate<PREFIX>(a, lane, ts, (int)(cur - (int64_t)hq * per_row), s, before);
  if (s >= a.num_seqs) return;   // unreachable for consistent context lengths
  int pos = (int)(cur - (int64_t)hq * per_row) - before;   // tile within the unit
  int ctx = scan_ctx<KEEP>(a, ts, s);

  // The first segment's query rows and block ids; later ones are loaded
  // while the segment before them streams (decode; the verification pass
  // loads each segment's at its start).
  SegPre<D, NG> pre;
  {
    const int skip = PREFIX ? prefix_skip(a, s, ctx) : 0;
    const int tb = (int)min((int64_t)unit_tiles<PREFIX>(a, s, ctx), pos + (end - cur));
    segment_preload<D, NG, NBUF, !CAUSAL>(
        a, lane, s, rows_of<NG, CAUSAL>(a, lane, s, hq / a.n_qgroups, hq % a.n_qgroups, ctx),
        skip + pos, skip + tb, pre);
  }

  while (true) {
    const int nt = unit_tiles<PREFIX>(a, s, ctx);
    const int skip = PREFIX ? prefix_skip(a, s, ctx) : 0;   // tiles before the unit's first
    const int tb = (int)min((int64_t)nt, pos + (end - cur));
    const int h = hq / a.n_qgroups;
    const int qg = hq % a.n_qgroups;
    const int u = hq * a.num_seqs + s;
    const bool whole = pos == 0 && tb == nt && skip == 0;

    if (pos == 0 && lane == 0) {
      int w0, w1;
      waves_of_range(cur, cur + nt, total, span_waves, w0, w1);
      a.unit_info[2 * u] = w0 + u;
      a.unit_info[2 * u + 1] = w1 - w0 + 1;
    }
    const Rows<NG> rw = rows_of<NG, CAUSAL>(a, lane, s, h, qg, ctx);

    // The next unit with work in this wave's range: the following
    // sequence, or the next (head, group); past the last, the prefix
    // units (after_last). The decode finds it and issues its preload now;
    // the verification pass, whose registers are spoken for, after this
    // segment.
    const int64_t cur_next = cur + (tb - pos);
    const bool more = cur_next < end;
    bool after_last = false;
    int hq2 = hq, s2 = s, ctx2 = ctx;
    auto find_next = [&]() {
      if (!more) return;
      do {
        if (++s2 == a.num_seqs) {
          s2 = 0;
          if (++hq2 >= n_hq) {
            after_last = true;
            break;
          }
        }
        ctx2 = scan_ctx<KEEP>(a, ts, s2);
      } while (unit_tiles<PREFIX>(a, s2, ctx2) == 0);
    };
    if (!CAUSAL) find_next();
    SegPre<D, NG> pre2;
    if (!CAUSAL && more && !after_last) {
      const int skip2 = PREFIX ? prefix_skip(a, s2, ctx2) : 0;
      const int tb2 = (int)min((int64_t)unit_tiles<PREFIX>(a, s2, ctx2), end - cur_next);
      segment_preload<D, NG, NBUF>(
          a, lane, s2,
          rows_of<NG, CAUSAL>(a, lane, s2, hq2 / a.n_qgroups, hq2 % a.n_qgroups, ctx2), skip2,
          skip2 + tb2, pre2);
    }

    if constexpr (VG > 0) {
      float vacc[VG][VM];
      float vm[VG], vl[VG];
      const bool ok =
          scan_shares_first<KEEP>(a, ts, s)
              ? process_segment_valu<D, false, NBUF, VG>(a, lane, s, h, ctx, pos, tb, qg == 0,
                                                         pre, vacc, vm, vl)
              : process_segment_valu<D, true, NBUF, VG>(a, lane, s, h, ctx, pos, tb, qg == 0,
                                                        pre, vacc, vm, vl);
      finish_rows_valu<D, VG>(a, lane, ok, whole, (int64_t)w + u, s, h, vacc, vm, vl);
    } else {
      f32x4_t acc[NG][VM];
      float m_run[NG], l_run[NG];
      // a member reading the shared prefix through the prefix units reads
      // its own tiles once: streamed
      const bool ok =
          skip == 0 && scan_shares_first<KEEP>(a, ts, s)
              ? process_segment<D, false, NG, CAUSAL, NBUF>(a, lane, s, h, rw, ctx, skip + pos,
                                                            skip + tb, qg == 0, pre, acc, m_run,
                                                            l_run)
              : process_segment<D, true, NG, CAUSAL, NBUF>(a, lane, s, h, rw, ctx, skip + pos,
                                                           skip + tb, qg == 0, pre, acc, m_run,
                                                           l_run);
      finish_rows<D, NG>(a, lane, ok, whole, (int64_t)w + u, rw, acc, m_run, l_run);
    }
    cur = cur_next;
    if (!more) break;
    if (CAUSAL) find_next();
    if (after_last) {
      if (PREFIX && w_pre == 0 && a.pre_units > 0) prefix_walk(pre_origin);
      return;
    }
    hq = hq2;
    s = s2;
    ctx = ctx2;
    pos = 0;
    if (CAUSAL) {
      const int skip2 = PREFIX ? prefix_skip(a, s, ctx) : 0;
      const int tb2 = (int)min((int64_t)unit_tiles<PREFIX>(a, s, ctx), end - cur);
      segment_preload<D, NG, NBUF, false>(
          a, lane, s, rows_of<NG, CAUSAL>(a, lane, s, hq / a.n_qgroups, hq % a.n_qgroups, ctx),
          skip2, skip2 + tb2, pre);
    } else {
      pre = pre2;
    }
  }
}

// The decode step's kernel: one query row per head, the append fused in.
// PREFIX: the split also holds a shared prefix's units (compiled apart, so
// the plain decode keeps its registers).
template <int D, bool PREFIX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2))) void paged_attn_balanced_kernel(DecodeArgs a) {
  balanced_body<D, 1, false, D == 128 ? kDecodeRing128 : kRing, PREFIX>(a);
}

// The decode's partition kernel with its scores and P.V on the vector ALUs
// (process_segment_valu), for comparison with the matrix-core kernel above:
// the same split, waves, ring and partials; VG rows per KV head. Two waves
// per SIMD at head_dim 128 (with two register sets) measured slower at one
// and two rows and spilled at four; at head_dim 64 with eight rows a few
// values spill.
template <int D, int VG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2))) void paged_attn_balanced_valu_kernel(DecodeArgs a) {
  balanced_body<D, 1, false, D == 128 ? kDecodeRing128 : kRing, false, VG>(a);
}

// The verification pass: q_len query tokens per sequence, causal among
// them, NG groups of 16 rows per wave. Held to two waves per SIMD's
// registers even with two groups (a couple of spilled values at head_dim
// 128): measured faster than one wave with no spills, as the compiler then
// schedules the loads of the next tile further ahead. PREFIX: the split
// also holds a shared prefix's units (pkv_paged_attn_verify_prefix; a
// prefix row is a member's (query token, head) pair); at head_dim 128 that
// instance needs more registers than two waves per SIMD hold, and runs one.
template <int D, int NG, bool PREFIX = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PREFIX && D == 128 ? 1 : 2))) void paged_attn_verify_kernel(DecodeArgs a) {
  balanced_body<D, NG, true, kRing, PREFIX>(a);
}

// Chunked prefill with the K/V tiles staged in LDS. A workgroup of
// kPfWaves waves takes 32 * kPfWaves query rows of one (sequence, KV head)
// (rows ordered (chunk token, head within the group), as everywhere); each
// wave serves 32 of them with 32x32x16 MFMAs (lane i: row i % 32; the two
// halves of the wave split every MFMA's inner dimension and every output
// column). The workgroup walks the cached context in tiles of kPfTile
// tokens (kPfTile / 16 blocks): all its threads load the next tile's K and
// V from the pool into registers while the waves compute the current tile
// from LDS, then store them into the other LDS buffer. LDS holds the tiles
// in MFMA operand order: for each (32-token group, 16-dim step) of K and
// each (block, 32-dim group) of V the 64 lanes' operands one after
// another, so every wave's LDS read is lane-linear and free of bank
// conflicts. The V slots of the sequence's last block past the context are
// zeroed there, once per workgroup. Per tile and wave: for each 32-token
// group, scores (K as A, q as B) accumulated over the head dimension; one
// running-max decision per tile (each row's 32 scores of a group sit in
// two lanes, 16 each); P split into bf16 hi + lo. A P.V MFMA's 16-long
// inner dimension is 8 tokens of one block per half-wave (4 and 4, 8
// apart) with the hi parts, and a second MFMA on the same V operand takes
// the lo parts: the V operand is 8 distinct values read straight from LDS.
// The 32x32x16 shape keeps the matrix pipe fed with few independent
// accumulators, where the 16x16x32 one needs many. Causal: rows see
// positions up to ctx - q_len + their token; tiles past the workgroup's
// last row are not loaded, and the masking runs only in the tiles that
// reach its first row's limit.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kPfWaves = 8;                      // waves per workgroup
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRows = 32 * kPfWaves;           // query rows per workgroup
constexpr int kPfTile = 64;                      // tokens per LDS tile
constexpr int kPfSub = kPfTile / 16;             // blocks per tile
constexpr int kPfGroups = kPfTile / 32;          // 32-token score groups per tile

template <int D>
struct PfSmem {
  // K slot (group, step): lane i's 16 bytes of the score MFMA's A operand,
  // token 32 * group + i % 32 of the tile, dims 16 * step + 8 * (i / 32) ..
  // + 7. V slot (block, dim group): lane i's 16 bytes of the P.V MFMA's A
  // operand, dim 32 * group + i % 32, tokens 4 * (i / 32) .. + 3 and then
  // 8 + 4 * (i / 32) .. + 3 of the block.
  uint16_t k[2][kPfGroups * (D / 16)][64][8];
  uint16_t v[2][kPfSub * (D / 32)][64][8];
};

template <int D>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2)))
void paged_prefill_lds_kernel(DecodeArgs a) {
  constexpr int KS = D / 16;                      // score MFMA steps
  constexpr int DG = D / 32;                      // P.V dim groups
  constexpr int K_SLOTS = kPfGroups * KS;
  constexpr int V_SLOTS = kPfSub * DG;
  constexpr int K_PER = K_SLOTS * 64 / kPfThreads;
  constexpr int V_PER = V_SLOTS * 64 / kPfThreads;
  static_assert(K_PER * kPfThreads == K_SLOTS * 64 && V_PER * kPfThreads == V_SLOTS * 64, "tile split");
  __shared__ PfSmem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;                       // half of the wave
  const int n_rt = (a.qrows + kPfRows - 1) / kPfRows;   // row tiles per (sequence, KV head)
  // Workgroup -> (sequence, KV head, row tile). The row tiles of one
  // (sequence, KV head) pair read the same K/V tiles, so they run on one XCD
  // (workgroup b runs on XCD b % kXcds) and share its L2. The pairs, ordered
  // longest context first (ties by sequence index) with a sequence's KV
  // heads adjacent, are dealt to the XCDs in a snake order (0..7, 7..0, ...):
  // every XCD gets a like share of short and long sequences, and starts its
  // longest pairs first. Ranking more sequences than the workgroup has
  // threads falls back to index order.
  const int n_pairs = a.num_seqs * a.n_kv;
  int pair, rt;
  if (n_pairs >= kXcds && (n_pairs % kXcds == 0 || n_pairs >= 4 * kXcds)) {
    const int xcd = blockIdx.x % kXcds;
    const int k_in_xcd = blockIdx.x / kXcds;
    const int deal = k_in_xcd / n_rt;
    pair = deal * kXcds + ((deal & 1) ? kXcds - 1 - xcd : xcd);
    rt = k_in_xcd % n_rt;
  } else {
    // Few pairs, or a count that would leave some XCDs a pair more than
    // others (fewer than 4 deals and not a whole number of them): a pair's
    // row tiles go round the XCDs instead (each XCD then reads the pair's
    // K/V into its own L2), so that every XCD has a like share of work.
    // 9, 12 and 20 pairs: 1-4 % faster than dealt; the dealt order is 2 %
    // faster where the pairs fill whole deals (its L2 reuse).
    pair = blockIdx.x / n_rt;
    rt = blockIdx.x % n_rt;
  }
  if (pair >= n_pairs) return;
  const int h = pair % a.n_kv;
  const int rank = pair / a.n_kv;
  int s = rank;
  if (a.num_seqs > 1 && a.num_seqs <= kPfThreads) {
    // rank by work (tiles to read); the K buffer of the second stage holds
    // the keys until the first tile is stored
    // (padded to a multiple of 4 with INT32_MIN, below every key, and read
    // four at a time)
    int* key = reinterpret_cast<int*>(&sm.k[1][0][0][0]);
    int* found = key + kPfThreads;
    const int n4 = (a.num_seqs + 3) & ~3;
    if (tid < n4)
      key[tid] = tid < a.num_seqs ? seq_tiles(a.context_lens[tid], a.q_len, a.max_ctx) : INT32_MIN;
    __syncthreads();
    if (tid < a.num_seqs) {
      const int mine = key[tid];
      int above = 0;
      for (int j = 0; j < n4; j += 4) {
        const int4 o = *reinterpret_cast<const int4*>(key + j);
        above += (o.x > mine || (o.x == mine && j < tid)) ? 1 : 0;
        above += (o.y > mine || (o.y == mine && j + 1 < tid)) ? 1 : 0;
        above += (o.z > mine || (o.z == mine && j + 2 < tid)) ? 1 : 0;
        above += (o.w > mine || (o.w == mine && j + 3 < tid)) ? 1 : 0;
      }
      if (above == rank) *found = tid;
    }
    __syncthreads();
    s = *found;
  }
  const int ctx = a.context_lens[s];
  const int qg = rt * kPfWaves + wave;              // this wave's 32-row group
  // this lane's query row
  const int gr = qg * 32 + (lane & 31);
  const bool row_valid = gr < a.qrows;
  const int tok = row_valid ? gr / a.group : 0;
  const int64_t row_index =
      row_valid ? ((int64_t)s * a.q_len + tok) * a.n_q + h * a.group + (gr - tok * a.group) : 0;
  const int lim = row_valid ? ctx - a.q_len + tok : 0x7fffffff;
  // this lane's share of its row's output: dims 32 dg + 8 g + 4 hf .. + 3
  auto write_row = [&](const f32x16_t (&v)[DG], float mul) __attribute__((always_inline)) {
    float* o = a.out + row_index * D + 4 * hf;
#pragma unroll
    for (int dg = 0; dg < DG; ++dg)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4_t*)(o + 32 * dg + 8 * g) =
            f32x4_t{v[dg][4 * g], v[dg][4 * g + 1], v[dg][4 * g + 2], v[dg][4 * g + 3]} * mul;
  };

  if (seq_tiles(ctx, a.q_len, a.max_ctx) == 0) {
    if (h == 0 && rt == 0 && tid == 0) flag_error(a.err_flag, PKV_DEVERR_CONTEXT);
    if (row_valid) {
      f32x16_t z[DG];
#pragma unroll
      for (int dg = 0; dg < DG; ++dg)
#pragma unroll
        for (int e = 0; e < 16; ++e) z[dg][e] = 1.f;
      write_row(z, __builtin_nanf(""));
    }
    return;
  }

  // the positions the workgroup's rows may see: [0, visible)
  const int row_last = min((rt + 1) * kPfRows, a.qrows) - 1;
  const int visible = ctx - a.q_len + row_last / a.group + 1;
  const int n_blocks = (visible + 15) >> 4;          // blocks of the sequence to read
  const int n_tiles = (n_blocks + kPfSub - 1) / kPfSub;
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks;
  const int64_t tile_elems = 16 * D;
  const int64_t head_off = (int64_t)h * tile_elems;
  const int64_t block_stride = (int64_t)a.n_kv * tile_elems;
  const int last_block = (ctx - 1) >> 4;
  const int last_valid = ctx - last_block * 16;
  // the first position that one of the workgroup's rows may not see (its
  // first row's limit + 1; every later row sees more)
  const int first_masked = ctx - a.q_len + 1 + (rt * kPfRows) / a.group;

  // this lane's q row, as the B operand of the score MFMA (dims
  // 16 step + 8 hf .. + 7). The scale is applied inside the exponent (one
  // fused multiply-add per score), which needs a positive factor: for a
  // negative scale the rows are negated (exact in bf16; the products and
  // their sum change sign only), and for a zero scale they are zeroed,
  // which gives every visible score 0.
  const float sl = a.scale_log2 == 0.f ? 1.f : fabsf(a.scale_log2);
  const uint32_t q_xor = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  const bool q_keep = row_valid && a.scale_log2 != 0.f;
  bf16x8_t qv[KS];
  {
    const uint16_t* q_row = a.q + row_index * D + 8 * hf;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      u32x4_t v = *(const u32x4_t*)(q_row + 16 * st);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = q_keep ? (v[e] ^ q_xor) : 0u;
      qv[st] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // global -> registers for tile t. The tile's block ids are the same for
  // the whole workgroup: loaded together first, checked, then every data
  // load is issued with no wait in between. Blocks past n_blocks read a
  // valid block and are zeroed (their positions lie past every valid row's
  // limit, but 0 * NaN would not be 0).
  bool bad = false;
  u32x4_t kst[K_PER];
  u32x2_t vst[V_PER][2];
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    int ids[kPfSub];
#pragma unroll
    for (int j = 0; j < kPfSub; ++j) {
      const int b = t * kPfSub + j;
      ids[j] = bt_row[b < n_blocks ? b : 0];
    }
#pragma unroll
    for (int j = 0; j < kPfSub; ++j) {
      const bool in = t * kPfSub + j < n_blocks;
      bad |= in && (ids[j] < 0 || ids[j] >= a.num_blocks);
      ids[j] = (in && ids[j] >= 0 && ids[j] < a.num_blocks) ? ids[j] : 0;
    }
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      // slot (group, step), lane': token 32 group + c (c = lane' % 32: block
      // 2 group + c / 16, row c % 16), dims 16 step + 8 (lane' / 32) .. + 7
      const int ch = tid + i * kPfThreads;
      const int slot = ch / 64;
      const int ln = ch % 64;
      const int grp = slot / KS;
      const int st = slot % KS;
      const int jb = 2 * grp + ((ln >> 4) & 1);
      int blk = ids[0];
#pragma unroll
      for (int j = 1; j < kPfSub; ++j) blk = jb == j ? ids[j] : blk;
      kst[i] = *(const u32x4_t*)(a.k_pool + blk * block_stride + head_off + (ln & 15) * D + 16 * st +
                                 8 * (ln >> 5));
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      // slot (block, dim group), lane': dim 32 group + lane' % 32, tokens
      // 4 (lane' / 32) .. + 3 and 8 + 4 (lane' / 32) .. + 3
      const int ch = tid + i * kPfThreads;
      const int slot = ch / 64;
      const int ln = ch % 64;
      const int jb = slot / DG;
      const int dg = slot % DG;
      int blk = ids[0];
#pragma unroll
      for (int j = 1; j < kPfSub; ++j) blk = jb == j ? ids[j] : blk;
      const uint16_t* row = a.v_pool + blk * block_stride + head_off + (32 * dg + (ln & 31)) * 16 + 4 * (ln >> 5);
      vst[i][0] = *(const u32x2_t*)row;
      vst[i][1] = *(const u32x2_t*)(row + 8);
    }
  };
  // registers -> LDS for tile t (the zeroing of blocks past n_blocks is
  // done here, after the tile's compute, so the loads stay in flight)
  auto store_tile = [&](int buf, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int ch = tid + i * kPfThreads;
      const int slot = ch / 64;
      const int ln = ch % 64;
      const bool in = t * kPfSub + 2 * (slot / KS) + ((ln >> 4) & 1) < n_blocks;
      *(u32x4_t*)&sm.k[buf][slot][ln][0] = in ? kst[i] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int ch = tid + i * kPfThreads;
      const int slot = ch / 64;
      const int ln = ch % 64;
      const int b = t * kPfSub + slot / DG;
      u32x2_t val[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        val[half] = b < n_blocks ? vst[i][half] : u32x2_t{0u, 0u};
        if (b == last_block && last_valid < 16) {   // slots past the context: zero (0 * NaN)
          const int first = 8 * half + 4 * (ln >> 5);
          val[half][0] &= (first < last_valid ? 0xFFFFu : 0u) | (first + 1 < last_valid ? 0xFFFF0000u : 0u);
          val[half][1] &= (first + 2 < last_valid ? 0xFFFFu : 0u) | (first + 3 < last_valid ? 0xFFFF0000u : 0u);
        }
      }
      *(u32x4_t*)&sm.v[buf][slot][ln][0] = u32x4_t{val[0][0], val[0][1], val[1][0], val[1][1]};
    }
  };

  f32x16_t acc[DG];
#pragma unroll
  for (int dg = 0; dg < DG; ++dg)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dg][e] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;   // l_run: this half-wave's tokens

  // -1 in the low (high) bf16 of a pair: a packed dot product with it
  // subtracts that half, widened exactly, from a float. The empty asm
  // statements keep the two words in registers as the bits written here
  // (no immediate operand whose meaning for a bf16 pair the encoding fixes)
  uint32_t neg_lo_bits = 0x0000BF80u, neg_hi_bits = 0xBF800000u;
  asm volatile("" : "+v"(neg_lo_bits));
  asm volatile("" : "+v"(neg_hi_bits));
  const bf16x2_t neg_lo = __builtin_bit_cast(bf16x2_t, neg_lo_bits);
  const bf16x2_t neg_hi = __builtin_bit_cast(bf16x2_t, neg_hi_bits);

  load_tile(0);
  store_tile(0, 0);
  __syncthreads();
  // A wave whose 32 rows all lie past the chunk's (a short chunk leaves
  // most of the workgroup's rows empty) only stages tiles and keeps the
  // barriers; it computes nothing.
  const bool computes = qg * 32 < a.qrows;
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    if (computes) {
      // Raw scores (q.k, the scale not yet applied) of the tile's 32-token
      // groups: lane i, register 4 g + e holds token 32 group + 8 g + 4 hf
      // + e of row i % 32. The two groups' chains are interleaved. Blocks
      // past those loaded hold zeros and lie past every valid row's limit;
      // positions past a row's limit or the context are masked (-inf) only
      // in the tiles that reach one of the workgroup's limits.
      f32x16_t x[kPfGroups];
#pragma unroll
      for (int grp = 0; grp < kPfGroups; ++grp)
#pragma unroll
        for (int e = 0; e < 16; ++e) x[grp][e] = 0.f;
#pragma unroll
      for (int st = 0; st < KS; ++st)
#pragma unroll
        for (int grp = 0; grp < kPfGroups; ++grp) {
          const bf16x8_t kr = *(const bf16x8_t*)&sm.k[buf][grp * KS + st][lane][0];
          x[grp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr, qv[st], x[grp], 0, 0, 0);
        }
      if ((t + 1) * kPfTile > first_masked) {
#pragma unroll
        for (int grp = 0; grp < kPfGroups; ++grp)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int p0 = t * kPfTile + 32 * grp + 8 * g + 4 * hf;   // this lane's first position
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (p0 + e >= ctx || p0 + e > lim) x[grp][4 * g + e] = -__builtin_inff();
          }
      }
      // running max per row (scaled, base 2), one decision per tile; P =
      // 2^(x * scale - m) split into bf16 hi + lo (hi rounded to nearest,
      // lo = P - hi rounded again: ~16 bits of P). The maximum is NaN-
      // propagating (a NaN score makes the row NaN, as the oracle's
      // would); the row's other half is in the lane 32 away, swapped in
      // with the gfx950 row swap.
      float raw = x[0][0];
#pragma unroll
      for (int grp = 0; grp < kPfGroups; ++grp)
#pragma unroll
        for (int e = (grp == 0 ? 1 : 0); e < 16; ++e) raw = __builtin_elementwise_maximum(raw, x[grp][e]);
      {
        const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(raw), __float_as_uint(raw), false, false);
        raw = __builtin_elementwise_maximum(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
      }
      const float mx = raw == -__builtin_inff() ? raw : raw * sl;
      if (__ballot(mx > m_run + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_run, mx);
        float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        if (m_new == -__builtin_inff()) alpha = 1.f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dg = 0; dg < DG; ++dg) acc[dg] *= alpha;
      }
      const float neg_m = m_run == -__builtin_inff() ? 0.f : -m_run;
      // P operands, per (group, block): the lane's tokens 4 hf .. + 3 (g =
      // 2 block) then 8 + 4 hf .. + 3 (g = 2 block + 1) of the block
      u32x4_t p_hi[kPfGroups][2], p_lo[kPfGroups][2];
#pragma unroll
      for (int grp = 0; grp < kPfGroups; ++grp)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[grp][4 * g], sl, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[grp][4 * g + 1], sl, neg_m));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[grp][4 * g + 2], sl, neg_m));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[grp][4 * g + 3], sl, neg_m));
          l_run += (p0 + p1) + (p2 + p3);
          const bf16x2_t h01 = __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t);
          const bf16x2_t h23 = __builtin_convertvector((f32x2_t){p2, p3}, bf16x2_t);
          const bf16x2_t l01 = __builtin_convertvector(
              (f32x2_t){__builtin_amdgcn_fdot2_f32_bf16(h01, neg_lo, p0, false),
                        __builtin_amdgcn_fdot2_f32_bf16(h01, neg_hi, p1, false)}, bf16x2_t);
          const bf16x2_t l23 = __builtin_convertvector(
              (f32x2_t){__builtin_amdgcn_fdot2_f32_bf16(h23, neg_lo, p2, false),
                        __builtin_amdgcn_fdot2_f32_bf16(h23, neg_hi, p3, false)}, bf16x2_t);
          const int half = 2 * (g & 1);
          p_hi[grp][g / 2][half] = __builtin_bit_cast(uint32_t, h01);
          p_hi[grp][g / 2][half + 1] = __builtin_bit_cast(uint32_t, h23);
          p_lo[grp][g / 2][half] = __builtin_bit_cast(uint32_t, l01);
          p_lo[grp][g / 2][half + 1] = __builtin_bit_cast(uint32_t, l23);
        }
      // P.V per block: one LDS read per dim group gives the lane's V
      // operand (the V slots past the context were zeroed when stored),
      // used by the hi and the lo MFMA; the dim groups' chains interleave
#pragma unroll
      for (int grp = 0; grp < kPfGroups; ++grp)
#pragma unroll
        for (int bl = 0; bl < 2; ++bl) {
          bf16x8_t vv[DG];
#pragma unroll
          for (int dg = 0; dg < DG; ++dg)
            vv[dg] = *(const bf16x8_t*)&sm.v[buf][(2 * grp + bl) * DG + dg][lane][0];
#pragma unroll
          for (int dg = 0; dg < DG; ++dg)
            acc[dg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[dg], __builtin_bit_cast(bf16x8_t, p_hi[grp][bl]),
                                                              acc[dg], 0, 0, 0);
#pragma unroll
          for (int dg = 0; dg < DG; ++dg)
            acc[dg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[dg], __builtin_bit_cast(bf16x8_t, p_lo[grp][bl]),
                                                              acc[dg], 0, 0, 0);
        }
    }
    if (t + 1 < n_tiles) {
      // the other buffer was last read in the previous tile, before the
      // barrier that ended it
      store_tile(buf ^ 1, t + 1);
      __syncthreads();
    }
  }
  // out = acc / l, l summed over the row's two halves; a bad block id
  // makes the rows NaN and sets the error bit
  const bool ok = !bad;
  if (!ok && lane == 0) flag_error(a.err_flag, PKV_DEVERR_BLOCK_ID);
  float l_tot;
  {
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_tot = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  }
  if (row_valid) write_row(acc, ok ? 1.0f / l_tot : __builtin_nanf(""));
}

// Merge kernel: one wave per (unit, query row). With reference maxima m_p,
// sums l_p and accumulators a_p of the row's partials (all relative to
// 2^(x - m_p)): M = max_p m_p, L = sum_p l_p 2^(m_p - M) and
// out = (sum_p 2^(m_p - M) a_p) / L, summed in partial order. The partials
// are the unit's slots, then (a member that reads the shared prefix) the
// slots of the prefix unit holding the row. Lane p holds
// partial p's weight; lane i owns dims PER*i .. PER*i + PER - 1; the
// accumulators are loaded eight partials at a time. A NaN maximum (a bad
// block id) makes the row NaN; a sequence with an invalid context length
// gets NaN rows and the error bit. Units one wave covered were written by
// the partition kernel and are skipped. A partial whose row saw nothing
// (maximum -inf, sum 0) has weight 0.
template <int D>
__global__ __launch_bounds__(256) void paged_attn_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;
  constexpr int PRE = 8;   // partials whose accumulators are loaded together
  const int lane = threadIdx.x & 63;
  const int row_id = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row_id >= a.n_units * a.rows) return;
  const int u = row_id / a.rows;
  const int g_in_slot = row_id % a.rows;
  const int s = u % a.num_seqs;
  const int hq = u / a.num_seqs;
  const int qg = hq % a.n_qgroups;
  const int gr = qg * a.group_rows + g_in_slot;
  if (gr >= a.qrows) return;
  const int i = gr / a.group;
  const int h = hq / a.n_qgroups;
  const int64_t out_row = ((int64_t)s * a.q_len + i) * a.n_q + h * a.group + (gr - i * a.group);
  float* o = a.out + out_row * D + lane * PER;
  const float nan = __builtin_nanf("");

  // The context length and (balanced split) the unit's partial range are
  // independent loads, issued together. The range is only used once the
  // context is known to be valid: for an invalid one the partition kernel
  // wrote nothing for the unit.
  const int ctx = a.context_lens[s];
  int2 info = make_int2(0, 0);
  if (a.part_tokens == 0) info = *(const int2*)(a.unit_info + 2 * u);
  const int nt = seq_tiles(ctx, a.q_len, a.max_ctx);
  if (nt == 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = nan;
    if (hq == 0 && gr == 0 && lane == 0) flag_error(a.err_flag, PKV_DEVERR_CONTEXT);
    return;
  }
  int64_t first;
  int n;
  if (a.part_tokens > 0) {
    const int tiles_per_part = a.part_tokens >> 4;
    n = (nt + tiles_per_part - 1) / tiles_per_part;
    first = (int64_t)u * a.p_max;
  } else {
    first = info.x;
    n = info.y;
  }
  // the prefix unit's partials of this row (decode rows: i = 0, head gr)
  int np = 0;
  int64_t pre_row = 0;
  const bool member = prefix_skip(a, s, ctx) > 0;
  if (member) {
    const int pr = (s - a.pre_first) * a.qrows + gr;
    const int2 pinfo = *(const int2*)(a.pre_info + 2 * (h * a.pre_qgroups + pr / kPrefixRows));
    np = pinfo.y;
    pre_row = (int64_t)pinfo.x * kPrefixRows + (pr % kPrefixRows);
  }
  const int tot = n + np;
  if (tot <= 1) return;   // written directly by the partition kernel

  // partial p: the unit's slot first + p, then prefix part p - n
  auto ml_of = [&](int pp) -> const float* {
    return pp < n ? a.ws_ml + ((first + pp) * a.rows + g_in_slot) * 2
                  : a.pre_ml + (pre_row + (int64_t)(pp - n) * kPrefixRows) * 2;
  };
  auto acc_of = [&](int pp) -> const float* {
    return (pp < n ? a.ws_acc + ((first + pp) * a.rows + g_in_slot) * D
                   : a.pre_acc + (pre_row + (int64_t)(pp - n) * kPrefixRows) * D) +
           lane * PER;
  };

  // One round trip for the first partials: lane p's (m, l), and the
  // accumulators of partials 0 .. PRE-1 (indices past tot read partial
  // tot-1 again and get weight 0).
  float v[PRE][PER];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const float* src = acc_of(k < tot ? k : tot - 1);
#pragma unroll
    for (int e = 0; e < PER; ++e) v[k][e] = src[e];
  }
  f32x2_t mine = lane < tot ? *(const f32x2_t*)ml_of(lane) : f32x2_t{-__builtin_inff(), 0.f};
  if (member) {
    // the partition kernel took this sequence's prefix tiles from the
    // prefix's table: its own table must start with the same blocks, else
    // the row is NaN (checked while the partials above are in flight; the
    // prefix partials are the prefix unit's whatever the table holds)
    const int32_t* row = a.block_tables + (int64_t)s * a.max_blocks;
    bool same = true;
    for (int t = lane; t < a.pre_tiles; t += 64) same = same && row[t] == a.pre_table[t];
    if (__ballot(!same) != 0) {
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = nan;
      if (hq == 0 && gr == 0 && lane == 0) flag_error(a.err_flag, PKV_DEVERR_PREFIX);
      return;
    }
  }

  float mx = mine[0];
  bool bad = mine[0] != mine[0];
  for (int pp = lane + 64; pp < tot; pp += 64) {
    const float mp = ml_of(pp)[0];
    bad |= mp != mp;
    mx = fmaxf(mx, mp);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (__ballot(bad) != 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = nan;
    return;
  }
  const float my_w = lane < tot ? __builtin_amdgcn_exp2f(mine[0] - mx) : 0.f;
  float lsum = mine[1] * my_w;
  for (int pp = lane + 64; pp < tot; pp += 64) {
    const float* mlp = ml_of(pp);
    lsum += mlp[1] * __builtin_amdgcn_exp2f(mlp[0] - mx);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);

  float res[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) res[e] = 0.f;
  // partials in runs of 64 (lane k holds the weight of partial base + k),
  // their accumulators PRE at a time
  for (int base = 0; base < tot; base += 64) {
    const float w_l = base == 0 ? my_w
                                : (base + lane < tot ? __builtin_amdgcn_exp2f(ml_of(base + lane)[0] - mx)
                                                     : 0.f);
    const int run = min(64, tot - base);
    for (int k0 = 0; k0 < run; k0 += PRE) {
      if (base + k0 > 0) {
#pragma unroll
        for (int k = 0; k < PRE; ++k) {
          const int pp = base + k0 + k;
          const float* src = acc_of(pp < tot ? pp : tot - 1);
#pragma unroll
          for (int e = 0; e < PER; ++e) v[k][e] = src[e];
        }
      }
#pragma unroll
      for (int k = 0; k < PRE; ++k) {
        const float wg = __shfl(w_l, k0 + k < 64 ? k0 + k : 63) * (k0 + k < run ? 1.f : 0.f);
#pragma unroll
        for (int e = 0; e < PER; ++e) res[e] += wg * v[k][e];
      }
    }
  }
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = res[e] * inv;
}

// ---------------------------------------------------------------------------
// host side

// Shape of one launch: decode (q_len 1, one 16-row group per wave, no mask)
// or the verification pass (q_len query tokens, causal, one or two 16-row
// groups per wave).
struct Geom {
  int num_seqs, n_q, n_kv, q_len, ng;
  bool causal;
  int qrows() const { return q_len * (n_q / n_kv); }
  int group_rows() const { return 16 * ng; }
  int rows() const { return qrows() < group_rows() ? qrows() : group_rows(); }
  int64_t qgroups() const { return (qrows() + group_rows() - 1) / group_rows(); }
  int64_t units() const { return (int64_t)n_kv * qgroups() * num_seqs; }
};

static Geom decode_geom(int num_seqs, int n_q, int n_kv) { return Geom{num_seqs, n_q, n_kv, 1, 1, false}; }

// The verification pass serves up to 32 rows per KV head from each K/V
// tile (two row groups); a decode with more than 16 query heads per KV
// head uses 16-row groups.
static Geom verify_geom(int num_seqs, int q_len, int n_q, int n_kv) {
  const int qrows = q_len * (n_q / n_kv);
  return Geom{num_seqs, n_q, n_kv, q_len, qrows > 16 ? 2 : 1, true};
}

// Chunked prefill: two 16-row groups per wave (32 rows).
static Geom prefill_geom(int num_seqs, int chunk_len, int n_q, int n_kv) {
  return Geom{num_seqs, n_q, n_kv, chunk_len, 2, true};
}

// Upper bound of the balanced split's wave count: at most kMaxSplitWaves,
// and no more than leaves kMinTilesPerWave tiles of the upper bound of the
// tile count per wave. The launch uses min(this, resident_waves()).
static int64_t split_wave_cap(const Geom& g, int max_ctx) {
  const int64_t tiles_ub = g.units() * ((max_ctx + 15) / 16);
  int64_t w = (tiles_ub + kMinTilesPerWave - 1) / kMinTilesPerWave;
  if (w > kMaxSplitWaves) w = kMaxSplitWaves;
  return w < 1 ? 1 : w;
}

template <typename K>
static int occupancy_blocks(K kernel) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 256, 0) != hipSuccess) return -1;
  return blocks;
}

static int kernel_blocks_per_cu(const Geom& g, int head_dim, bool prefix) {
  if (!g.causal)
    // both instantiations hold the same waves per SIMD (one at head_dim
    // 128, two at 64)
    return head_dim == 128 ? occupancy_blocks(paged_attn_balanced_kernel<128, false>)
                           : occupancy_blocks(paged_attn_balanced_kernel<64, false>);
  if (prefix) {
    if (g.ng == 1)
      return head_dim == 128 ? occupancy_blocks(paged_attn_verify_kernel<128, 1, true>)
                             : occupancy_blocks(paged_attn_verify_kernel<64, 1, true>);
    return head_dim == 128 ? occupancy_blocks(paged_attn_verify_kernel<128, 2, true>)
                           : occupancy_blocks(paged_attn_verify_kernel<64, 2, true>);
  }
  if (g.ng == 1)
    return head_dim == 128 ? occupancy_blocks(paged_attn_verify_kernel<128, 1>)
                           : occupancy_blocks(paged_attn_verify_kernel<64, 1>);
  return head_dim == 128 ? occupancy_blocks(paged_attn_verify_kernel<128, 2>)
                         : occupancy_blocks(paged_attn_verify_kernel<64, 2>);
}

// prefix: the verification pass's instance with a shared prefix's units.
static int resident_waves(const Geom& g, int head_dim, bool prefix = false) {
  // [kernel: decode, verify 1 group, verify 2, the same with a prefix][head_dim == 128][device]
  static int cache[5][2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  const bool pre = prefix && g.causal;
  const int kind = !g.causal ? 0 : (g.ng == 1 ? (pre ? 3 : 1) : (pre ? 4 : 2));
  int& slot = cache[kind][head_dim == 128][dev];
  if (slot > 0) return slot;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  const int blocks = kernel_blocks_per_cu(g, head_dim, pre);
  if (blocks < 1 || cus < 1) return -1;
  // the decode's split uses one wave per SIMD (4 per compute unit) for
  // head_dim 128 and two for head_dim 64, whose tiles are half the bytes:
  // enough loads in flight, few per-wave start-up costs, and every wave
  // resident. The verification pass does q_len times the decode's matrix
  // and softmax work per tile: two waves per SIMD, so one computes while
  // the other's loads are in flight.
  const int want = (head_dim == 128 && !g.causal) ? 4 : 8;
  const int per_cu = blocks * kWaves < want ? blocks * kWaves : want;
  slot = cus * per_cu;
  return slot;
}

// Workspace of the balanced split: per unit its first partial slot and
// partial count (2 x int32, rounded up to 256 bytes), then the partial
// slots. Fixed partitions: the partial slots only.
static size_t unit_info_bytes(const Geom& g) {
  return (size_t)((g.units() * 8 + 255) / 256 * 256);
}

static int64_t slot_count(const Geom& g, int max_ctx, int part) {
  if (part > 0) {
    const int p_max = (max_ctx + part - 1) / part;
    return p_max <= 1 ? 0 : g.units() * p_max;
  }
  return split_wave_cap(g, max_ctx) + g.units();
}

static size_t workspace_bytes(const Geom& g, int d, int max_ctx, int part) {
  const size_t slots_bytes =
      (size_t)slot_count(g, max_ctx, part) * g.rows() * (2 + d) * sizeof(float);
  return (part > 0 ? 0 : unit_info_bytes(g)) + slots_bytes;
}

// Shared prefix: 16-row groups of member rows per KV head, and the bytes
// after the decode's workspace (rounded up to 256 bytes): each prefix
// unit's first slot and count, then its partial slots, 16 rows each. A
// prefix unit's slot is wave + unit, as for the decode's units, so there
// are at most (waves + units) slots.
static int prefix_qgroups(int rows_per_member, int count) {
  return (int)(((int64_t)count * rows_per_member + kPrefixRows - 1) / kPrefixRows);
}

static size_t prefix_bytes(const Geom& g, int d, int max_ctx, int count) {
  const int64_t units = (int64_t)g.n_kv * prefix_qgroups(g.qrows(), count);
  const int64_t slots = split_wave_cap(g, max_ctx) + units;
  return (size_t)((units * 8 + 255) / 256 * 256) +
         (size_t)slots * kPrefixRows * (2 + d) * sizeof(float);
}

}  // namespace pkv

using namespace pkv;

static bool valid_partition_arg(int32_t p) { return p >= 0 && p % 16 == 0 && p <= 1024; }

static bool valid_heads(int32_t num_seqs, int32_t n_q, int32_t n_kv, int32_t d, int32_t max_ctx) {
  return num_seqs > 0 && n_q > 0 && n_kv > 0 && d > 0 && max_ctx > 0 && n_q % n_kv == 0;
}

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t n_q_heads,
                                             int32_t n_kv_heads, int32_t head_dim,
                                             int32_t max_context_len,
                                             int32_t partition_tokens) {
  if (!valid_heads(num_seqs, n_q_heads, n_kv_heads, head_dim, max_context_len)) return 0;
  if (!valid_partition_arg(partition_tokens)) return 0;
  return workspace_bytes(decode_geom(num_seqs, n_q_heads, n_kv_heads), head_dim, max_context_len,
                         partition_tokens);
}

extern "C" size_t pkv_verify_workspace_bytes(int32_t num_seqs, int32_t q_len, int32_t n_q_heads,
                                             int32_t n_kv_heads, int32_t head_dim,
                                             int32_t max_context_len) {
  if (!valid_heads(num_seqs, n_q_heads, n_kv_heads, head_dim, max_context_len)) return 0;
  if (q_len < 1 || q_len > kMaxQueryTokens) return 0;
  if (q_len == 1)
    return workspace_bytes(decode_geom(num_seqs, n_q_heads, n_kv_heads), head_dim,
                           max_context_len, 0);
  return workspace_bytes(verify_geom(num_seqs, q_len, n_q_heads, n_kv_heads), head_dim,
                         max_context_len, 0);
}

extern "C" int32_t pkv_decode_split_waves(int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t head_dim, int32_t max_context_len) {
  if (!valid_heads(num_seqs, n_q_heads, n_kv_heads, 1, max_context_len)) return PKV_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  const Geom g = decode_geom(num_seqs, n_q_heads, n_kv_heads);
  const int res = resident_waves(g, head_dim);
  if (res < 1) return PKV_EHIP;
  const int64_t cap = split_wave_cap(g, max_context_len);
  return (int32_t)(res < cap ? res : cap);
}

// Host-side checks and launch geometry shared by the entry points.
static int prepare(DecodeArgs& a, int& head_dim_out, const Geom& g, float* out, const void* q,
                   const void* k_pool, const void* v_pool, const int32_t* block_tables,
                   const int32_t* context_lens, int32_t max_blocks_per_seq, int32_t num_blocks,
                   int32_t head_dim, float scale, int32_t max_context_len,
                   int32_t partition_tokens, void* workspace, size_t workspace_bytes_given,
                   int32_t* err_flag, bool split = true, bool prefix_units = false) {
  const int32_t num_seqs = g.num_seqs;
  if (num_seqs < 0 || max_blocks_per_seq < 1 || num_blocks < 1 || g.n_q < 1 || g.n_kv < 1 ||
      max_context_len < 1)
    return PKV_EINVAL;
  if (g.n_q % g.n_kv != 0) return PKV_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if ((int64_t)max_context_len > 16 * (int64_t)max_blocks_per_seq) return PKV_EINVAL;
  if (!valid_partition_arg(partition_tokens)) return PKV_EINVAL;
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
  a.n_q = g.n_q;
  a.n_kv = g.n_kv;
  a.group = g.n_q / g.n_kv;
  a.q_len = g.q_len;
  a.qrows = g.qrows();
  a.group_rows = g.group_rows();
  a.n_qgroups = (int)g.qgroups();
  a.rows = g.rows();
  a.max_ctx = max_context_len;
  a.part_tokens = partition_tokens;
  a.p_max = partition_tokens > 0 ? (max_context_len + partition_tokens - 1) / partition_tokens : 0;
  a.scale_log2 = scale * kLog2e;
  a.pre_table = nullptr;
  a.pre_first = a.pre_count = a.pre_tiles = 0;
  a.pre_qgroups = a.pre_units = 0;
  a.pre_cost_num = kPrefixCostNum;
  a.pre_cost_den = kPrefixCostDen;
  a.pre_info = nullptr;
  a.pre_ml = a.pre_acc = nullptr;
  head_dim_out = head_dim;

  const int64_t units = g.units();
  if (units > (int64_t)INT32_MAX / 64) return PKV_EINVAL;
  // tiles of one (head, group) row of the split are counted in 32 bits
  if ((int64_t)num_seqs * ((max_context_len + 15) / 16) > (int64_t)INT32_MAX / 2) return PKV_EINVAL;
  a.n_units = (int)units;
  if (num_seqs == 0) return PKV_OK;
  a.k_new = nullptr;
  a.v_new = nullptr;
  if (!split) {   // one wave per unit, no workspace
    a.unit_info = nullptr;
    a.ws_ml = a.ws_acc = nullptr;
    a.n_waves = (int)units;
    const int64_t wgs = (units + kWaves - 1) / kWaves;
    a.wg_per_xcd = (int)((wgs + kXcds - 1) / kXcds);
    return PKV_OK;
  }

  const size_t need = workspace_bytes(g, head_dim, max_context_len, partition_tokens);
  if (need > 0 && (workspace == nullptr || workspace_bytes_given < need)) return PKV_EWORKSPACE;
  const int64_t slots = slot_count(g, max_context_len, partition_tokens);
  const size_t info = partition_tokens > 0 ? 0 : unit_info_bytes(g);
  a.unit_info = partition_tokens > 0 ? nullptr : (int32_t*)workspace;
  a.ws_ml = slots > 0 ? (float*)((char*)workspace + info) : nullptr;
  a.ws_acc = slots > 0 ? a.ws_ml + 2 * slots * a.rows : nullptr;

  int64_t waves;
  if (partition_tokens > 0) {
    waves = units * a.p_max;
    if (waves > (int64_t)INT32_MAX / 2) return PKV_EINVAL;
    a.n_waves = 0;
  } else {
    const int res = resident_waves(g, head_dim, prefix_units);
    if (res < 1) return PKV_EHIP;
    const int64_t cap = split_wave_cap(g, max_context_len);
    waves = res < cap ? res : cap;
    a.n_waves = (int)waves;
  }
  const int64_t wgs = (waves + kWaves - 1) / kWaves;
  a.wg_per_xcd = (int)((wgs + kXcds - 1) / kXcds);
  return PKV_OK;
}

static int launch_partition(const DecodeArgs& a, int head_dim, hipStream_t st) {
  const unsigned grid = (unsigned)a.wg_per_xcd * kXcds;
  if (a.part_tokens > 0) {
    if (head_dim == 128)
      hipLaunchKernelGGL(paged_attn_fixed_kernel<128>, dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(paged_attn_fixed_kernel<64>, dim3(grid), dim3(256), 0, st, a);
  } else if (a.pre_tiles > 0) {   // a shared prefix's units in the split
    if (head_dim == 128)
      hipLaunchKernelGGL((paged_attn_balanced_kernel<128, true>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((paged_attn_balanced_kernel<64, true>), dim3(grid), dim3(256), 0, st, a);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((paged_attn_balanced_kernel<128, false>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((paged_attn_balanced_kernel<64, false>), dim3(grid), dim3(256), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

static int launch_verify(const DecodeArgs& a, int head_dim, hipStream_t st) {
  const unsigned grid = (unsigned)a.wg_per_xcd * kXcds;
  const bool two = a.group_rows == 32;
  if (a.pre_tiles > 0) {   // a shared prefix's units in the split
    if (head_dim == 128) {
      if (two)
        hipLaunchKernelGGL((paged_attn_verify_kernel<128, 2, true>), dim3(grid), dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((paged_attn_verify_kernel<128, 1, true>), dim3(grid), dim3(256), 0, st, a);
    } else {
      if (two)
        hipLaunchKernelGGL((paged_attn_verify_kernel<64, 2, true>), dim3(grid), dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((paged_attn_verify_kernel<64, 1, true>), dim3(grid), dim3(256), 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
  }
  if (head_dim == 128) {
    if (two)
      hipLaunchKernelGGL((paged_attn_verify_kernel<128, 2>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((paged_attn_verify_kernel<128, 1>), dim3(grid), dim3(256), 0, st, a);
  } else {
    if (two)
      hipLaunchKernelGGL((paged_attn_verify_kernel<64, 2>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((paged_attn_verify_kernel<64, 1>), dim3(grid), dim3(256), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

static int launch_merge(const DecodeArgs& a, int head_dim, hipStream_t st) {
  const unsigned mgrid = (unsigned)(((int64_t)a.n_units * a.rows + kWaves - 1) / kWaves);
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
#define PKV_DECODE_PREP_ARGS                                                                  \
  decode_geom(num_seqs, n_q_heads, n_kv_heads), out, q, k_pool, v_pool, block_tables,         \
      context_lens, max_blocks_per_seq, num_blocks, head_dim, scale, max_context_len,        \
      partition_tokens, workspace, workspace_bytes_given, err_flag

extern "C" int pkv_paged_attn_partition(PKV_DECODE_PARAMS) {
  DecodeArgs a;
  int d = 0;
  const int rc = prepare(a, d, PKV_DECODE_PREP_ARGS);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  return launch_partition(a, d, (hipStream_t)stream);
}

extern "C" int pkv_paged_attn_merge(PKV_DECODE_PARAMS) {
  DecodeArgs a;
  int d = 0;
  const int rc = prepare(a, d, PKV_DECODE_PREP_ARGS);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  return launch_merge(a, d, (hipStream_t)stream);
}

// The partition kernel, then the merge kernel.
static int decode_launch(DecodeArgs& a, int d, hipStream_t st) {
  const int rc = launch_partition(a, d, st);
  return rc != PKV_OK ? rc : launch_merge(a, d, st);
}

extern "C" int pkv_paged_attn_decode(PKV_DECODE_PARAMS) {
  DecodeArgs a;
  int d = 0;
  const int rc = prepare(a, d, PKV_DECODE_PREP_ARGS);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  return decode_launch(a, d, (hipStream_t)stream);
}

#define PKV_STEP_PARAMS                                                                      \
  float *out, const void *q, const void *k_new, const void *v_new, void *k_pool, void *v_pool, \
      const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,              \
      int32_t max_blocks_per_seq, int32_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,   \
      int32_t head_dim, float scale, int32_t max_context_len, int32_t partition_tokens,        \
      void *workspace, size_t workspace_bytes_given, int32_t *err_flag, void *stream

// The append and the partition kernel of a decode step: with the balanced
// split one launch (the append inside the partition kernel), with a fixed
// partition size kv_append then the partition kernel.
static int step_partition(DecodeArgs& a, int& d, PKV_STEP_PARAMS) {
  const int rc = prepare(a, d, PKV_DECODE_PREP_ARGS);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  if (!k_new || !v_new) return PKV_EINVAL;
  if (partition_tokens == 0) {
    a.k_new = (const uint16_t*)k_new;
    a.v_new = (const uint16_t*)v_new;
    return launch_partition(a, d, (hipStream_t)stream);
  }
  const int arc = pkv_kv_append(k_pool, v_pool, k_new, v_new, block_tables, context_lens,
                                num_seqs, max_blocks_per_seq, num_blocks, n_kv_heads, head_dim,
                                err_flag, stream);
  return arc != PKV_OK ? arc : launch_partition(a, d, (hipStream_t)stream);
}

#define PKV_STEP_ARGS                                                                         \
  out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, num_seqs,                 \
      max_blocks_per_seq, num_blocks, n_q_heads, n_kv_heads, head_dim, scale, max_context_len, \
      partition_tokens, workspace, workspace_bytes_given, err_flag, stream

extern "C" int pkv_decode_step_partition(PKV_STEP_PARAMS) {
  DecodeArgs a;
  int d = 0;
  return step_partition(a, d, PKV_STEP_ARGS);
}

extern "C" int pkv_decode_step_partition_valu(PKV_STEP_PARAMS) {
  if (partition_tokens != 0) return PKV_EINVAL;
  if (n_kv_heads > 0 && n_q_heads % n_kv_heads == 0 && n_q_heads / n_kv_heads > kVecMaxG)
    return PKV_EUNSUPPORTED;
  DecodeArgs a;
  int d = 0;
  const int rc = prepare(a, d, PKV_DECODE_PREP_ARGS);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  if (!k_new || !v_new) return PKV_EINVAL;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  const int vg = a.group <= 2 ? a.group : (a.group <= 4 ? 4 : (a.group == 5 ? 5 : 8));
  const unsigned grid = (unsigned)a.wg_per_xcd * kXcds;
  const hipStream_t st = (hipStream_t)stream;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, st, a); };
  if (d == 128) {
    switch (vg) {
      case 1: go(paged_attn_balanced_valu_kernel<128, 1>); break;
      case 2: go(paged_attn_balanced_valu_kernel<128, 2>); break;
      case 4: go(paged_attn_balanced_valu_kernel<128, 4>); break;
      case 5: go(paged_attn_balanced_valu_kernel<128, 5>); break;
      default: go(paged_attn_balanced_valu_kernel<128, 8>); break;
    }
  } else {
    switch (vg) {
      case 1: go(paged_attn_balanced_valu_kernel<64, 1>); break;
      case 2: go(paged_attn_balanced_valu_kernel<64, 2>); break;
      case 4: go(paged_attn_balanced_valu_kernel<64, 4>); break;
      case 5: go(paged_attn_balanced_valu_kernel<64, 5>); break;
      default: go(paged_attn_balanced_valu_kernel<64, 8>); break;
    }
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

extern "C" int pkv_decode_step(PKV_STEP_PARAMS) {
  DecodeArgs a;
  int d = 0;
  const int rc = step_partition(a, d, PKV_STEP_ARGS);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  return launch_merge(a, d, (hipStream_t)stream);
}

static bool valid_prefix_args(int32_t num_seqs, int32_t max_blocks_per_seq,
                              const int32_t* prefix_table, int32_t prefix_blocks,
                              int32_t prefix_first_seq, int32_t prefix_num_seqs) {
  if (prefix_blocks < 0 || prefix_first_seq < 0 || prefix_num_seqs < 0) return false;
  if ((int64_t)prefix_first_seq + prefix_num_seqs > num_seqs) return false;
  if (prefix_blocks > max_blocks_per_seq) return false;
  if (prefix_blocks > 0 && prefix_num_seqs > 0 && !prefix_table) return false;
  return true;
}

static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// The shared prefix's part of a call (decode or verification pass): the
// prefix units' bookkeeping and partials after the call's own workspace.
static int attach_prefix(DecodeArgs& a, const Geom& g, int head_dim, int max_ctx, void* workspace,
                         size_t workspace_bytes_given, const int32_t* prefix_table,
                         int32_t prefix_blocks, int32_t prefix_first_seq,
                         int32_t prefix_num_seqs) {
  const size_t base = round256(workspace_bytes(g, head_dim, max_ctx, 0));
  if (workspace_bytes_given < base + prefix_bytes(g, head_dim, max_ctx, prefix_num_seqs))
    return PKV_EWORKSPACE;
  a.pre_table = prefix_table;
  a.pre_first = prefix_first_seq;
  a.pre_count = prefix_num_seqs;
  a.pre_tiles = prefix_blocks;
  a.pre_cost_num = g.causal ? kVerifyPrefixCostNum : kPrefixCostNum;
  a.pre_cost_den = g.causal ? kVerifyPrefixCostDen : kPrefixCostDen;
  a.pre_qgroups = prefix_qgroups(g.qrows(), prefix_num_seqs);
  const int64_t units = (int64_t)g.n_kv * a.pre_qgroups;
  // tile indices of the split (sequences' and prefix units') fit 62 bits;
  // the unit and slot counts fit 32
  if (units > (int64_t)INT32_MAX / 64) return PKV_EINVAL;
  a.pre_units = (int)units;
  a.pre_info = (int32_t*)((char*)workspace + base);
  a.pre_ml = (float*)((char*)workspace + base + (units * 8 + 255) / 256 * 256);
  const int64_t slots = split_wave_cap(g, max_ctx) + units;
  a.pre_acc = a.pre_ml + 2 * kPrefixRows * slots;
  return PKV_OK;
}

extern "C" size_t pkv_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t n_q_heads,
                                                    int32_t n_kv_heads, int32_t head_dim,
                                                    int32_t max_context_len, int32_t prefix_blocks,
                                                    int32_t prefix_num_seqs) {
  const size_t base =
      pkv_decode_workspace_bytes(num_seqs, n_q_heads, n_kv_heads, head_dim, max_context_len, 0);
  if (base == 0 || prefix_blocks <= 0 || prefix_num_seqs <= 0) return base;
  return round256(base) + prefix_bytes(decode_geom(num_seqs, n_q_heads, n_kv_heads), head_dim,
                                       max_context_len, prefix_num_seqs);
}

extern "C" int pkv_decode_step_prefix(float* out, const void* q, const void* k_new,
                                      const void* v_new, void* k_pool, void* v_pool,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t max_blocks_per_seq,
                                      int32_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t head_dim, float scale, int32_t max_context_len,
                                      const int32_t* prefix_table, int32_t prefix_blocks,
                                      int32_t prefix_first_seq, int32_t prefix_num_seqs,
                                      void* workspace, size_t workspace_bytes_given,
                                      int32_t* err_flag, void* stream) {
  if (!valid_prefix_args(num_seqs, max_blocks_per_seq, prefix_table, prefix_blocks,
                         prefix_first_seq, prefix_num_seqs))
    return PKV_EINVAL;
  DecodeArgs a;
  int d = 0;
  const int32_t partition_tokens = 0;
  const int rc = prepare(a, d, PKV_DECODE_PREP_ARGS);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  if (!k_new || !v_new) return PKV_EINVAL;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  if (prefix_blocks > 0 && prefix_num_seqs > 0) {
    const int prc = attach_prefix(a, decode_geom(num_seqs, n_q_heads, n_kv_heads), head_dim,
                                  max_context_len, workspace, workspace_bytes_given, prefix_table,
                                  prefix_blocks, prefix_first_seq, prefix_num_seqs);
    if (prc != PKV_OK) return prc;
  }
  const hipStream_t st = (hipStream_t)stream;
  const int prc = launch_partition(a, d, st);
  return prc != PKV_OK ? prc : launch_merge(a, d, st);
}

extern "C" int pkv_paged_attn_verify(float* out, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs, int32_t q_len,
                                     int32_t max_blocks_per_seq, int32_t num_blocks,
                                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                     float scale, int32_t max_context_len, void* workspace,
                                     size_t workspace_bytes_given, int32_t* err_flag,
                                     void* stream) {
  if (q_len < 1 || q_len > kMaxQueryTokens || n_kv_heads < 1) return PKV_EINVAL;
  if (q_len == 1)   // one query token: the decode itself
    return pkv_paged_attn_decode(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs,
                                 max_blocks_per_seq, num_blocks, n_q_heads, n_kv_heads, head_dim,
                                 scale, max_context_len, 0, workspace, workspace_bytes_given,
                                 err_flag, stream);
  DecodeArgs a;
  int d = 0;
  const int rc = prepare(a, d, verify_geom(num_seqs, q_len, n_q_heads, n_kv_heads), out, q,
                         k_pool, v_pool, block_tables, context_lens, max_blocks_per_seq,
                         num_blocks, head_dim, scale, max_context_len, 0, workspace,
                         workspace_bytes_given, err_flag);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  const int vrc = launch_verify(a, d, (hipStream_t)stream);
  return vrc != PKV_OK ? vrc : launch_merge(a, d, (hipStream_t)stream);
}

extern "C" size_t pkv_verify_prefix_workspace_bytes(int32_t num_seqs, int32_t q_len,
                                                    int32_t n_q_heads, int32_t n_kv_heads,
                                                    int32_t head_dim, int32_t max_context_len,
                                                    int32_t prefix_blocks,
                                                    int32_t prefix_num_seqs) {
  if (!valid_heads(num_seqs, n_q_heads, n_kv_heads, head_dim, max_context_len)) return 0;
  if (q_len < 1 || q_len > kMaxQueryTokens) return 0;
  const Geom g = verify_geom(num_seqs, q_len, n_q_heads, n_kv_heads);
  const size_t base = workspace_bytes(g, head_dim, max_context_len, 0);
  if (prefix_blocks <= 0 || prefix_num_seqs <= 0) return base;
  return round256(base) + prefix_bytes(g, head_dim, max_context_len, prefix_num_seqs);
}

extern "C" int pkv_paged_attn_verify_prefix(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs, int32_t q_len,
    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
    int32_t head_dim, float scale, int32_t max_context_len, const int32_t* prefix_table,
    int32_t prefix_blocks, int32_t prefix_first_seq, int32_t prefix_num_seqs, void* workspace,
    size_t workspace_bytes_given, int32_t* err_flag, void* stream) {
  if (q_len < 1 || q_len > kMaxQueryTokens || n_kv_heads < 1) return PKV_EINVAL;
  if (!valid_prefix_args(num_seqs, max_blocks_per_seq, prefix_table, prefix_blocks,
                         prefix_first_seq, prefix_num_seqs))
    return PKV_EINVAL;
  const Geom g = verify_geom(num_seqs, q_len, n_q_heads, n_kv_heads);
  const bool pre = prefix_blocks > 0 && prefix_num_seqs > 0;
  DecodeArgs a;
  int d = 0;
  const int rc = prepare(a, d, g, out, q, k_pool, v_pool, block_tables, context_lens,
                         max_blocks_per_seq, num_blocks, head_dim, scale, max_context_len, 0,
                         workspace, workspace_bytes_given, err_flag, true, pre);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  if (pre) {
    const int prc = attach_prefix(a, g, head_dim, max_context_len, workspace,
                                  workspace_bytes_given, prefix_table, prefix_blocks,
                                  prefix_first_seq, prefix_num_seqs);
    if (prc != PKV_OK) return prc;
  }
  const int vrc = launch_verify(a, d, (hipStream_t)stream);
  return vrc != PKV_OK ? vrc : launch_merge(a, d, (hipStream_t)stream);
}

extern "C" int pkv_paged_prefill(float* out, const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t chunk_len, int32_t max_blocks_per_seq,
                                 int32_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, float scale, int32_t max_context_len,
                                 int32_t* err_flag, void* stream) {
  if (chunk_len < 1 || chunk_len > kMaxChunkTokens || n_kv_heads < 1) return PKV_EINVAL;
  DecodeArgs a;
  int d = 0;
  const int rc = prepare(a, d, prefill_geom(num_seqs, chunk_len, n_q_heads, n_kv_heads), out, q,
                         k_pool, v_pool, block_tables, context_lens, max_blocks_per_seq,
                         num_blocks, head_dim, scale, max_context_len, 0, nullptr, 0, err_flag,
                         false);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  // one workgroup per (sequence, KV head, kPfRows rows); the (sequence, KV
  // head) pairs are dealt to the XCDs, kXcds at a time, each with all its
  // row tiles (the kernel's mapping), so the grid is rounded up to whole deals
  // (pairs not dealt, as the kernel decides: one workgroup per row tile,
  // in order)
  const int64_t pairs = (int64_t)num_seqs * n_kv_heads;
  const int64_t deals = (pairs + kXcds - 1) / kXcds;
  const int64_t n_rt = (a.qrows + kPfRows - 1) / kPfRows;
  const bool dealt = pairs >= kXcds && (pairs % kXcds == 0 || pairs >= 4 * kXcds);
  const int64_t grid64 = dealt ? deals * kXcds * n_rt : pairs * n_rt;
  if (grid64 > INT32_MAX) return PKV_EINVAL;
  const unsigned grid = (unsigned)grid64;
  if (d == 128)
    hipLaunchKernelGGL(paged_prefill_lds_kernel<128>, dim3(grid), dim3(kPfThreads), 0,
                       (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(paged_prefill_lds_kernel<64>, dim3(grid), dim3(kPfThreads), 0,
                       (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}
