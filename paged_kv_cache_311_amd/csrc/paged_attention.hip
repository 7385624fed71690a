// Paged decode attention for gfx950 (MI355X).
//
// One decode step: every sequence's single new query attends to all of
// that sequence's cached tokens, read through its block table from a
// shared pool of 16-token blocks ("Your GPU was mostly empty..." [TEQ],
// "The OS already solved this in the 1960s"; "vLLM and PagedAttention"
// [IV], "Architecture, step by step", step 3).  The arithmetic is scaled
// dot-product attention (Vaswani et al. 2017, eq. 1); paging only changes
// where each token's key and value are fetched from.
//
// Work decomposition (balanced, persistent)
//   tile      = one (block, kv head) pair of one sequence: 16 tokens x
//               head_size contiguous elements of K and the same of V.
//   segment   = all tiles of one (sequence, group of GC query heads that
//               share a kv head); segments are laid end to end in
//               sequence-major order, giving T tiles in total.
//   range     = an equal share of consecutive tiles of that flattened
//               order.  The grid holds two resident waves per SIMD and
//               every wave takes an equal run of consecutive ranges (one,
//               unless a cap on the tokens per piece makes them shorter), so
//               each wave streams the same number of bytes whatever the
//               length mix (no empty or straggling workgroups).  With two waves per
//               SIMD rather than more, the hardware's preference for the
//               oldest wave leaves less of a spread in finishing times.
//   piece     = the part of one segment inside one range.  A wave keeps an
//               online softmax per piece; a piece that is a whole segment
//               writes the output directly, a piece of a split segment
//               writes float32 partials (running max, sum, unnormalized
//               accumulator).  The range holding a split segment's last
//               tile names that segment in a per-range descriptor, and a
//               second, light kernel merges the pieces of every segment a
//               descriptor names (a wave each, or a workgroup when the
//               segment is split many ways).
//
// Per tile (one wave), with one or two heads per group (and every E4M3 or
// float32 pool):
//   QK  = MFMA chain: the key tile is the B operand exactly as loaded (lane
//         l holds token l%16), the query rows are replicated so every lane
//         receives the logits of its own token for all heads of the group.
//   softmax = online, in log2 units; the running max per head is wave
//         uniform (DPP row reduction) and the accumulator is rescaled only
//         when it grows.
//   PV  = VALU FMA in float32 over value tiles loaded as contiguous 1 KiB
//         rows per instruction; probabilities reach the value layout through
//         a 16 x GC LDS buffer owned by the wave.
// With four or eight heads per group and 16-bit pools, both products run on
// the matrix cores instead:
//   S^T = K Q^T  (MFMA 16x16x32): A = the key tile as loaded, B = the query
//         rows, head h of the group on lane column h; lane l receives tokens
//         4(l/16) .. +3 of head l % 16.
//   softmax = online and lane-local: a head's 16 logits sit in lanes l,
//         l^16, l^32, l^48 (row-swap permutes for the max and the sum); the
//         max is raised only when a tile's exceeds it by 2^8.
//   O^T += V^T P^T (MFMA 16x16x32): B = the probabilities as the first
//         product left them, each split into its 16-bit rounding and the
//         remainder (so the product keeps float32 accuracy); A = the value
//         tile, stored as rows in the wave's LDS and read back with the
//         transposing LDS read.  Lane l holds dims 16b + 4(l/16) .. +3 of
//         head l % 16, so rescales and the final 1/sum are lane-local.
//   The next tile's loads are issued before the current tile is computed
//   (E4M3 pools compute while they are in flight; 16-bit pools wait for
//   them first and rely on the SIMD's other wave for the overlap).
//   A tile only this wave reads in the call is loaded with the
//   non-temporal cache policy (a faster stream from HBM); a tile that a
//   neighbouring sequence also maps (shared prompt blocks) keeps the
//   default policy, so its other readers find it in L2.
//
// Appending variant: the same kernel also caches each sequence's newest
// token -- in its last tile the lanes of that row read the new key and
// value rows instead of the pool, and one head group per kv head stores
// them into the slot.
//
// Masking: tokens at or beyond the context length in the last block are
// excluded by select (logit -inf, value zeroed), never by multiplying
// garbage by zero, so NaN-filled free slots cannot leak into the result.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "pkv_device.h"

namespace pkv {

constexpr int kWavesPerWG = 4;
constexpr int kThreads = kWavesPerWG * kWave;
constexpr int kMaxWGs = 1024;                   // at most 4 waves per SIMD
constexpr int kMaxWaves = kMaxWGs * kWavesPerWG;
constexpr int kWavesPerSimd = 2;                // resident waves the grid is sized for
constexpr int kWavesPerSimdFp8 = 3;             // ... with E4M3 pools
constexpr int kMinTilesPerRange = 4;
constexpr int kMaxPartition = 4096;             // tokens per piece, when capped
constexpr int kSoloPieces = 8;                  // merged by one wave up to this many
constexpr int kMergeRounds = 8;                 // merge grid: at most this x the decode grid
// 16-bit queries with at least this many heads per group compute both
// products on the matrix cores: the value product in the float32 VALU
// costs 16 x D FMAs per head and tile, and from four heads up that work,
// not the stream, sets the pace (measured on one MI355X, 64 query / 8 kv
// heads over 16 x 32K bfloat16 tokens: 423 -> 351 us; 32 / 8: 354 -> 351;
// with one head per group the matrix-core path is 4% slower).
constexpr int kPvMfmaMinGc = 4;
constexpr int kPvMfmaMinGcFp8 = 4;              // ... with E4M3 pools
// A head's running max is raised only when a tile's max exceeds it by more
// than this (log2 units), so the accumulator is rescaled rarely;
// probabilities then stay below 2^kPvSlack.
constexpr float kPvSlack = 8.f;
// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt left at their maxima
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitAllLoads = 0x0F70;

// Sequences one launch covers: their segment table lives in LDS.  The
// host splits larger batches into consecutive launches.
constexpr int kLdsSeqs = 2048;
// Batches of at most this many sequences can be laid out sorted (see
// sort_by_first_block).
constexpr int kSortSeqs = 512;

// DT: query / output element; KT: pool element (DT itself, or E4M3 codes
// with 16-bit queries); AP: the call also appends each sequence's newest
// token (its rows come in beside the pools).
template <int DT, int KT, int D, int GC, bool AP = true>
struct DecodeCfg {
  static constexpr bool kFp8 = KT == PKV_FP8_E4M3;
  static_assert(KT == DT || (kFp8 && (DT == PKV_F16 || DT == PKV_BF16)), "pool format");
  static constexpr int kEsz = Elt<KT>::kBytes;       // pool element bytes
  static constexpr int kEszQ = Elt<DT>::kBytes;      // query / output element bytes
  static constexpr int kEpc = Elt<KT>::kPer16B;      // pool elements per 16-B chunk
  static constexpr int kEpcQ = Elt<DT>::kPer16B;     // output elements per 16-B chunk
  static constexpr int kRowB = D * kEsz;             // pool bytes per token row
  static constexpr int kRowQ = D * kEszQ;            // query / output bytes per row
  static constexpr int kNch = kRowB / 16;            // 16-B chunks per pool row
  static constexpr int kTileB = kBlockSize * kRowB;  // bytes per (block, kv head)
  static constexpr int kNld = kTileB / 1024;         // 16-B loads per lane per tile
  static constexpr int kTpl = kWave / kNch;          // tokens per 1-KiB value load
  // MFMA k-steps per chain: one per key chunk, two for E4M3 chunks (16
  // codes widen to two 8-element operands); as many q registers
  static constexpr int kNq = kFp8 ? 2 * kNld : kNld;
  // Both products on the matrix cores: S^T = K Q^T (head h of the group on
  // lane column h) and O^T += V^T P^T with the values read transposed from
  // LDS.  Otherwise QK is Q K^T with replicated query rows and PV runs in
  // the float32 VALU.
  static constexpr bool kPvMfma =
      DT != PKV_F32 && (GC >= (kFp8 ? kPvMfmaMinGcFp8 : kPvMfmaMinGc) || GC == 16);
  static constexpr int kGcq = GC < 4 ? GC : 4;       // heads per MFMA chain
  static constexpr int kNqg = kPvMfma ? 1 : (GC + 3) / 4;  // MFMA chains per tile
  static constexpr int kVS = D * 2 + 32;             // LDS value row stride (matrix-core path)
  static constexpr int kNdb = D / 16;                // 16-dim output blocks (matrix-core path)
  static_assert(GC <= 8 || kPvMfma, "16 heads per group: matrix-core path only");
  static_assert(kNch * 16 == kRowB, "row must be a whole number of 16-B chunks");
  static_assert(kNld * 4 == kNch, "key tile: 4 lane groups x kNld chunks per row");
  static_assert(kNch >= 4 && kNch <= 32, "lane-group reduction assumes 4..32 chunks");
  static_assert(GC == 1 || GC == 2 || GC == 4 || GC == 8 || GC == 16, "heads per group");
  // Waves per SIMD the register allocator must leave room for: 3 (168
  // VGPRs) where the kernel fits without spilling (one head per group with
  // 16-bit K/V or 64-wide rows, two heads with 64-wide rows), 2 (256 VGPRs)
  // for up to four heads per group, otherwise whatever it needs.
  static constexpr bool kNarrow = kEsz <= 2 || D == 64;
  static constexpr int kMinWaves =
      kPvMfma ? (kFp8 ? 3 : 2)
              : (kNarrow && (GC == 1 || (GC == 2 && D == 64)) ? 3 : (kNarrow && GC <= 4 ? 2 : 1));
  // Sixteen heads per group (16-bit pools): one wave per SIMD, with the
  // next tile in flight during the compute (below).  A tile's products and
  // softmax for 16 heads take long enough that a wave which waits for its
  // next tile before computing leaves the stream idle meanwhile, and half
  // the waves make half the split pieces (measured on one MI355X, 32 query
  // / 2 kv heads over 16 x 32K bfloat16 tokens, decode call: 100 us at two
  // waves per SIMD, 106 with the next tile in flight there, 95 at one wave
  // with it, 114 at one wave without it; with 4 or 8 heads per group one
  // wave per SIMD is within 1% of two).
  static constexpr bool kWide = kPvMfma && !kFp8 && GC == 16;
  static constexpr int kGridWaves = kFp8 ? kWavesPerSimdFp8 : (kWide ? 1 : kWavesPerSimd);
  // E4M3 tiles: the next tile's loads stay in flight while the current
  // tile is computed (also 16-bit tiles with sixteen heads per group, see
  // kWide).  Other 16-bit tiles: the wave waits for them as well before
  // computing; their stream is at the HBM ceiling already and more loads
  // in flight only add contention (measured on one MI355X: overlapping is
  // 15% faster on the 32K-token grouped workload with E4M3 pools, 3.7%
  // slower with bfloat16 pools).
  static constexpr bool kOverlapNext = kFp8 || kWide;
  // Appending: new-token rows a wave holds in LDS before writing them
  static constexpr int kNewRecs = !AP ? 0 : kPvMfma ? 4 : 8;
  // E4M3 appending: new-row elements each lane encodes, and their bytes
  static constexpr int kEncPerLane = D / kWave;
  static constexpr int kEncBytes = kEncPerLane * kEszQ;
  static_assert(!kFp8 || kEszQ == 2, "E4M3 pools go with 16-bit queries and new rows");
  // Float32 partials of split pieces are staged in the wave's LDS and
  // written to the workspace when the wave ends (or when its stage is
  // full).  A store counts against the same wait counter as the tile
  // loads, so a partial stored in the middle of a wave's stream holds up
  // its next tile until the store is acknowledged: measured on one MI355X,
  // 16 x 32K bf16 tokens at 512-token partitions (four pieces per wave,
  // every wave at a piece end at the same time), the decode kernel takes
  // 373 us storing them as it goes against 336 us not storing them.  A
  // staged record holds acc [GC][D] then (max, sum) per head, padded to
  // 16 bytes; the stage gets what the workgroup's LDS share leaves (the
  // resident workgroups of a CU split its 160 KiB), at most 8 records.
  static constexpr int kPartFloats = GC * D + 2 * GC;
  static constexpr int kPartStride = (kPartFloats + 3) / 4 * 4;
  static constexpr int kLdsFixed =
      kLdsSeqs * 8 + kSortSeqs * 4 +
      kWavesPerWG * ((kFp8 && AP ? 2 * D : 16) + (kNewRecs > 0 ? kNewRecs * 2 * kRowB : 16)) +
      kWavesPerWG * (kPvMfma ? kBlockSize * kVS + 4 : kBlockSize * GC * 4 + 16) + 64;
  static constexpr int kLdsPerWg = 160 * 1024 / kGridWaves - 1024;
  static constexpr int kStageFit = (kLdsPerWg - kLdsFixed) / kWavesPerWG / (kPartStride * 4);
  static constexpr int kStageRecs = kStageFit < 1 ? 0 : (kStageFit > 8 ? 8 : kStageFit);
};

struct DecodeParams {
  void* out;
  const char* query;
  const char* kcache;
  const char* vcache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale_log2;    // softmax scale (times the key scale of an E4M3 pool) x log2 e
  float v_scale;       // value scale of an E4M3 pool (1 otherwise)
  int num_seqs, num_heads, num_kv_heads, max_blocks;
  int group;           // query heads per kv head
  int hgk;             // head groups per kv head: ceil(group / GC)
  int64_t num_blocks;
  int tile_cap;        // max tiles per range (0: no cap)
  int r_max;           // ranges the workspace holds
  int* header;         // [2]  ranges R and tiles per range q of this call
  int4* desc;          // [R]  split segment ending in range r: s, hg, P, nb
  int4* desc_first;    // [R]  split segment holding range r's first tile: s, hg, P, nb
  float* part_ml;      // [R][2][GC][2]  running max (log2 units), sum
  float* part_acc;     // [R][2][GC][D]  unnormalized accumulator
  // Appending variant (null otherwise): each sequence's newest token
  // (position L - 1), its key and value rows [S][Hkv][D] of this launch.
  // Its tile takes them from here, and one wave per (sequence, kv head)
  // writes them to the token's slot.
  const char* new_k;
  const char* new_v;
  float k_enc, v_enc;  // E4M3 pools: the scales new rows are encoded with
  // Optional (null: the neighbour rule): per pool block, nonzero when more
  // than one sequence maps it.
  const uint8_t* block_shared;
};

// Head groups.  A kv head's `group` query heads are cut into hgk groups of
// GC heads (GC a power of two up to 8, hgk = ceil(group / GC)); the last
// group of a kv head may be partial.  Its missing heads are computed on a
// copy of a real one and never stored, so a tile is read once per group of
// GC heads even when GC does not divide the group.
__device__ __forceinline__ int kv_head_of(const DecodeParams& p, int hg) { return hg / p.hgk; }
__device__ __forceinline__ int first_head(const DecodeParams& p, int hg, int gc) {
  const int g = hg / p.hgk;
  return g * p.group + (hg - g * p.hgk) * gc;
}
__device__ __forceinline__ int heads_in_group(const DecodeParams& p, int hg, int gc) {
  const int left = p.group - (hg % p.hgk) * gc;
  return left < gc ? left : gc;
}

struct Tile {
  // K in MFMA-B layout (lane l: token l%16, chunks (l/16) + 4m), V as
  // contiguous 1-KiB slices (lane l: bytes ld*1024 + 16l of the tile).
  u32x4 k[8];
  u32x4 v[8];
};

// ------------------------------------------------------ wave utilities --
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ int wave_incl_scan_i(int x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ int sread(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int clamp_len(int L, int max_tokens) {
  return L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
}

__device__ __forceinline__ int blocks_of(int L) { return (L + kBlockSize - 1) / kBlockSize; }


// With the caller's sharing flags, the sequences of a batch of at most
// kSortSeqs are laid out in the flattened order sorted by their first
// block: the siblings of a request (parallel samples, beams) share their
// prompt's blocks from the first one on, so they then sit side by side
// whatever their order in the batch, and the waves that read a shared
// block read it at about the same time, mostly from L2.  One wave sorts
// the keys (first block mod 2^20, sequence) in registers with a bitonic
// network; the keys are distinct, so the order is deterministic.  Larger
// batches, and calls without flags, keep the batch order.

__device__ __forceinline__ bool sorts_batch(const DecodeParams& p) {
  return p.block_shared != nullptr && p.num_seqs <= kSortSeqs;
}

// Places e in 1 .. n-1 of a wave's key array (element e = r * 64 + lane)
// whose first block (key >> 11) differs from element e - 1's.
template <int R>
__device__ __forceinline__ int first_block_runs(const uint32_t (&key)[R], int n, int lane) {
  int runs = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = r * kWave + lane;
    const uint32_t up = (uint32_t)__shfl_up((int)key[r], 1, kWave);
    const uint32_t last = (uint32_t)__shfl((int)key[r > 0 ? r - 1 : 0], kWave - 1, kWave);
    const uint32_t prev = lane > 0 ? up : last;
    runs += (e > 0 && e < n && (prev >> 11) != (key[r] >> 11)) ? 1 : 0;
  }
  return wave_sum_i(runs);
}

// order[i] = the sequence at position i of the flattened order, for the
// first num_seqs <= N positions (one wave; N a power of two from 64 to
// kSortSeqs, element e = r * 64 + lane in register r).
template <int N>
__device__ void sort_by_first_block(const DecodeParams& p, const int* len, int* order,
                                    int lane) {
  constexpr int R = N / kWave;
  uint32_t key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = r * kWave + lane;
    uint32_t k = 0xFFFFFFFFu;  // past the batch: sorted last
    if (e < p.num_seqs) {
      const uint32_t fb =
          len[e] > 0 ? (uint32_t)p.block_tables[(int64_t)e * p.max_blocks] & 0xFFFFFu : 0xFFFFFu;
      k = (fb << 11) | (uint32_t)e;  // e < 2^11
    }
    key[r] = k;
  }
  const int runs_batch = first_block_runs<R>(key, p.num_seqs, lane);
  // bitonic network, ascending
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= kWave) {  // partners in two registers of the same lane
        const int rj = j / kWave;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r & rj) continue;
          const int e = r * kWave + lane;
          const bool up = (e & k) == 0;
          const uint32_t a = key[r], b = key[r | rj];
          const bool swap = up ? a > b : a < b;
          key[r] = swap ? b : a;
          key[r | rj] = swap ? a : b;
        }
      } else {  // partners in lanes lane ^ j: every register's exchange
                // is issued before any is used
        uint32_t o[R];
#pragma unroll
        for (int r = 0; r < R; ++r) o[r] = (uint32_t)__shfl_xor((int)key[r], j, kWave);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int e = r * kWave + lane;
          const bool keep_min = ((e & k) == 0) == ((e & j) == 0);
          key[r] = keep_min ? min(key[r], o[r]) : max(key[r], o[r]);
        }
      }
    }
  }
  // A batch whose sibling groups are already contiguous keeps its own
  // order: the sorted order has as many runs of equal first blocks as the
  // batch order exactly then.  (Measured on one MI355X, decode call us,
  // beam search / parallel sampling batches with the siblings side by
  // side: 103 / 376 in their own order, 108 / 390 sorted; shuffled: 112 /
  // 417 in their order, 110 / 380 sorted.)
  const int runs_sorted = first_block_runs<R>(key, p.num_seqs, lane);
  const bool keep = runs_batch == runs_sorted;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = r * kWave + lane;
    if (i < p.num_seqs) order[i] = keep ? i : (int)(key[r] & 0x7FFu);
  }
}

__device__ void sort_batch(const DecodeParams& p, const int* len, int* order, int lane) {
  if (p.num_seqs <= 64) sort_by_first_block<64>(p, len, order, lane);
  else if (p.num_seqs <= 128) sort_by_first_block<128>(p, len, order, lane);
  else if (p.num_seqs <= 256) sort_by_first_block<256>(p, len, order, lane);
  else sort_by_first_block<kSortSeqs>(p, len, order, lane);
}

// Segment table of this launch's sequences, built in LDS by every thread of
// the workgroup: len[s] = clamped context length of sequence s, order[i] the
// sequence at position i of the flattened order (when the batch is sorted;
// else position i is sequence i), incl[i] = tiles of positions 0..i
// (blocks x head groups), summed.  Returns T = incl[S-1].
__device__ int build_segment_table(const DecodeParams& p, int head_groups, int* incl, int* len,
                                   int* order, int* wsum, int lane, int w) {
  const int S = p.num_seqs;
  const int max_tokens = p.max_blocks * kBlockSize;
  const int per = (S + kThreads - 1) / kThreads;  // positions per thread, contiguous
  const int s0 = threadIdx.x * per;
  const bool sorted = sorts_batch(p);
  int sum = 0;
  for (int k = 0; k < per; ++k) {
    const int s = s0 + k;
    if (s < S) {
      const int L = clamp_len(p.context_lens[s], max_tokens);
      len[s] = L;
      sum += blocks_of(L) * head_groups;
    }
  }
  if (sorted) {
    __syncthreads();
    if (w == 0) sort_batch(p, len, order, lane);
    __syncthreads();
    sum = 0;
    for (int k = 0; k < per; ++k) {
      const int i = s0 + k;
      if (i < S) sum += blocks_of(len[order[i]]) * head_groups;
    }
  }
  const int inc = wave_incl_scan_i(sum, lane);
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  int run = inc - sum;
  int total = 0;
#pragma unroll
  for (int j = 0; j < kWavesPerWG; ++j) {
    const int t = wsum[j];
    run += j < w ? t : 0;
    total += t;
  }
  for (int k = 0; k < per; ++k) {
    const int i = s0 + k;
    if (i < S) {
      run += blocks_of(len[sorted ? order[i] : i]) * head_groups;
      incl[i] = run;
    }
  }
  __syncthreads();
  return sread(total);
}

// Position (in the flattened order) whose tiles hold flattened tile x < T:
// the first i with incl[i] > x.
__device__ __forceinline__ int seq_of(const int* incl, int S, int x) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (incl[mid] > x) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// How the T flattened tiles are cut into ranges: R ranges of q tiles (the
// last one shorter), range r covering tiles [r q, min((r + 1) q, T)).  Wave
// v of NWV takes ranges [v R / NWV, (v + 1) R / NWV).  Both kernels derive
// the same map.
struct RangeMap {
  int q, R, T;
  __device__ __forceinline__ int start(int r) const { return r * q; }
  __device__ __forceinline__ int end(int r) const { return min((r + 1) * q, T); }
  __device__ __forceinline__ int of(int x) const { return x / q; }
};

// An equal share of the tiles per wave (at least kMinTilesPerRange, at
// most the tiles-per-piece cap when there is one).
__device__ RangeMap plan_ranges(int T, int nwaves, int cap) {
  RangeMap m;
  m.T = T;
  int q = T / nwaves + (T % nwaves != 0);
  q = q < kMinTilesPerRange ? kMinTilesPerRange : q;
  if (cap > 0 && q > cap) q = cap;
  m.q = q;
  m.R = T / q + (T % q != 0);
  return m;
}

// N = 2 or 4 bytes at p (aligned to N).
template <int N>
__device__ __forceinline__ uint32_t load_lane_bytes(const char* p) {
  static_assert(N == 2 || N == 4, "2 or 4 bytes");
  if constexpr (N == 4) return *reinterpret_cast<const uint32_t*>(p);
  else return (uint32_t)*reinterpret_cast<const uint16_t*>(p);
}

// The low 16 bits of x as a float16 / bfloat16 value, widened exactly.
template <int DT>
__device__ __forceinline__ float bits16_to_float(uint32_t x) {
  if constexpr (DT == PKV_BF16) return __builtin_bit_cast(float, (x & 0xFFFFu) << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xFFFFu));
}

// Eight E4M3 codes (two words) widened exactly to one 16-bit MFMA operand
// by the packed conversions to float16 / bfloat16 (scale 1: every E4M3
// value is representable in both formats).
template <int DT>
__device__ __forceinline__ u32x4 widen_e4m3x8(int w0, int w1) {
  u32x4 r;
  if constexpr (DT == PKV_F16) {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, true));
  } else {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true));
  }
  return r;
}

// S^T = K Q^T for one tile: the key tile (E4M3 codes widened, as in
// qk_mfma) is the A operand and the query rows the B operand, so lane l
// receives tokens 4(l/16) .. +3 of head l % 16.
template <int DT, int KT, int NQ>
__device__ __forceinline__ floatx4 kq_mfma(const u32x4 (&q)[NQ], const Tile& t) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < NQ; ++m) {
    if constexpr (KT == PKV_FP8_E4M3) {
      const u32x4 kc = t.k[m / 2];
      acc = mfma32<DT>(widen_e4m3x8<DT>((int)kc[2 * (m % 2)], (int)kc[2 * (m % 2) + 1]), q[m],
                       acc);
    } else {
      acc = mfma32<DT>(t.k[m], q[m], acc);
    }
  }
  return acc;
}

template <int DT, int KT, int NQ>
__device__ __forceinline__ floatx4 qk_mfma(const u32x4 (&q)[NQ], const Tile& t) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < NQ; ++m) {
    if constexpr (KT == PKV_FP8_E4M3) {
      // k-step m takes half m % 2 of key chunk m / 2 (the query is read in
      // the same order, so the dot products are unchanged)
      const u32x4 kc = t.k[m / 2];
      const u32x4 kb = widen_e4m3x8<DT>((int)kc[2 * (m % 2)], (int)kc[2 * (m % 2) + 1]);
      if constexpr (DT == PKV_F16)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, q[m]),
                                                     __builtin_bit_cast(half8, kb), acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, q[m]), __builtin_bit_cast(bf16x8, kb), acc, 0, 0, 0);
    } else if constexpr (DT == PKV_F16) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          __builtin_bit_cast(half8, q[m]), __builtin_bit_cast(half8, t.k[m]), acc, 0, 0, 0);
    } else if constexpr (DT == PKV_BF16) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, q[m]), __builtin_bit_cast(bf16x8, t.k[m]), acc, 0, 0, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_float(q[m], e), lane_float(t.k[m], e),
                                                   acc, 0, 0, 0);
    }
  }
  return acc;
}

// Store kEpc floats as one 16-byte chunk of the output type.
template <int DT>
__device__ __forceinline__ void store_chunk(char* dst, const float* x) {
  u32x4 v;
  if constexpr (DT == PKV_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = float_to_bits<DT>(x[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = float_to_bits<DT>(x[2 * i]) | (float_to_bits<DT>(x[2 * i + 1]) << 16);
  }
  store16(dst, v);
}

// ------------------------------------------------------- split merging --
// Merging the pieces k = 0..np-1 of a split segment (ranges rf..rf+np-1):
//   out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k,  M = max_k m_k.
// A wave folds a subset of the pieces into a running (max, sum, acc)
// state; every lane owns 16-byte chunks of the [GC][D] accumulator.
template <int D, int GC>
struct FoldState {
  static constexpr int kChunks = GC * D / 4;
  static constexpr int kCpl = (kChunks + kWave - 1) / kWave;
  // pieces whose loads go out together (registers: kBatch x kCpl chunks)
  static constexpr int kBatch = kCpl == 1 ? 8 : (kCpl <= 4 && GC < 16 ? 4 : 2);
  // Slices of a segment's merge over the waves of its ranges hold at least
  // 8 chunks each; they pay only when a state has more of them than the
  // four waves of a workgroup could take.  Then a workgroup merges a
  // segment in at most two batches per wave and slices take longer ones
  // (at once for groups of 16 heads, whose workgroup merge would spill).
  static constexpr int kMaxSlices = (kChunks + 7) / 8;
  static constexpr bool kSliced = kMaxSlices > kWavesPerWG;
  static constexpr int kWorkgroupPieces =
      !kSliced ? 0x7fffffff : (GC >= 16 ? 8 : 2 * kWavesPerWG * kBatch);
  float M[GC], S[GC];
  floatx4 O[kCpl];
};

struct Split {
  int s, hg, P, nb, rf, np;
  bool rf_tail;  // range rf's piece of this segment sits in its second slot
};

__device__ __forceinline__ Split split_of(const int4& d, const RangeMap& m) {
  Split x;
  x.s = d.x;
  x.hg = d.y;
  x.P = d.z;
  x.nb = d.w;
  x.rf = m.of(x.P);
  x.np = m.of(x.P + x.nb - 1) - x.rf + 1;
  x.rf_tail = x.P != m.start(x.rf);
  return x;
}

// Slot of piece k's partials (range rf + k; the first range's piece may be
// that range's second).
__device__ __forceinline__ int64_t piece_slot(const Split& sp, int k) {
  return (int64_t)(sp.rf + k) * 2 + ((k == 0 && sp.rf_tail) ? 1 : 0);
}

// One piece's partials as a lane holds them: (max, sum) per head, and the
// lane's chunks of the accumulator.
template <int D, int GC>
struct PieceRegs {
  float ml[GC][2];
  u32x4 ac[FoldState<D, GC>::kCpl];
};

template <int D, int GC>
__device__ __forceinline__ void load_piece(const DecodeParams& p, int64_t sl, int lane,
                                           PieceRegs<D, GC>& x) {
  using F = FoldState<D, GC>;
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    x.ml[g][0] = p.part_ml[(sl * GC + g) * 2 + 0];
    x.ml[g][1] = p.part_ml[(sl * GC + g) * 2 + 1];
  }
#pragma unroll
  for (int j = 0; j < F::kCpl; ++j) {
    const int c = min(lane + j * kWave, F::kChunks - 1);
    x.ac[j] = load16(p.part_acc + sl * GC * D + c * 4);
  }
}

template <int D, int GC>
__device__ __forceinline__ void fold_init(FoldState<D, GC>& st) {
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    st.M[g] = -INFINITY;
    st.S[g] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < FoldState<D, GC>::kCpl; ++j) st.O[j] = floatx4{0.f, 0.f, 0.f, 0.f};
}

// st <- st folded with one more piece (every piece's max is finite)
template <int D, int GC>
__device__ __forceinline__ void fold_one(FoldState<D, GC>& st, const PieceRegs<D, GC>& x,
                                         int lane) {
  using F = FoldState<D, GC>;
  float a[GC], bb[GC];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const float mk = x.ml[g][0];
    const float Mn = fmaxf(st.M[g], mk);
    a[g] = __builtin_amdgcn_exp2f(st.M[g] - Mn);
    bb[g] = __builtin_amdgcn_exp2f(mk - Mn);
    st.S[g] = st.S[g] * a[g] + x.ml[g][1] * bb[g];
    st.M[g] = Mn;
  }
#pragma unroll
  for (int j = 0; j < F::kCpl; ++j) {
    const int g = min(lane + j * kWave, F::kChunks - 1) * 4 / D;
    float ag = a[0], bg = bb[0];
#pragma unroll
    for (int gg = 1; gg < GC; ++gg) {
      ag = g == gg ? a[gg] : ag;
      bg = g == gg ? bb[gg] : bg;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) st.O[j][e] = fmaf(st.O[j][e], ag, bg * float_of(x.ac[j][e]));
  }
}

// Fold pieces k0, k0 + kstep, ... < np into `st`.  Loads go out in batches
// with no wait between them (indices past the end are clamped to piece k0
// and skipped when folding), so a batch costs one memory round trip.
template <int D, int GC>
__device__ void fold_pieces(const DecodeParams& p, const Split& sp, int k0, int kstep,
                            int lane, FoldState<D, GC>& st) {
  using F = FoldState<D, GC>;
  constexpr int kBatch = F::kBatch;
  fold_init<D, GC>(st);
  for (int kb = k0; kb < sp.np; kb += kBatch * kstep) {
    PieceRegs<D, GC> x[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int k = kb + b * kstep;
      load_piece<D, GC>(p, piece_slot(sp, k < sp.np ? k : k0), lane, x[b]);
    }
    // keep the whole batch's loads ahead of the folding (the scheduler
    // would otherwise interleave them, one round trip per piece)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (kb + b * kstep >= sp.np) break;
      fold_one<D, GC>(st, x[b], lane);
    }
  }
}

template <int DT, int D, int GC>
__device__ __forceinline__ void store_merged(const DecodeParams& p, const Split& sp, int c,
                                             const floatx4& o, float inv) {
  if (c * 4 / D >= heads_in_group(p, sp.hg, GC)) return;  // a padding head
  char* dst = (char*)p.out +
              (((int64_t)sp.s * p.num_heads + first_head(p, sp.hg, GC)) * D + c * 4) *
                  Elt<DT>::kBytes;
  store4<DT>(dst, o * inv);
}

// The merged output of a segment from its folded state.
template <int DT, int D, int GC>
__device__ __forceinline__ void store_state(const DecodeParams& p, const Split& sp,
                                            const FoldState<D, GC>& st, int lane) {
  using F = FoldState<D, GC>;
#pragma unroll
  for (int j = 0; j < F::kCpl; ++j) {
    const int c = lane + j * kWave;
    if (c < F::kChunks) {
      const int g = c * 4 / D;
      float sg = st.S[0];
#pragma unroll
      for (int gg = 1; gg < GC; ++gg) sg = g == gg ? st.S[gg] : sg;
      store_merged<DT, D, GC>(p, sp, c, st.O[j], 1.f / sg);
    }
  }
}

// A segment of few pieces: one wave folds them all and writes the output.
template <int DT, int D, int GC>
__device__ void merge_by_wave(const DecodeParams& p, const Split& sp, int lane) {
  FoldState<D, GC> st;
  fold_pieces<D, GC>(p, sp, 0, 1, lane, st);
  store_state<DT, D, GC>(p, sp, st, lane);
}

// A segment of many pieces: wave w folds pieces w, w+4, ...; the four wave
// states are then combined through LDS.
template <int D, int GC>
struct MergeSmem {
  float m[kWavesPerWG][GC];
  float l[kWavesPerWG][GC];
  floatx4 o[kWavesPerWG][GC * D / 4];
};

template <int DT, int D, int GC>
__device__ void merge_by_workgroup(const DecodeParams& p, const Split& sp, int lane, int w,
                                   MergeSmem<D, GC>& sm) {
  using F = FoldState<D, GC>;
  F st;
  fold_pieces<D, GC>(p, sp, w, kWavesPerWG, lane, st);
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      sm.m[w][g] = st.M[g];
      sm.l[w][g] = st.S[g];
    }
  }
#pragma unroll
  for (int j = 0; j < F::kCpl; ++j) {
    const int c = lane + j * kWave;
    if (c < F::kChunks) sm.o[w][c] = st.O[j];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < F::kChunks; c += kThreads) {
    const int g = c * 4 / D;
    float Mx = sm.m[0][g];
#pragma unroll
    for (int v = 1; v < kWavesPerWG; ++v) Mx = fmaxf(Mx, sm.m[v][g]);
    float Sx = 0.f;
    floatx4 Ox = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < kWavesPerWG; ++v) {
      const float wt = __builtin_amdgcn_exp2f(sm.m[v][g] - Mx);  // idle wave: 0
      Sx = fmaf(sm.l[v][g], wt, Sx);
      Ox += sm.o[v][c] * wt;
    }
    store_merged<DT, D, GC>(p, sp, c, Ox, 1.f / Sx);
  }
  __syncthreads();
}

// A segment split into more pieces than a workgroup merges in two batches
// is merged by the waves of the ranges it spans.  With n ranges whose first
// tile lies in the segment (at most one per 8 chunks), the k-th of them
// takes the k-th of n contiguous runs of the [GC][D] accumulator's 16-B
// chunks.  Its lanes are CL chunk lanes x 64 / CL piece lanes: lane (c, i)
// folds chunk c of pieces i, i + 64 / CL, ... (kSliceUnroll pieces' loads
// go out together; the chunk lanes read contiguous bytes of a piece), then
// the piece lanes of each chunk are combined.  Runs of up to 8 chunks take
// 8 chunk lanes; wider runs (few pieces, so few ranges) take 16, so that a
// run still costs one round trip per batch of pieces.
constexpr int kSliceUnroll = 8;

template <int DT, int D, int GC, int CL>
__device__ void merge_slice_run(const DecodeParams& p, const Split& sp, int cbeg, int cend,
                                int lane) {
  constexpr int PL = kWave / CL;
  const int cl = lane % CL;
  const int pl = lane / CL;
  for (int c0 = cbeg; c0 < cend; c0 += CL) {
    const int c = min(c0 + cl, cend - 1);
    const int g = c * 4 / D;
    float M = -INFINITY, S = 0.f;
    floatx4 O = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < sp.np; i0 += PL * kSliceUnroll) {
      float mm[kSliceUnroll], ll[kSliceUnroll];
      u32x4 aa[kSliceUnroll];
#pragma unroll
      for (int u = 0; u < kSliceUnroll; ++u) {
        const int i = min(i0 + pl + u * PL, sp.np - 1);
        const int64_t sl = piece_slot(sp, i);
        mm[u] = p.part_ml[(sl * GC + g) * 2 + 0];
        ll[u] = p.part_ml[(sl * GC + g) * 2 + 1];
        aa[u] = load16(p.part_acc + sl * GC * D + c * 4);
      }
      // keep the batch's loads ahead of the folding, and fold without
      // branches (a lane past the last piece folds with weight 0): a branch
      // per piece lets the compiler sink each load into its branch, one
      // round trip per piece
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kSliceUnroll; ++u) {
        const bool ok = i0 + pl + u * PL < sp.np;
        const float Mn = ok ? fmaxf(M, mm[u]) : M;  // every piece's max is finite
        const float a = ok ? __builtin_amdgcn_exp2f(M - Mn) : 1.f;
        const float b = ok ? __builtin_amdgcn_exp2f(mm[u] - Mn) : 0.f;
        S = S * a + ll[u] * b;
#pragma unroll
        for (int e = 0; e < 4; ++e) O[e] = fmaf(O[e], a, b * float_of(aa[u][e]));
        M = Mn;
      }
    }
    // lanes without a piece hold max -inf and weigh 0
    const float Mw = max_over_lane_groups<CL>(M);
    const float wt = __builtin_amdgcn_exp2f(M - Mw);
    const float Sw = sum_over_lane_groups<CL>(S * wt);
    floatx4 Ow;
#pragma unroll
    for (int e = 0; e < 4; ++e) Ow[e] = sum_over_lane_groups<CL>(O[e] * wt);
    if (pl == 0 && c0 + cl < cend) store_merged<DT, D, GC>(p, sp, c0 + cl, Ow, 1.f / Sw);
  }
}

template <int DT, int D, int GC>
__device__ void merge_slice(const DecodeParams& p, const Split& sp, int r, int lane) {
  constexpr int kChunks = GC * D / 4;
  const int first = sp.rf + (sp.rf_tail ? 1 : 0);  // range rf starts in another segment
  // slices of at least 8 chunks: a wave's round trip then brings a full row
  // of chunk lanes (narrow states use the first few ranges)
  const int n = min(sp.rf + sp.np - first, FoldState<D, GC>::kMaxSlices);
  const int cpp = (kChunks + n - 1) / n;
  const int cbeg = (r - first) * cpp;
  const int cend = min(cbeg + cpp, kChunks);
  if (cpp > 8)
    merge_slice_run<DT, D, GC, 16>(p, sp, cbeg, cend, lane);
  else
    merge_slice_run<DT, D, GC, 8>(p, sp, cbeg, cend, lane);
}

// ------------------------------------------------------------ main kernel --
constexpr int kPrepAhead = 3;   // tiles left in a window when the next one is prepared

// Window::info, per tile: head group (bits 0-15), valid tokens (16-20), flags.
constexpr int kPieceFirst = 1 << 21;
constexpr int kPieceLast = 1 << 22;
constexpr int kSegStart = 1 << 23;
constexpr int kSegEnd = 1 << 24;
constexpr int kRangeFirst = 1 << 25;
constexpr int kShared = 1 << 26;  // a neighbouring sequence maps the same block here

__device__ __forceinline__ int pick(bool c, int a, int b) { return c ? a : b; }

// Up to 64 consecutive tiles of one range, lane j describing tile x + j.
struct Window {
  int r, x, cnt;    // range, first flattened tile, tiles (wave-uniform)
  int ends_range;   // the range's last tile lies in this window
  int id;           // lane j: physical block (clamped into the pool)
  int s;            // lane j: sequence
  int info;         // lane j: head group, valid tokens, flags
};

// Where the tiles x .. x + 63 of range r are: sequence, head group and
// block of each (segment table in LDS) and the block id (one gather from
// the block table).  The lane of the range's first tile also writes the
// range's descriptor.
__device__ Window prepare_window(const DecodeParams& p, const RangeMap& m, const int* incl,
                                 const int* len, const int* order, int head_groups, int r,
                                 int xw, int lane) {
  Window wd;
  const int x0 = m.start(r);
  const int x1 = m.end(r);
  wd.r = r;
  wd.x = xw;
  wd.cnt = min(kWave, x1 - xw);
  wd.ends_range = xw + wd.cnt == x1;
  wd.id = 0;
  wd.s = 0;
  wd.info = 0;
  const int x = xw + lane;
  if (lane < wd.cnt) {
    const int i = seq_of(incl, p.num_seqs, x);
    const int s = sorts_batch(p) ? order[i] : i;
    const int excl = i > 0 ? incl[i - 1] : 0;
    const int nb = (incl[i] - excl) / head_groups;
    const int local = x - excl;
    const int hg = local / nb;
    const int n = local - hg * nb;
    const int64_t b_raw = p.block_tables[(int64_t)s * p.max_blocks + n];
    const int64_t b = b_raw < 0 ? 0 : (b_raw >= p.num_blocks ? p.num_blocks - 1 : b_raw);
    // A tile is read by several waves in one call, and is worth keeping in
    // cache, when its kv head serves more than one head group (each group
    // reads it), or when its block is shared between sequences.  The
    // caller's flags say which blocks are ([TEQ] "Paging's second gift":
    // each block carries a reference count, kept by the runtime).  Without
    // them, sequences of one request (parallel samples, beams) are taken to
    // sit side by side: a block that the previous or the next sequence maps
    // at the same index counts as shared (both neighbours' entries are read
    // on every path, from rows clamped into the batch).  Every other tile
    // is read once per call.
    bool shared = head_groups > p.num_kv_heads;
    if (p.block_shared != nullptr) {
      shared = shared || p.block_shared[b] != 0;
    } else {
      const int sp = s > 0 ? s - 1 : s;
      const int sn = s + 1 < p.num_seqs ? s + 1 : s;
      const int64_t b_prev = p.block_tables[(int64_t)sp * p.max_blocks + n];
      const int64_t b_next = p.block_tables[(int64_t)sn * p.max_blocks + n];
      shared = shared || (sp != s && n * kBlockSize < len[sp] && b_prev == b_raw) ||
               (sn != s && n * kBlockSize < len[sn] && b_next == b_raw);
    }
    wd.id = (int)b;
    wd.s = s;
    int f = hg | (min(kBlockSize, len[s] - n * kBlockSize) << 16) | (shared ? kShared : 0);
    if (n == 0) f |= kSegStart | kPieceFirst;
    if (n == nb - 1) f |= kSegEnd | kPieceLast;
    if (x == x1 - 1) f |= kPieceLast;
    if (x == x0) {
      f |= kRangeFirst | kPieceFirst;
      // a range's first piece is the last piece of a split segment exactly
      // when the segment began in an earlier range and ends in this one
      p.desc[r] = (n > 0 && nb - n <= x1 - x0) ? int4{s, hg, x - n, nb} : int4{-1, 0, 0, 0};
      // and the segment this range starts in, when it spans several ranges
      // (for merges in slices)
      if (p.desc_first != nullptr)
        p.desc_first[r] =
            (n > 0 || nb - n > x1 - x0) ? int4{s, hg, x - n, nb} : int4{-1, 0, 0, 0};
    }
    wd.info = f;
  }
  return wd;
}

template <int DT, int KT, int D, int GC, bool AP>
__global__ __launch_bounds__(kThreads, (DecodeCfg<DT, KT, D, GC, AP>::kMinWaves)) void
paged_decode_kernel(const DecodeParams p) {
  using C = DecodeCfg<DT, KT, D, GC, AP>;
  constexpr int NLD = C::kNld;
  constexpr int EPC = C::kEpc;

  __shared__ float sm_p[kWavesPerWG][C::kPvMfma ? 1 : kBlockSize * GC];
  // matrix-core path: each wave's value tile as rows, read back transposed
  __shared__ __attribute__((aligned(16))) char sm_v[kWavesPerWG][C::kPvMfma ? kBlockSize * C::kVS : 16];
  __shared__ __attribute__((aligned(16)))
  float sm_stage[kWavesPerWG][C::kStageRecs > 0 ? C::kStageRecs * C::kPartStride : 4];
  __shared__ int sm_incl[kLdsSeqs];
  __shared__ int sm_len[kLdsSeqs];
  __shared__ int sm_order[kSortSeqs];
  // E4M3 appending: each wave's encoded new key and value rows
  __shared__ __attribute__((aligned(16))) uint8_t sm_new[kWavesPerWG][C::kFp8 && AP ? 2 * D : 16];
  // appending: each wave's new-token rows waiting to be written
  __shared__ __attribute__((aligned(16)))
  char sm_newrec[kWavesPerWG][C::kNewRecs > 0 ? C::kNewRecs * 2 * C::kRowB : 16];
  __shared__ int sm_wsum[kWavesPerWG];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = sread(threadIdx.x >> 6);  // wave index, known uniform to the compiler
  // XCD-aware wave numbering: workgroups are dealt round-robin to the 8
  // XCDs, so give each XCD a contiguous block of wave ids (and therefore of
  // the flattened tile order) to keep shared table rows in one L2.
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int per_xcd = nwg >> 3;
  const int wg_l = (nwg & 7) == 0 ? xcd * per_xcd + (blockIdx.x >> 3) : blockIdx.x;
  const int v = wg_l * kWavesPerWG + w;
  const int nwaves = nwg * kWavesPerWG;

  const int head_groups = p.num_kv_heads * p.hgk;
  const int T = build_segment_table(p, head_groups, sm_incl, sm_len, sm_order, sm_wsum, lane, w);

  // sequences with no cached token: their output is zero
  for (int base = 0; base < p.num_seqs; base += kWave) {
    const int s = base + lane;
    const bool empty = s < p.num_seqs && sm_len[s] == 0;
    unsigned long long z = __ballot(empty && s % nwaves == v);
    while (z) {
      const int l = __ffsll((long long)z) - 1;
      z &= z - 1;
      const int64_t row0 = (int64_t)(base + l) * p.num_heads * D;
      for (int i = lane; i < p.num_heads * D; i += kWave) store_elem<DT>(p.out, row0 + i, 0.f);
    }
  }

  const RangeMap map = plan_ranges(T, nwaves, p.tile_cap);
  if (v == 0 && lane == 0) {
    p.header[0] = map.R;
    p.header[1] = map.q;
  }
  // Wave v takes the consecutive ranges [r_first, r_end), an equal share
  // (within one) of them: its tiles are one contiguous run of the flattened
  // order, and when there are fewer ranges than waves the busy waves are
  // spread evenly over the wave numbering (so over XCDs and CUs).
  const int r_first = (int)((int64_t)v * map.R / nwaves);
  const int r_end = (int)((int64_t)(v + 1) * map.R / nwaves);
  if (r_first >= r_end) return;

  float* pw = sm_p[w];
  const int row = lane & 15;
  const int jg = lane >> 4;
  const uint32_t koff_lane = (uint32_t)(row * C::kRowB + jg * 16);
  const uint32_t voff_lane = (uint32_t)(lane * 16);
  const int64_t block_stride = (int64_t)p.num_kv_heads * C::kTileB;

  // query rows as MFMA A operands: row r of chain c is head c*4 + r % kGcq
  using QRegs = u32x4[C::kNqg][C::kNq];
  // E4M3 pools, appending: this lane's D / 64 elements of the newest
  // token's key and value rows (16-bit), loaded with each piece's q
  uint32_t new_kw = 0u, new_vw = 0u;
  auto load_q = [&](QRegs& q, int s, int hg) {
    if constexpr (C::kFp8) {
      if constexpr (AP) {
        const int64_t nrow = ((int64_t)s * p.num_kv_heads + kv_head_of(p, hg)) * C::kRowQ;
        new_kw = load_lane_bytes<C::kEncBytes>(p.new_k + nrow + lane * C::kEncBytes);
        new_vw = load_lane_bytes<C::kEncBytes>(p.new_v + nrow + lane * C::kEncBytes);
      }
    }
#pragma unroll
    for (int c = 0; c < C::kNqg; ++c) {
      // head within the group: lane column `row` on the matrix-core path
      const int hi = C::kPvMfma ? row : c * 4 + (row % C::kGcq);
      const int nv = heads_in_group(p, hg, GC);
      const int head = first_head(p, hg, GC) + (hi < nv ? hi : nv - 1);
      const char* qrow = p.query + ((int64_t)s * p.num_heads + head) * C::kRowQ;
      // k-step m reads the query elements of key chunk jg + 4m (E4M3: half
      // m % 2 of chunk jg + 4 (m / 2), 16 codes per chunk)
#pragma unroll
      for (int m = 0; m < C::kNq; ++m)
        q[c][m] = load16(qrow + (C::kFp8 ? (jg + 4 * (m / 2)) * 32 + (m % 2) * 16
                                         : (jg + 4 * m) * 16));
    }
  };
  // A tile that only this wave reads in this call is streamed past the
  // cache; a shared one (kShared) and the last block of an appending
  // sequence are read with the default policy.  The three paths issue the
  // same number of loads, so the wait counts do not depend on the path (this
  // file is compiled with uniform regions left unstructurized: structurizing
  // the branch would add a path that issues no load, and the waits after
  // the join would assume it).
  auto load_tile = [&](Tile& t, int id, int hg, int s_t, int info_t) {
    const int g = kv_head_of(p, hg);
    const int64_t off = (int64_t)id * block_stride + (int64_t)g * C::kTileB;
    const char* kb = p.kcache + off;
    const char* vb = p.vcache + off;
    if (!C::kFp8 && AP && (info_t & kSegEnd)) {
      // the sequence's last block: the lanes of its newest token (row
      // valid - 1) read that token's rows from the new keys and values
      const int nt = ((info_t >> 16) & 31) - 1;
      const int64_t nrow = ((int64_t)s_t * p.num_kv_heads + g) * C::kRowB;
#pragma unroll
      for (int m = 0; m < NLD; ++m)
        t.k[m] = load16(row == nt ? p.new_k + nrow + jg * 16 + m * 64 : kb + koff_lane + m * 64);
#pragma unroll
      for (int m = 0; m < NLD; ++m) {
        const uint32_t o = voff_lane + m * 1024;
        t.v[m] = load16((int)(o / C::kRowB) == nt ? p.new_v + nrow + o % C::kRowB : vb + o);
      }
    } else {
      const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kb, C::kTileB);
      const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vb, C::kTileB);
      if (info_t & kShared) {
#pragma unroll
        for (int m = 0; m < NLD; ++m) t.k[m] = load16_buffer<kCacheDefault>(kr, koff_lane + m * 64);
#pragma unroll
        for (int m = 0; m < NLD; ++m)
          t.v[m] = load16_buffer<kCacheDefault>(vr, voff_lane + m * 1024);
      } else {
#pragma unroll
        for (int m = 0; m < NLD; ++m)
          t.k[m] = load16_buffer<kCacheNonTemporal>(kr, koff_lane + m * 64);
#pragma unroll
        for (int m = 0; m < NLD; ++m)
          t.v[m] = load16_buffer<kCacheNonTemporal>(vr, voff_lane + m * 1024);
      }
    }
  };
  // E4M3 pools, appending, in the sequence's last tile: each lane encodes
  // its D / 64 elements of the new key and value rows exactly as
  // reshape_and_cache_fp8 does (the float32 quotient by the pool's scale,
  // nearest code), the codes meet in the wave's LDS, and the lanes that
  // hold row nt of the tile take them in place of what the pool held.
  auto substitute_new_token = [&](Tile& t, int nt) __attribute__((always_inline)) {
    uint32_t kc = 0u, vc = 0u;
#pragma unroll
    for (int e = 0; e < C::kEncPerLane; ++e) {
      kc |= e4m3_code(bits16_to_float<DT>(new_kw >> (16 * e)) / p.k_enc) << (8 * e);
      vc |= e4m3_code(bits16_to_float<DT>(new_vw >> (16 * e)) / p.v_enc) << (8 * e);
    }
    uint8_t* codes = sm_new[w];  // the key row's D codes, then the value row's
    if constexpr (C::kEncPerLane == 2) {
      *reinterpret_cast<uint16_t*>(codes + 2 * lane) = (uint16_t)kc;
      *reinterpret_cast<uint16_t*>(codes + D + 2 * lane) = (uint16_t)vc;
    } else {
      codes[lane] = (uint8_t)kc;
      codes[D + lane] = (uint8_t)vc;
    }
    __builtin_amdgcn_wave_barrier();
    if (row == nt) {
#pragma unroll
      for (int m = 0; m < NLD; ++m)
        t.k[m] = *reinterpret_cast<const u32x4*>(codes + (jg + 4 * m) * 16);
    }
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      if (m * C::kTpl + lane / C::kNch == nt)
        t.v[m] = *reinterpret_cast<const u32x4*>(codes + D + (lane % C::kNch) * 16);
    }
    __builtin_amdgcn_wave_barrier();
  };
  // Appending: the first head group of each kv head writes the newest
  // token's key and value rows (held by the lanes that loaded them) into
  // its slot, once the tile has arrived.
  // The writes are deferred: a store counts against the wait counter the
  // tile loads use, so one issued mid-stream would hold up the next tile
  // until acknowledged.  The lanes holding the new token's row copy it from
  // the tile (after substitution, for E4M3 pools: the codes) into a record
  // of the wave's LDS, and the wave writes its records to their slots after
  // its last tile (or when all kNewRecs are taken).  Measured on one
  // MI355X, decode call us on the 64-sequence OPT-13B-shaped batch, plain
  // / appending: 16-bit pools 188.7 / 193.5 storing at once, 189.0 with the
  // writes skipped; E4M3 pools 110.6 / 119.6 / 114.1.
  int n_new = 0;
  int new_id = 0, new_g = 0, new_nt = 0;  // lane k: record k's block, kv head, slot row
  char* const new_rec = sm_newrec[w];
  auto write_new_tokens = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_wave_barrier();
    for (int k = 0; k < n_new; ++k) {
      const int id = __builtin_amdgcn_readlane(new_id, k);
      const int g = __builtin_amdgcn_readlane(new_g, k);
      const int nt = __builtin_amdgcn_readlane(new_nt, k);
      const int64_t off = (int64_t)id * block_stride + (int64_t)g * C::kTileB + nt * C::kRowB;
      const char* rec = new_rec + k * 2 * C::kRowB;
      for (int c = lane; c < C::kNch; c += kWave) {
        store16(const_cast<char*>(p.kcache) + off + c * 16,
                *reinterpret_cast<const u32x4*>(rec + c * 16));
        store16(const_cast<char*>(p.vcache) + off + c * 16,
                *reinterpret_cast<const u32x4*>(rec + C::kRowB + c * 16));
      }
    }
    __builtin_amdgcn_wave_barrier();
    n_new = 0;
  };
  auto store_new_token = [&](const Tile& t, int id, int hg, int info_t) {
    const int g = kv_head_of(p, hg);
    if (hg != g * p.hgk) return;  // another head group of this kv head
    const int nt = ((info_t >> 16) & 31) - 1;
    if (n_new == C::kNewRecs) write_new_tokens();
    char* rec = new_rec + n_new * 2 * C::kRowB;
    if (row == nt) {
#pragma unroll
      for (int m = 0; m < NLD; ++m) *reinterpret_cast<u32x4*>(rec + (jg + 4 * m) * 16) = t.k[m];
    }
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      if (m * C::kTpl + lane / C::kNch == nt)
        *reinterpret_cast<u32x4*>(rec + C::kRowB + (lane % C::kNch) * 16) = t.v[m];
    }
    if (lane == n_new) {
      new_id = id;
      new_g = g;
      new_nt = nt;
    }
    ++n_new;
  };

  // the wave's stream of tiles: windows cw (being computed) and nw (next)
  Window cw =
      prepare_window(p, map, sm_incl, sm_len, sm_order, head_groups, r_first, map.start(r_first),
                     lane);
  Window nw = cw;
  bool have_nw = false;
  bool no_more = false;  // no range after the current one
  int ci = 0;

  // q of the current piece (the next piece's, once the current piece's
  // last tile is computed)
  QRegs qa;

  // the current piece (set at every piece's first tile; defined here too,
  // since undefined loop-carried values get lowered to reads of arbitrary
  // registers, which may be waiting on a load)
  float m_run[GC], l_run[GC], acc[GC][EPC];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[g][e] = 0.f;
  }
  // matrix-core path: lane l keeps head l % 16 of the group, its running
  // max and (partial) sum, and O^T dims 16b + 4(l/16) .. +3 in block b
  float om_run = -INFINITY, ol_run = 0.f;
  floatx4 oacc[C::kPvMfma ? C::kNdb : 1];
#pragma unroll
  for (int b = 0; b < (C::kPvMfma ? C::kNdb : 1); ++b) oacc[b] = floatx4{0.f, 0.f, 0.f, 0.f};
  bool pc_seg_start = false;
  int pc_slot = 0;

  bool done = false;  // the wave's last tile is computed

  // Staged partials: record k of the wave's stage belongs to workspace slot
  // stage_slot of lane k; n_staged records are waiting.
  float* const stage = sm_stage[w];
  int n_staged = 0;
  int stage_slot = 0;
  auto flush_stage = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_wave_barrier();
    for (int k = 0; k < n_staged; ++k) {
      const int64_t slot = __builtin_amdgcn_readlane(stage_slot, k);
      const float* src = stage + k * C::kPartStride;
      for (int c = lane; c < GC * D / 4; c += kWave)
        store16(p.part_acc + slot * GC * D + c * 4, *reinterpret_cast<const u32x4*>(src + c * 4));
      if (lane < 2 * GC) p.part_ml[slot * GC * 2 + lane] = src[GC * D + lane];
    }
    __builtin_amdgcn_wave_barrier();
    n_staged = 0;
  };
  // The record a piece's partials go into: the next free one of the stage
  // (a full stage leaves the piece to store its partials at once).
  auto stage_record = [&](int slot) __attribute__((always_inline)) -> float* {
    if (lane == n_staged) stage_slot = slot;
    return stage + (n_staged++) * C::kPartStride;
  };
  // the next window: of this range, or the wave's next range
  auto prepare_next = [&]() __attribute__((always_inline)) {
    const int r2 = cw.ends_range ? cw.r + 1 : cw.r;
    // both flags set on both paths: a store through a selected address
    // would keep them in memory
    have_nw = r2 < r_end;
    no_more = r2 >= r_end;
    if (r2 < r_end)
      nw = prepare_window(p, map, sm_incl, sm_len, sm_order, head_groups, r2,
                          cw.ends_range ? map.start(r2) : cw.x + cw.cnt, lane);
  };
  auto step = [&](Tile& tc, Tile& tn) __attribute__((always_inline)) {
    if (done) return;
    // 1. look ahead: the next window is prepared a few tiles before this one
    // runs out.  Its block-table gather is waited for at once (its flags
    // need the ids), so with 16-bit pools, which wait for the next tile
    // before computing anyway, it is prepared after that tile's loads are
    // issued and the two round trips overlap -- unless the next tile is
    // already the next window's first.
    const bool prep = !have_nw && !no_more && cw.cnt - ci <= kPrepAhead;
    const bool prep_first = prep && (C::kOverlapNext || ci + 1 >= cw.cnt);
    if (prep_first) prepare_next();

    // 2. issue the loads of the next tile
    const int info = __builtin_amdgcn_readlane(cw.info, ci);
    const int s = __builtin_amdgcn_readlane(cw.s, ci);
    const int hg = info & 0xffff;
    const int valid = (info >> 16) & 31;  // >= 1; < 16 only in a sequence's last block
    const bool in_cw = ci + 1 < cw.cnt;
    const bool more = in_cw || have_nw;
    // by value: a conditional over the two windows' fields would select
    // addresses and keep the windows in memory
    const int j = in_cw ? ci + 1 : 0;
    const int info_n = __builtin_amdgcn_readlane(pick(in_cw, cw.info, nw.info), j);
    const int s_n = __builtin_amdgcn_readlane(pick(in_cw, cw.s, nw.s), j);
    // Issued on every step; after the wave's last tile it reloads that tile
    // (just read, so served by L2).  A load issued on some paths only would
    // make the wait for this tile's data also wait for the next tile's.
    const int id_n = __builtin_amdgcn_readlane(pick(in_cw, cw.id, nw.id), j);
    const int id_c = __builtin_amdgcn_readlane(cw.id, ci);
    load_tile(tn, more ? id_n : id_c, more ? (info_n & 0xffff) : hg, more ? s_n : s,
              more ? info_n : info);
    if (prep && !prep_first) prepare_next();
    if constexpr (!C::kOverlapNext) __builtin_amdgcn_s_waitcnt(kWaitAllLoads);

    // 3. compute the current tile
    if constexpr (C::kFp8) {
      if (AP && (info & kSegEnd)) substitute_new_token(tc, valid - 1);
    }
    if (info & kPieceFirst) {
      if constexpr (C::kPvMfma) {
        om_run = -INFINITY;
        ol_run = 0.f;
#pragma unroll
        for (int b = 0; b < C::kNdb; ++b) oacc[b] = floatx4{0.f, 0.f, 0.f, 0.f};
      } else {
#pragma unroll
        for (int g = 0; g < GC; ++g) {
          m_run[g] = -INFINITY;
          l_run[g] = 0.f;
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[g][e] = 0.f;
        }
      }
      pc_seg_start = (info & kSegStart) != 0;
      pc_slot = cw.r * 2 + ((info & kRangeFirst) ? 0 : 1);
    }
    if constexpr (C::kPvMfma) {
      // S^T = K Q^T: lane l gets tokens 4(l/16) .. +3 of head l % 16
      const floatx4 rr = kq_mfma<DT, KT, C::kNq>(qa[0], tc);
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = 4 * jg + i < valid ? rr[i] * p.scale_log2 : -INFINITY;
      if (AP && (info & kSegEnd))
        store_new_token(tc, __builtin_amdgcn_readlane(cw.id, ci), hg, info);
      // the value tile into the wave's LDS rows as 16-bit elements (E4M3
      // codes widened exactly), rows past the context zeroed
      char* sv = sm_v[w];
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld) {
        const int tok = ld * C::kTpl + lane / C::kNch;
        u32x4 vv = tc.v[ld];
        if (valid < kBlockSize && tok >= valid) vv = u32x4{0u, 0u, 0u, 0u};
        if constexpr (C::kFp8) {
          char* dst = sv + tok * C::kVS + (lane % C::kNch) * 32;
          store16(dst, widen_e4m3x8<DT>((int)vv[0], (int)vv[1]));
          store16(dst + 16, widen_e4m3x8<DT>((int)vv[2], (int)vv[3]));
        } else {
          store16(sv + tok * C::kVS + (lane % C::kNch) * 16, vv);
        }
      }
      __builtin_amdgcn_wave_barrier();
      // online softmax, lane-local (a head's 16 tokens sit in lanes l, l^16,
      // l^32, l^48)
      const float m_tile = max4rows(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      const bool grow = m_tile > om_run + kPvSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? m_tile : om_run;
        const float alpha = __builtin_amdgcn_exp2f(om_run - m_new);
        om_run = m_new;
        ol_run *= alpha;
#pragma unroll
        for (int b = 0; b < C::kNdb; ++b) oacc[b] *= alpha;
      }
      float pe[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pe[i] = __builtin_amdgcn_exp2f(x[i] - om_run);
      ol_run += (pe[0] + pe[1]) + (pe[2] + pe[3]);
      // P^T as the B operand: k slots 8(l/16) .. +3 hold the four
      // probabilities rounded to the 16-bit type, slots +4 .. +7 what that
      // rounding left out; the values fill both halves alike
      const u32x4 pb = split_probs<DT>(pe);
      // O^T += V^T P^T: lane l reads dim 16b + l % 16 of tokens 4(l/16) .. +3
      const char* vsrc = sv + (4 * jg + (row >> 2)) * C::kVS + (row & 3) * 8;
#pragma unroll
      for (int b = 0; b < C::kNdb; ++b) {
        const uint2 va = read_tr16(vsrc + 32 * b);
        oacc[b] = mfma32<DT>(u32x4{va.x, va.y, va.x, va.y}, pb, oacc[b]);
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      float sc[GC];
#pragma unroll
      for (int c = 0; c < C::kNqg; ++c) {
        const floatx4 rr = qk_mfma<DT, KT, C::kNq>(qa[c], tc);
#pragma unroll
        for (int j = 0; j < C::kGcq; ++j) sc[c * 4 + j] = rr[j] * p.scale_log2;
      }
      if (row >= valid) {
#pragma unroll
        for (int g = 0; g < GC; ++g) sc[g] = -INFINITY;
      }
      if (AP && (info & kSegEnd))
        store_new_token(tc, __builtin_amdgcn_readlane(cw.id, ci), hg, info);
      // The running max is raised (to the tile's max, and the state
      // rescaled) only when a logit exceeds it by more than kPvSlack, so
      // most tiles need no reduction over the lanes; probabilities then
      // stay below 2^kPvSlack.
      float pr[GC];
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        if (__builtin_amdgcn_ballot_w64(sc[g] > m_run[g] + kPvSlack)) {
          const float tmax = uniform(row_max16(sc[g]));
          const float alpha = __builtin_amdgcn_exp2f(m_run[g] - tmax);
          l_run[g] *= alpha;
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[g][e] *= alpha;
          m_run[g] = tmax;
        }
        pr[g] = __builtin_amdgcn_exp2f(sc[g] - m_run[g]);
        l_run[g] += pr[g];
      }
      if (lane < kBlockSize) {
#pragma unroll
        for (int g = 0; g < GC; ++g) pw[lane * GC + g] = pr[g];
      }
      // value rows past the context zeroed (only a sequence's last block
      // has them)
      if (valid < kBlockSize) {
#pragma unroll
        for (int ld = 0; ld < NLD; ++ld) {
          if (ld * C::kTpl + lane / C::kNch >= valid) tc.v[ld] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld) {
        const int tok = ld * C::kTpl + lane / C::kNch;
        float pv[GC];
#pragma unroll
        for (int g = 0; g < GC; ++g) pv[g] = pw[tok * GC + g];
        float fv[EPC];
        widen_chunk<KT>(tc.v[ld], fv);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
#pragma unroll
          for (int g = 0; g < GC; ++g) acc[g][e] = fmaf(pv[g], fv[e], acc[g][e]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (C::kPvMfma && (info & kPieceLast)) {
      // the head's sum over its four lanes; the accumulator is complete
      const float l_tot = sum4rows(ol_run);
      const int h0 = first_head(p, hg, GC);
      const int nv = heads_in_group(p, hg, GC);
      const float vs = C::kFp8 ? p.v_scale : 1.f;  // partials hold the values' scale
      if (pc_seg_start && (info & kSegEnd)) {  // a whole segment: final output
        if (row < nv) {
          const float inv = vs / l_tot;
          char* dst = (char*)p.out + (((int64_t)s * p.num_heads + h0 + row) * D + 4 * jg) * C::kEszQ;
#pragma unroll
          for (int b = 0; b < C::kNdb; ++b) store4<DT>(dst + 16 * b * C::kEszQ, oacc[b] * inv);
        }
      } else if (C::kStageRecs > 0 && n_staged < C::kStageRecs) {  // split piece: staged
        float* rec = stage_record(pc_slot);
        if (row < GC) {
#pragma unroll
          for (int b = 0; b < C::kNdb; ++b)
            *reinterpret_cast<floatx4*>(rec + row * D + 4 * jg + 16 * b) = oacc[b] * vs;
          if (jg == 0) {
            rec[GC * D + 2 * row] = om_run;
            rec[GC * D + 2 * row + 1] = l_tot;
          }
        }
      } else if (row < GC) {  // a piece of a split segment: float32 partials
        const int64_t slot = pc_slot;
        float* dst = p.part_acc + (slot * GC + row) * D + 4 * jg;
#pragma unroll
        for (int b = 0; b < C::kNdb; ++b)
          store16(dst + 16 * b, u32x4{bits_of(oacc[b][0] * vs), bits_of(oacc[b][1] * vs),
                                      bits_of(oacc[b][2] * vs), bits_of(oacc[b][3] * vs)});
        if (jg == 0) {
          p.part_ml[(slot * GC + row) * 2 + 0] = om_run;
          p.part_ml[(slot * GC + row) * 2 + 1] = l_tot;
        }
      }
    }
    if (!C::kPvMfma && (info & kPieceLast)) {
      // piece totals: l over the 16 token lanes; acc over lanes sharing a chunk
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        l_run[g] = row_sum16(l_run[g]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[g][e] = sum_over_lane_groups<C::kNch>(acc[g][e]);
      }
      const int h0 = first_head(p, hg, GC);
      const int nv = heads_in_group(p, hg, GC);
      if (pc_seg_start && (info & kSegEnd)) {  // a whole segment: final output
        if (lane < C::kNch) {
#pragma unroll
          for (int g = 0; g < GC; ++g) {
            if (g >= nv) break;  // padding heads
            const float inv = (C::kFp8 ? p.v_scale : 1.f) / l_run[g];
            float o[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[e] = acc[g][e] * inv;
            char* dst = (char*)p.out +
                        (((int64_t)s * p.num_heads + h0 + g) * D + lane * EPC) * C::kEszQ;
#pragma unroll
            for (int e = 0; e < EPC; e += C::kEpcQ) store_chunk<DT>(dst + e * C::kEszQ, o + e);
          }
        }
      } else if (C::kStageRecs > 0 && n_staged < C::kStageRecs) {  // split piece: staged
        const float vs = C::kFp8 ? p.v_scale : 1.f;  // partials hold the values' scale
        float* rec = stage_record(pc_slot);
        if (lane < C::kNch) {
#pragma unroll
          for (int g = 0; g < GC; ++g) {
#pragma unroll
            for (int e = 0; e < EPC; e += 4)
              *reinterpret_cast<floatx4*>(rec + g * D + lane * EPC + e) =
                  floatx4{acc[g][e] * vs, acc[g][e + 1] * vs, acc[g][e + 2] * vs,
                          acc[g][e + 3] * vs};
          }
        }
        if (lane == 0) {
#pragma unroll
          for (int g = 0; g < GC; ++g) {
            rec[GC * D + 2 * g] = m_run[g];
            rec[GC * D + 2 * g + 1] = l_run[g];
          }
        }
      } else {  // a piece of a split segment: float32 partials
        const int64_t slot = pc_slot;
        const float vs = C::kFp8 ? p.v_scale : 1.f;  // partials hold the values' scale
        if (lane < C::kNch) {
#pragma unroll
          for (int g = 0; g < GC; ++g) {
            float* dst = p.part_acc + (slot * GC + g) * D + lane * EPC;
#pragma unroll
            for (int e = 0; e < EPC; e += 4)
              store16(dst + e, u32x4{bits_of(acc[g][e] * vs), bits_of(acc[g][e + 1] * vs),
                                     bits_of(acc[g][e + 2] * vs), bits_of(acc[g][e + 3] * vs)});
          }
        }
        if (lane == 0) {
#pragma unroll
          for (int g = 0; g < GC; ++g) {
            p.part_ml[(slot * GC + g) * 2 + 0] = m_run[g];
            p.part_ml[(slot * GC + g) * 2 + 1] = l_run[g];
          }
        }
      }
    }

    // 4. the next tile opens a new segment: its q goes into the registers
    // this tile has finished with, and arrives with that tile's own data (a
    // wave's tiles are one contiguous run, so a piece that does not start
    // its segment continues the previous piece's and keeps its q)
    if (more && (info_n & kSegStart)) load_q(qa, s_n, info_n & 0xffff);

    // 5. advance
    if (++ci == cw.cnt) {
      done = !have_nw;
      cw = nw;
      have_nw = false;
      ci = 0;
    }
  };

  // two register tiles, alternating: the next tile is in flight while the
  // current one is computed, across piece, window and range boundaries
  Tile ta, tb;
  {
    const int info = __builtin_amdgcn_readlane(cw.info, 0);
    load_tile(ta, __builtin_amdgcn_readlane(cw.id, 0), info & 0xffff,
              __builtin_amdgcn_readlane(cw.s, 0), info);
    load_q(qa, __builtin_amdgcn_readlane(cw.s, 0), info & 0xffff);
  }
  // One exit, at the end of the body: leaving between the two steps leaves
  // the second step's loop-carried values undefined on that path, and
  // those get materialized from arbitrary registers -- which can hold a
  // load in flight, so every step would wait for it.
  for (;;) {
    step(ta, tb);
    step(tb, ta);
    if (done) break;
  }
  if constexpr (C::kStageRecs > 0) flush_stage();
  if constexpr (AP) write_new_tokens();
}

// ----------------------------------------------------------- merge kernel --
// A wave per range, workgroups taking four ranges at a time.  A range whose
// descriptor names a split segment of few pieces merges it alone; the four
// waves together merge a segment of more pieces; every range of a segment
// split into still more pieces takes its slice of that segment's merge.  A
// wave loads the next descriptors while it merges (the workspace holds
// r_max of each, so the loads are in bounds before R is known).
template <int DT, int D, int GC>
__global__ __launch_bounds__(kThreads, 2) void paged_decode_merge_kernel(const DecodeParams p) {
  using F = FoldState<D, GC>;
  __shared__ MergeSmem<D, GC> sm;
  __shared__ int4 sm_desc[kWavesPerWG];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = sread(threadIdx.x >> 6);
  const int stride = gridDim.x * kWavesPerWG;
  const int4 none = int4{-1, 0, 0, 0};
  int base = blockIdx.x * kWavesPerWG;
  int4 dn = base + w < p.r_max ? p.desc[base + w] : none;
  int4 fn = F::kSliced && base + w < p.r_max ? p.desc_first[base + w] : none;
  // Most split segments of a batch of short contexts are cut once, between
  // the end of range r - 1 and the start of range r: the partials of those
  // two pieces are loaded with the first descriptor, and used if it names
  // exactly that split (one round trip saved; slots 2r - 1 and 2r are
  // inside the workspace whatever it holds).  Only for states of one chunk
  // per lane (one or two heads per group): wider groups come with long
  // contexts split many ways, where the loads would be wasted.
  constexpr bool kSpec = F::kCpl == 1;
  PieceRegs<D, GC> spec[kSpec ? 2 : 1];
  const int r_spec = base + w;
  if constexpr (kSpec) {
    const int64_t s1 = r_spec < p.r_max ? 2 * (int64_t)r_spec : 0;
    load_piece<D, GC>(p, s1 > 0 ? s1 - 1 : 0, lane, spec[0]);
    load_piece<D, GC>(p, s1, lane, spec[1]);
  }
  RangeMap m;
  const int R = p.header[0];
  m.R = R;
  m.q = p.header[1];
  m.T = 0;  // range ends are not needed here
  for (; base < R; base += stride) {
    const int r = base + w;
    const int4 d = r < R ? dn : none;
    const int4 f = r < R ? fn : none;
    if (r + stride < min(R, p.r_max)) {
      dn = p.desc[r + stride];
      if constexpr (F::kSliced) fn = p.desc_first[r + stride];
    }
    if (d.x >= 0) {
      const Split sp = split_of(d, m);
      if (kSpec && r == r_spec && sp.np == 2 && sp.rf == r - 1 && sp.rf_tail) {
        F st;
        fold_init<D, GC>(st);
        fold_one<D, GC>(st, spec[0], lane);
        fold_one<D, GC>(st, spec[kSpec ? 1 : 0], lane);
        store_state<DT, D, GC>(p, sp, st, lane);
      } else if (sp.np <= kSoloPieces) {
        merge_by_wave<DT, D, GC>(p, sp, lane);
      }
    }
    if (F::kSliced && f.x >= 0) {
      const Split sp = split_of(f, m);
      if (sp.np > F::kWorkgroupPieces) merge_slice<DT, D, GC>(p, sp, r, lane);
    }
    if (lane == 0) sm_desc[w] = d;
    __syncthreads();
#pragma unroll 1
    for (int u = 0; u < kWavesPerWG; ++u) {
      const int4 du = sm_desc[u];
      if (du.x < 0) continue;
      const Split sp = split_of(du, m);
      if (sp.np > kSoloPieces && sp.np <= F::kWorkgroupPieces)
        merge_by_workgroup<DT, D, GC>(p, sp, lane, w, sm);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ host --
// Resident workgroups of a kernel on the current device (memoized: the
// answer depends only on the device and the kernel's resources).
// The memo is a fixed table (no heap allocation on any call); once full,
// further answers are computed afresh each time.
struct OccupancyMemo {
  int dev;
  const void* kernel;
  int wgs;
};
constexpr int kOccupancyMemo = 512;

static int resident_workgroups(const void* kernel, int waves_per_simd) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static OccupancyMemo memo[kOccupancyMemo];
  static int memo_n = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < memo_n; ++i)
    if (memo[i].dev == dev && memo[i].kernel == kernel) return memo[i].wgs;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess)
    return 0;
  // a workgroup puts one wave on each SIMD of its CU
  if (per_cu > waves_per_simd) per_cu = waves_per_simd;
  int n = cus * (per_cu > 0 ? per_cu : 1);
  n = n > kMaxWGs ? kMaxWGs : n;
  if (memo_n < kOccupancyMemo) memo[memo_n++] = OccupancyMemo{dev, kernel, n};
  return n;
}

template <int DT, int KT, int D, int GC>
static hipError_t launch_decode(DecodeParams a, hipStream_t st) {
  if (!FoldState<D, GC>::kSliced) a.desc_first = nullptr;  // no merges in slices
  // the appending kernel where the call carries new rows
  const bool ap = a.new_k != nullptr;
  const void* k = ap ? reinterpret_cast<const void*>(&paged_decode_kernel<DT, KT, D, GC, true>)
                     : reinterpret_cast<const void*>(&paged_decode_kernel<DT, KT, D, GC, false>);
  const int nwg = resident_workgroups(k, DecodeCfg<DT, KT, D, GC>::kGridWaves);
  if (nwg <= 0) return hipErrorInvalidDevice;
  // The merge kernel takes a range per wave per round.  Without a cap there
  // are at most as many ranges as decode waves; with one, up to tiles / cap:
  // enough workgroups for one round (at most kMergeRounds times the decode
  // grid), so merges in slices of many-piece segments all run at once.
  int64_t ranges = (int64_t)nwg * kWavesPerWG;
  if (a.tile_cap > 0) {
    const int64_t tiles = (int64_t)a.num_seqs * a.max_blocks * a.num_kv_heads * a.hgk;
    const int64_t rc = (tiles + a.tile_cap - 1) / a.tile_cap;
    ranges = rc > ranges ? rc : ranges;
  }
  int64_t mwg = (ranges + kWavesPerWG - 1) / kWavesPerWG;
  mwg = mwg < (int64_t)nwg * kMergeRounds ? mwg : (int64_t)nwg * kMergeRounds;
  if (ap)
    hipLaunchKernelGGL((paged_decode_kernel<DT, KT, D, GC, true>), dim3(nwg), dim3(kThreads), 0,
                       st, a);
  else
    hipLaunchKernelGGL((paged_decode_kernel<DT, KT, D, GC, false>), dim3(nwg), dim3(kThreads), 0,
                       st, a);
  hipLaunchKernelGGL((paged_decode_merge_kernel<DT, D, GC>), dim3((unsigned)mwg),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int DT, int KT, int D>
static hipError_t dispatch_gc(const DecodeParams& a, int gc, hipStream_t st) {
  switch (gc) {
    case 1: return launch_decode<DT, KT, D, 1>(a, st);
    case 2: return launch_decode<DT, KT, D, 2>(a, st);
    case 4: return launch_decode<DT, KT, D, 4>(a, st);
    case 8: return launch_decode<DT, KT, D, 8>(a, st);
    default:
      if constexpr (DT != PKV_F32) return launch_decode<DT, KT, D, 16>(a, st);
      return hipErrorInvalidValue;  // never chosen for these pools
  }
}

template <int DT, int KT>
static hipError_t dispatch_d(const DecodeParams& a, int d, int gc, hipStream_t st) {
  return d == 64 ? dispatch_gc<DT, KT, 64>(a, gc, st) : dispatch_gc<DT, KT, 128>(a, gc, st);
}

// Heads per head group: the smallest power of two that holds a kv head's
// query heads, at most 16 where both products run on the matrix cores
// (16-bit queries, whose lane columns hold 16 heads) and 8 otherwise (larger
// groups are cut into groups of that size, the last one possibly partial).
// One wave then reads each tile for all of them.
static int heads_per_wg(int num_heads, int num_kv_heads, bool matrix_pv) {
  const int group = num_heads / num_kv_heads;
  if (matrix_pv && group >= 9) return 16;
  return group >= 5 ? 8 : group >= 3 ? 4 : group;
}
// Head groups of the whole batch row: num_kv_heads * ceil(group / gc).
static int64_t head_groups_of(int num_heads, int num_kv_heads, int gc) {
  const int group = num_heads / num_kv_heads;
  return (int64_t)num_kv_heads * ((group + gc - 1) / gc);
}

// Largest number of ranges any launch can form (partials are 2 per range).
static int64_t max_ranges(int64_t max_tiles, int tile_cap) {
  int64_t r = kMaxWaves;
  if (tile_cap > 0) {
    const int64_t rc = (max_tiles + tile_cap - 1) / tile_cap;
    r = rc > r ? rc : r;
  }
  return r;
}

// Workspace: header [2 ints], two range descriptors [r][4 ints] each (the
// split segment ending in the range, the one its first tile lies in), then
// (max, sum) [r][2][gc][2] and accumulators [r][2][gc][head_size] in
// float32; each part 256-B aligned.  Every call writes what it reads.
struct WorkspaceLayout {
  size_t header, desc, desc_first, part_ml, part_acc, total;
};
static WorkspaceLayout workspace_layout(int64_t r, int gc, int head_size) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WorkspaceLayout l;
  l.header = 0;
  l.desc = 256;
  l.desc_first = up(l.desc + (size_t)r * 16);
  l.part_ml = up(l.desc_first + (size_t)r * 16);
  l.part_acc = up(l.part_ml + (size_t)r * 2 * gc * 2 * sizeof(float));
  l.total = up(l.part_acc + (size_t)r * 2 * gc * head_size * sizeof(float));
  return l;
}

static bool partition_ok(int ps) {
  return ps == 0 || (ps >= kBlockSize && ps <= kMaxPartition && ps % kBlockSize == 0);
}

// ----------------------------------------- scratch of the allocation-free call --
// paged_attention_decode_noalloc keeps the split-context workspace (header,
// range descriptors, float32 partials) in this file-scope device array
// instead of caller memory.  Every device the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: the device address of this device's copy
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is ever passed to a kernel.  The decode
// kernel writes every header field, descriptor and partial the merge kernel
// reads, so nothing in it needs clearing between calls; two calls that
// overlap on one device share it and race.
constexpr size_t kScratchBytes = (size_t)PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

static void* scratch_address(int dev) {
  static std::mutex mu;
  static void* addr[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    addr[dev] = ptr;
  }
  return addr[dev];
}

}  // namespace pkv

extern "C" size_t paged_attention_workspace_bytes(int num_seqs, int num_heads,
                                                  int num_kv_heads, int head_size,
                                                  int max_blocks_per_seq, int block_size,
                                                  int partition_size) {
  using namespace pkv;
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads ||
      head_size <= 0 || max_blocks_per_seq <= 0 || block_size != kBlockSize ||
      !partition_ok(partition_size))
    return 0;
  // the pools' format is not an argument: size for both head-group choices
  const int per_launch = num_seqs < kLdsSeqs ? num_seqs : kLdsSeqs;
  size_t total = 0;
  for (const bool matrix_pv : {false, true}) {
    const int gc = heads_per_wg(num_heads, num_kv_heads, matrix_pv);
    const int64_t max_tiles =
        (int64_t)per_launch * max_blocks_per_seq * head_groups_of(num_heads, num_kv_heads, gc);
    const int64_t r = max_ranges(max_tiles, partition_size / kBlockSize);
    const size_t t = workspace_layout(r, gc, head_size).total;
    total = t > total ? t : total;
  }
  return total;
}

namespace pkv {

// Both decode entry points: validation, workspace layout and one launch
// (decode + merge) per kLdsSeqs sequences.  kv_dtype is dtype itself or
// PKV_FP8_E4M3 (with 16-bit queries).
static int decode_impl(void* out, const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_tables,
                       const int32_t* context_lens, float scale, float k_scale, float v_scale,
                       int num_kv_heads, int num_seqs, int num_heads, int head_size,
                       int block_size, int max_blocks_per_seq, int64_t num_blocks,
                       int partition_size, void* workspace, size_t workspace_bytes, int dtype,
                       int kv_dtype, void* stream, const void* new_key = nullptr,
                       const void* new_value = nullptr, bool static_scratch = false,
                       const uint8_t* block_shared = nullptr) {
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if ((new_key == nullptr) != (new_value == nullptr)) return PKV_ERR_INVALID_ARG;

  if (((uintptr_t)new_key | (uintptr_t)new_value) & 15u) return PKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || num_blocks > INT32_MAX)
    return PKV_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (kv_dtype != dtype && !(kv_dtype == PKV_FP8_E4M3 && dtype != PKV_F32))
    return PKV_ERR_UNSUPPORTED;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale > 3.0e38f || v_scale > 3.0e38f)
    return PKV_ERR_INVALID_ARG;  // finite and positive (NaN fails both tests)
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PKV_ERR_UNSUPPORTED;
  if (!partition_ok(partition_size)) return PKV_ERR_INVALID_ARG;
  if (((uintptr_t)query | (uintptr_t)key_cache | (uintptr_t)value_cache | (uintptr_t)out) &
      15u)
    return PKV_ERR_INVALID_ARG;  // rows are read and written 16 bytes at a time
  // 16 heads per group only where both products run on the matrix cores
  const bool matrix_pv = dtype != PKV_F32;
  const int gc = heads_per_wg(num_heads, num_kv_heads, matrix_pv);
  const int64_t hgs = head_groups_of(num_heads, num_kv_heads, gc);
  if (hgs > 0xFFFF) return PKV_ERR_INVALID_ARG;  // head group: 16 bits
  // flattened tile positions within one launch are 32-bit
  const int per_launch = num_seqs < kLdsSeqs ? num_seqs : kLdsSeqs;
  if ((int64_t)per_launch * max_blocks_per_seq * hgs > INT32_MAX) return PKV_ERR_INVALID_ARG;
  const int tile_cap = partition_size / kBlockSize;
  const int64_t launch_tiles = (int64_t)per_launch * max_blocks_per_seq * hgs;
  int64_t r;
  if (static_scratch) {
    // The file-scope scratch of this device stands in for the workspace,
    // sized for the waves this device's grid can hold rather than for any
    // device: the grid never exceeds cus x waves per SIMD workgroups.
    if (num_seqs == 0) return PKV_OK;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return PKV_ERR_HIP;
    const int gw = kv_dtype == PKV_FP8_E4M3 ? kWavesPerSimdFp8 : kWavesPerSimd;
    const int64_t wgs = (int64_t)cus * gw < kMaxWGs ? (int64_t)cus * gw : kMaxWGs;
    r = wgs * kWavesPerWG;
    if (tile_cap > 0 && (launch_tiles + tile_cap - 1) / tile_cap > r)
      r = (launch_tiles + tile_cap - 1) / tile_cap;
    if (r > INT32_MAX || workspace_layout(r, gc, head_size).total > kScratchBytes)
      return PKV_ERR_WORKSPACE;
    workspace = scratch_address(dev);
    if (workspace == nullptr) return PKV_ERR_HIP;
    workspace_bytes = kScratchBytes;
  } else {
    if (num_seqs == 0) return PKV_OK;
    const size_t need = paged_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads,
                                                        head_size, max_blocks_per_seq,
                                                        block_size, partition_size);
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    r = max_ranges(launch_tiles, tile_cap);
    if (r > INT32_MAX) return PKV_ERR_INVALID_ARG;
  }
  if ((uintptr_t)workspace & 15u) return PKV_ERR_INVALID_ARG;

  DecodeParams a{};
  a.out = out;
  a.query = (const char*)query;
  a.kcache = (const char*)key_cache;
  a.vcache = (const char*)value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.block_shared = block_shared;
  // exp(x) = 2^(x log2 e); an E4M3 pool's key scale multiplies every logit
  a.scale_log2 = scale * k_scale * 1.4426950408889634f;
  a.v_scale = v_scale;
  a.k_enc = k_scale;
  a.v_enc = v_scale;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.hgk = (a.group + gc - 1) / gc;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.tile_cap = tile_cap;
  a.r_max = (int)r;
  const WorkspaceLayout wl = workspace_layout(r, gc, head_size);
  a.header = (int*)((char*)workspace + wl.header);
  a.desc = (int4*)((char*)workspace + wl.desc);
  a.desc_first = (int4*)((char*)workspace + wl.desc_first);
  a.part_ml = (float*)((char*)workspace + wl.part_ml);
  a.part_acc = (float*)((char*)workspace + wl.part_acc);
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();  // start from a clean error state
  // one launch (decode + merge) per kLdsSeqs sequences, in stream order;
  // they share the workspace, which each launch leaves ready for the next
  const int esz = dtype == PKV_F32 ? 4 : 2;
  const int64_t row = (int64_t)num_heads * head_size * esz;
  const int64_t new_row = (int64_t)num_kv_heads * head_size * esz;
  for (int s0 = 0; s0 < num_seqs; s0 += kLdsSeqs) {
    DecodeParams b = a;
    b.num_seqs = num_seqs - s0 < kLdsSeqs ? num_seqs - s0 : kLdsSeqs;
    b.out = (char*)out + s0 * row;
    b.query = (const char*)query + s0 * row;
    b.block_tables = block_tables + (int64_t)s0 * max_blocks_per_seq;
    b.context_lens = context_lens + s0;
    b.new_k = new_key ? (const char*)new_key + s0 * new_row : nullptr;
    b.new_v = new_value ? (const char*)new_value + s0 * new_row : nullptr;
    hipError_t e;
    if (kv_dtype == PKV_FP8_E4M3) {
      e = dtype == PKV_F16 ? dispatch_d<PKV_F16, PKV_FP8_E4M3>(b, head_size, gc, st)
                           : dispatch_d<PKV_BF16, PKV_FP8_E4M3>(b, head_size, gc, st);
    } else {
      switch (dtype) {
        case PKV_F32: e = dispatch_d<PKV_F32, PKV_F32>(b, head_size, gc, st); break;
        case PKV_F16: e = dispatch_d<PKV_F16, PKV_F16>(b, head_size, gc, st); break;
        default: e = dispatch_d<PKV_BF16, PKV_BF16>(b, head_size, gc, st); break;
      }
    }
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // namespace pkv

extern "C" int paged_attention_decode(void* out, const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, float scale,
                                      int num_kv_heads, int num_seqs, int num_heads,
                                      int head_size, int block_size, int max_blocks_per_seq,
                                      int64_t num_blocks, int partition_size, void* workspace,
                                      size_t workspace_bytes, int dtype,
                                      const uint8_t* block_shared, void* stream) {
  return pkv::decode_impl(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                          1.f, 1.f, num_kv_heads, num_seqs, num_heads, head_size, block_size,
                          max_blocks_per_seq, num_blocks, partition_size, workspace,
                          workspace_bytes, dtype, dtype, stream, nullptr, nullptr, false,
                          block_shared);
}

extern "C" int paged_attention_decode_append(
    void* out, const void* query, void* key_cache, void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const void* new_key,
    const void* new_value, float scale, int num_kv_heads, int num_seqs, int num_heads,
    int head_size, int block_size, int max_blocks_per_seq, int64_t num_blocks,
    int partition_size, void* workspace, size_t workspace_bytes, int dtype,
    const uint8_t* block_shared, void* stream) {
  if (!new_key || !new_value) return PKV_ERR_INVALID_ARG;
  return pkv::decode_impl(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                          1.f, 1.f, num_kv_heads, num_seqs, num_heads, head_size, block_size,
                          max_blocks_per_seq, num_blocks, partition_size, workspace,
                          workspace_bytes, dtype, dtype, stream, new_key, new_value, false,
                          block_shared);
}

extern "C" int paged_attention_decode_fp8(void* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          const int32_t* context_lens, float scale,
                                          float k_scale, float v_scale, int num_kv_heads,
                                          int num_seqs, int num_heads, int head_size,
                                          int block_size, int max_blocks_per_seq,
                                          int64_t num_blocks, int partition_size,
                                          void* workspace, size_t workspace_bytes, int dtype,
                                          const uint8_t* block_shared, void* stream) {
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  return pkv::decode_impl(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                          k_scale, v_scale, num_kv_heads, num_seqs, num_heads, head_size,
                          block_size, max_blocks_per_seq, num_blocks, partition_size, workspace,
                          workspace_bytes, dtype, PKV_FP8_E4M3, stream, nullptr, nullptr, false,
                          block_shared);
}

extern "C" int paged_attention_decode_noalloc(void* out, const void* query,
                                              const void* key_cache, const void* value_cache,
                                              const int32_t* block_tables,
                                              const int32_t* context_lens, float scale,
                                              int num_kv_heads, int num_seqs, int num_heads,
                                              int head_size, int block_size,
                                              int max_blocks_per_seq, int64_t num_blocks,
                                              int partition_size, int dtype, void* stream) {
  return pkv::decode_impl(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                          1.f, 1.f, num_kv_heads, num_seqs, num_heads, head_size, block_size,
                          max_blocks_per_seq, num_blocks, partition_size, nullptr, 0, dtype,
                          dtype, stream, nullptr, nullptr, true);
}

extern "C" int paged_attention_decode_append_fp8(
    void* out, const void* query, void* key_cache, void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const void* new_key,
    const void* new_value, float scale, float k_scale, float v_scale, int num_kv_heads,
    int num_seqs, int num_heads, int head_size, int block_size, int max_blocks_per_seq,
    int64_t num_blocks, int partition_size, void* workspace, size_t workspace_bytes, int dtype,
    const uint8_t* block_shared, void* stream) {
  if (!new_key || !new_value) return PKV_ERR_INVALID_ARG;
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  return pkv::decode_impl(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                          k_scale, v_scale, num_kv_heads, num_seqs, num_heads, head_size,
                          block_size, max_blocks_per_seq, num_blocks, partition_size, workspace,
                          workspace_bytes, dtype, PKV_FP8_E4M3, stream, new_key, new_value, false,
                          block_shared);
}
