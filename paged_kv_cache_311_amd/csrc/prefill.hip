// Paged prefill attention for gfx950 (MI355X).
//
// A chunk of new tokens of each sequence -- a whole prompt, or the next
// piece of one after a cached prefix -- attends to the sequence's cached
// tokens through its block table.  The new tokens' keys and values are
// already in the pool (written by reshape_and_cache, as the prompt is
// written into the blocks the runtime assigned: "PagedAttention KV cache
// memory management" [AITJ], "A request lifecycle: allocation, growth,
// sharing and release"); new token i of a sequence of L tokens with n new
// ones sits at position L - n + i and sees tokens 0 .. L - n + i, the
// decoder's masked self-attention (Vaswani et al. 2017, section 3.2.3, and
// eq. 1 for the attention itself).  Keys and values are read through the
// block table as in decoding ("vLLM and PagedAttention" [IV],
// "Architecture, step by step", step 3).
//
// Unlike decoding, many query rows share every key and value: the work is
// a dense contraction and runs on MFMA.
//
// Work decomposition
//   placement = every (sequence, kv head)'s row tiles on one XCD, in a run,
//               so they share its keys and values in that XCD's L2.
//   rows      = (new token, query head of the group) pairs of one
//               (sequence, kv head), token-major: row r is token r / G,
//               head r % G of the group (G = Hq / Hkv).
//   workgroup = 128 rows of one (sequence, kv head): 4 waves x 2 blocks
//               of 16 rows.  It walks the keys 32 at a time (two pool
//               blocks), from token 0 to the last position its rows see.
//   per step  = the 256 threads load the two blocks' K and V tiles
//               straight from the pool into one of three LDS buffers (16 B
//               per lane, no register stage): step s computes from its
//               buffer while step s + 1's tiles land in the next and step
//               s + 2's are issued into the third.  The table entries a step
//               needs are read (scalar loads) one step before its tiles.
//
// Per step and wave (transposed products, so no operand needs a shuffle):
//   S^T = K Q^T  MFMA 16x16x32: A = key rows from LDS as stored, B = the
//                wave's query rows (registers, loaded once).  Lane l gets
//                keys 4(l/16) .. +3 of row l % 16 (and of the second block).
//   softmax      online, in log2 units, per row; a row's 32 values sit in
//                4 lanes (l, l^16, l^32, l^48); masked by select.
//   O^T += V^T P^T  MFMA 16x16x32: B = the probabilities exactly as the
//                QK left them (8 keys per lane: 4 of each block, the k
//                order of both operands permuted alike), A = values read
//                from LDS rows with the transposing 8-byte read, two per
//                lane and 16-dim block.
//                Lane l holds output dims 16j + 4(l/16) .. +3 of row
//                l % 16, so the rescale by the row's running max and the
//                final 1/sum are lane-local.  Each lane sums its own 8
//                probabilities of the row as packed (two-term dot products
//                with ones, into float32), and the row's 4 lanes add their
//                parts once, at the end.
//   Masking selects only on the steps that reach past a wave's earliest
//   row.  A row's max is raised only when a step's exceeds it by 2^8 (so
//   probabilities stay below 256) and the rescale then runs for the wave;
//   each lane tests its own 8 scores first, so the maximum across a row's
//   lanes is taken only on the steps that raise some row's max.
//
// Precision: products accumulate in float32; the probabilities enter the
// second product rounded to the input type (as the values are), and the
// row sums add those same rounded probabilities (in float32), so the
// weights of a row's values sum to one.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {
namespace prefill {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRB = 2;                      // 16-row blocks per wave
constexpr int kRows = kWaves * kRB * 16;    // rows per workgroup
constexpr int kKeys = 2 * kBlockSize;       // tokens per step (two pool blocks)
constexpr int kXcds = 8;                    // accelerator dies (each with its own L2)
// Pairs interleaved per XCD bundle: about 32 row tiles' worth, at least 4
// pairs (measured on one MI355X: 16 pairs of 4 tiles beat both a
// one-pair-at-a-time order and a whole-XCD interleave by 13%; with three
// waves per SIMD, 8 pairs of 4 tiles beat 16 by 3% and 4 or 6 pairs are
// as fast; with 64 tiles per pair, 4 pairs beat 1 by 7%, 2 by 0.4% and 8
// by 1.5%).
constexpr int kBundleTiles = 32;
constexpr int kMinBundle = 4;
// A row's running max is raised only when a step's max exceeds it by more
// than this (log2 units); probabilities then stay below 2^kSlack and the
// accumulator is rescaled rarely.
constexpr float kSlack = 8.f;
// Waves per SIMD: three workgroups per CU (168 VGPRs; 3 x 48 KiB of LDS at
// D = 128).  Measured on one MI355X: 3-5% faster than two, with the value
// reads split in halves to fit.
constexpr int kWavesPerSimd = 3;
// Batches of up to this many sequences are dealt heaviest first (each wave
// of each workgroup, empty ones too, ranks the sequences itself, a lane per
// sequence; the loop over them is the cost).
constexpr int kMaxSortSeqs = 32;
static_assert(kMaxSortSeqs <= kWave, "a lane per sequence");

// LDS: three buffers of K [32 tokens][D] and V [32 tokens][D], rows
// unpadded.  Within a row, the pool row's 16-B chunk c sits at chunk
// c ^ kswz(row) (keys) or c ^ vswz(row) (values), so that the 16 rows of a
// key read, and the 4 rows of a transposing value read, fall on distinct
// banks.
template <int D>
struct Lds {
  static constexpr int kRowB = D * 2;
  static constexpr int kCpr = kRowB / 16;                // 16-B chunks per row
  static constexpr int kRowsPer256 = 256 / kRowB;        // rows per 256 B (64 banks)
  static constexpr int kBuf = kKeys * kRowB;             // one tensor of one step
  static constexpr int kBytes = 6 * kBuf;                // K, V x 3 buffers
  static __device__ __forceinline__ int kswz(int row) { return (row / kRowsPer256) % kCpr; }
  static __device__ __forceinline__ int vswz(int row) { return 2 * ((row % 4) / kRowsPer256); }
};

struct Params {
  void* out;
  const char* query;
  const char* kcache;
  const char* vcache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  float scale_log2;  // |softmax scale| x log2 e, at least 1e-30
  int num_seqs, num_heads, num_kv_heads, max_blocks;
  int64_t num_blocks;
  int row_tiles;     // 128-row tiles per (sequence, kv head) the grid covers
  int bundle;        // (sequence, kv head) pairs interleaved on an XCD
  int sort_seqs;     // deal the pairs in the order of their sequences' work
};



// The two 16-bit values of a word, each made finite where asked: an
// infinity or NaN (exponent all ones) becomes the largest finite value of
// its sign (a NaN's sign bit is ignored: +).
template <int DT>
__device__ __forceinline__ uint32_t finite_pair(uint32_t w, bool lo, bool hi) {
  constexpr uint32_t kExp = DT == PKV_BF16 ? 0x7F80u : 0x7C00u;
  constexpr uint32_t kMax = DT == PKV_BF16 ? 0x7F7Fu : 0x7BFFu;  // largest finite
  const uint32_t a = w & 0xFFFFu, b = w >> 16;
  const bool nan_a = (a & 0x7FFFu) > kExp, nan_b = (b & 0x7FFFu) > kExp;
  const uint32_t fa = (a & kExp) == kExp ? ((nan_a ? 0u : (a & 0x8000u)) | kMax) : a;
  const uint32_t fb = (b & kExp) == kExp ? ((nan_b ? 0u : (b & 0x8000u)) | kMax) : b;
  return (lo ? fa : a) | ((hi ? fb : b) << 16);
}

// A sequence's chunk: its first row, its new tokens, its context length.
struct SeqInfo {
  int s, q0, n, L;
};

// The sequence of rank r when the sequences are ordered by their work (new
// tokens x average keys they see, heaviest first; ties by index), and its
// chunk.  Each wave ranks on its own, lane t holding sequence t (at most
// one wave's worth of sequences), so no LDS or barrier is involved, and
// the chunk of the chosen sequence comes from the lane that loaded it.
__device__ __forceinline__ SeqInfo seq_of_rank(const Params& p, int r) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool in = lane < p.num_seqs;
  int q0 = 0, n = 0, L = 0;
  if (in) {
    q0 = p.query_start_loc[lane];
    n = p.query_start_loc[lane + 1] - q0;
    L = p.context_lens[lane];
  }
  const int max_tokens = p.max_blocks * kBlockSize;
  const float nn = (float)(n > 0 ? n : 0);
  const float lc = (float)(L < 0 ? 0 : (L > max_tokens ? max_tokens : L));
  const float wt = nn * (2.f * lc - nn);
  int rank = 0;
  for (int u = 0; u < p.num_seqs; ++u) {
    const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), u));
    rank += (wu > wt || (wu == wt && u < lane)) ? 1 : 0;
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(in && rank == r);
  const int s = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
  return SeqInfo{s, __builtin_amdgcn_readlane(q0, s), __builtin_amdgcn_readlane(n, s),
                 __builtin_amdgcn_readlane(L, s)};
}

// c + the two 16-bit values of w (float32 sum)
template <int DT>
__device__ __forceinline__ float dot2_ones(uint32_t w, float c) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  if constexpr (DT == PKV_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), __builtin_bit_cast(h2, 0x3C003C00u), c,
                                  false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w),
                                           __builtin_bit_cast(b2, 0x3F803F80u), c, false);
}

// a buffer index as a type (for the unrolled copies of a step)
template <int P>
struct Phase {
  static constexpr int value = P;
};

// Whether any of the eight 16-bit values of a 16-B chunk is an infinity or
// NaN: a value's exponent field plus its lowest bit carries into the
// value's top bit exactly when the field is all ones.
template <int DT>
__device__ __forceinline__ bool nonfinite_any(u32x4 v) {
  constexpr uint32_t kExp = DT == PKV_BF16 ? 0x7F807F80u : 0x7C007C00u;
  constexpr uint32_t kLow = DT == PKV_BF16 ? 0x00800080u : 0x04000400u;
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) c |= (v[i] & kExp) + kLow;
  return (c & 0x80008000u) != 0;
}

template <int DT, int D, bool kNeg>
__global__ __launch_bounds__(kThreads, kWavesPerSimd) void paged_prefill_kernel(const Params p) {
  using LD = Lds<D>;
  constexpr int NKS = D / 32;                    // QK k-steps of 32 dims
  constexpr int NDB = D / 16;                    // output blocks of 16 dims
  constexpr int CPR = D / 8;                     // 16-B chunks per token row
  __shared__ __attribute__((aligned(16))) char lds[LD::kBytes];

  // workgroup -> (sequence, kv head, row tile).  Workgroups are dealt to
  // the 8 XCDs round-robin; every (sequence, kv head) belongs to one XCD.
  // On an XCD, its pairs are taken `bundle` at a time, and within a bundle
  // the row tiles go out latest (heaviest) first across its pairs: the
  // tiles that run together share their keys and values in that XCD's L2,
  // and the longest ones start first.  With sort_seqs, the pairs are dealt
  // in the order of their sequences' work, heaviest first, so the longest
  // workgroups of the whole grid start first (a batch of prompts of mixed
  // lengths otherwise ends on a tail of long workgroups).
  const int xcd = blockIdx.x & (kXcds - 1);
  const int k = blockIdx.x / kXcds;
  const int per_bundle = p.bundle * p.row_tiles;
  const int bdl = k / per_bundle;
  const int in_b = k - bdl * per_bundle;
  const int rank = in_b / p.bundle;
  const int sg = ((bdl * p.bundle + (in_b - rank * p.bundle)) * kXcds) + xcd;
  if (sg >= p.num_seqs * p.num_kv_heads) return;  // padding of the grid
  const int vs = sg / p.num_kv_heads;  // the sequence's place in the dealing order
  const int g = sg - vs * p.num_kv_heads;
  SeqInfo si;
  if (p.sort_seqs) {
    si = seq_of_rank(p, vs);
  } else {
    si.s = vs;
    si.q0 = p.query_start_loc[vs];
    si.n = p.query_start_loc[vs + 1] - si.q0;
    si.L = p.context_lens[vs];
  }
  const int s = si.s;
  const int tile = p.row_tiles - 1 - rank;

  const int G = p.num_heads / p.num_kv_heads;
  const int q0 = si.q0;
  const int n = si.n;
  const int rows = n * G;
  const int R0 = tile * kRows;
  if (n <= 0 || R0 >= rows) return;  // uniform per workgroup
  const int max_tokens = p.max_blocks * kBlockSize;
  int Lc = si.L;
  Lc = Lc < 0 ? 0 : (Lc > max_tokens ? max_tokens : Lc);
  const int base = Lc - n;  // position of the chunk's first token
  const int last_row = min(rows - 1, R0 + kRows - 1);
  const int nkv = min(base + last_row / G + 1, Lc);  // tokens this workgroup reads
  const int nsteps = nkv > 0 ? (nkv + kKeys - 1) / kKeys : 0;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;

  // this lane's rows (one per 16-row block) and their query operands.  A
  // negative scale is carried by the queries (kNeg: their signs flipped),
  // so that the softmax works with a positive one and a row's largest score
  // is its largest scaled logit.
  constexpr uint32_t qsign = kNeg ? 0x80008000u : 0u;
  u32x4 q[kRB][NKS];
  int pos[kRB];
  int64_t row_off[kRB];  // element offset of the row in query / out
  bool row_ok[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int r = R0 + (w * kRB + rb) * 16 + col;
    row_ok[rb] = r < rows;
    const int rc = row_ok[rb] ? r : rows - 1;
    const int i = rc / G;
    pos[rb] = base + i;
    row_off[rb] = ((int64_t)(q0 + i) * p.num_heads + g * G + (rc - i * G)) * D;
#pragma unroll
    for (int m = 0; m < NKS; ++m)
      q[rb][m] = row_ok[rb] ? load16(p.query + (row_off[rb] + 32 * m + 8 * grp) * 2) ^ qsign
                            : u32x4{0u, 0u, 0u, 0u};
  }

  // Tiles go from the pool straight into LDS (global_load_lds, 16 B per
  // lane): each wave instruction fills 1 KiB of one buffer, whole token
  // rows of one pool block, lane l taking the LDS slot l (row l / CPR of the
  // KiB, chunk l % CPR) and reading the pool chunk the swizzle puts there.
  // A wave's KiBs of a step lie in one pool block, so it needs one block id
  // per step (read from the table with a scalar load a step before use).
  constexpr int kTileBytes = kBlockSize * D * 2;
  constexpr int kRowsPerKiB = 1024 / LD::kRowB;
  constexpr int kDma = kKeys * LD::kRowB / 1024 / kWaves;  // KiBs per wave per tensor
  static_assert(kDma * kWaves * 1024 == kKeys * LD::kRowB, "whole KiBs per wave");
  static_assert(kDma * kRowsPerKiB <= kBlockSize, "a wave's rows in one pool block");
  const int64_t blk_bytes = (int64_t)p.num_kv_heads * kTileBytes;
  const int64_t head_bytes = (int64_t)g * kTileBytes;
  const int32_t* table = p.block_tables + (int64_t)s * p.max_blocks;
  const int row_w0 = w * kDma * kRowsPerKiB;      // the wave's first row of a step
  const int dma_half = row_w0 / kBlockSize;       // its pool block of the step's two
  uint32_t ksrc[kDma], vsrc[kDma];                // pool byte offsets inside the tile
#pragma unroll
  for (int u = 0; u < kDma; ++u) {
    const int row = row_w0 + u * kRowsPerKiB + lane / CPR;
    const int ch = lane % CPR;
    ksrc[u] = (uint32_t)((row % kBlockSize) * LD::kRowB + (ch ^ LD::kswz(row)) * 16);
    vsrc[u] = (uint32_t)((row % kBlockSize) * LD::kRowB + (ch ^ LD::vswz(row)) * 16);
  }
  const int nblk = (Lc + kBlockSize - 1) / kBlockSize;
  // The table is read with scalar loads (the address is the same for the
  // whole wave); their waits share the LDS counter, and each falls at the
  // head of a step, where no LDS operation is in flight.
  const __attribute__((address_space(4))) int32_t* ctab =
      (const __attribute__((address_space(4))) int32_t*)table;
  // the block id of the wave's rows of a step (blocks past the context:
  // the sequence's first block, a table entry of the context)
  auto read_id = [&](int step) __attribute__((always_inline)) -> int {
    const int bi = step * (kKeys / kBlockSize) + dma_half;
    return ctab[bi < nblk ? bi : 0];
  };
  const int max_blk = (int)(p.num_blocks - 1);
  char* const lds_k = lds;
  char* const lds_v = lds + 3 * LD::kBuf;
  const uint32_t lds_k_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_k;
  const uint32_t lds_v_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_v;
  // The wave's KiBs of a step into buffer buf.  The loads are written out
  // (M0 = the KiB's LDS address, one wait state after writing it), so that
  // the compiler counts no LDS write in them: it would otherwise hold every
  // transposing LDS read until all such loads in flight had landed, the
  // next steps' too.  The waits that order them are the explicit ones below.
  auto dma = [&](int id, int buf) __attribute__((always_inline)) {
    const int64_t b = min(max(id, 0), max_blk);  // clamped into the pool
    const char* kt = p.kcache + b * blk_bytes + head_bytes;
    const char* vt = p.vcache + b * blk_bytes + head_bytes;
#pragma unroll
    for (int u = 0; u < kDma; ++u) {
      const uint32_t kib = (uint32_t)((w * kDma + u) * 1024 + buf * LD::kBuf);
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :
                   : "v"(ksrc[u]), "s"(kt), "{m0}"(lds_k_addr + kib)
                   : "memory");
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :
                   : "v"(vsrc[u]), "s"(vt), "{m0}"(lds_v_addr + kib)
                   : "memory");
    }
  };
  // Once a step's tiles have landed: on the steps that mask keys for some
  // row of the workgroup (or reach past the context), each lane makes its
  // own slots safe.  A masked probability is an exact zero, but the second
  // product still meets the value it multiplies (0 x inf = NaN): tokens past
  // the context become zeros, whatever the slot read in their place holds,
  // and the non-finite values of keys past the workgroup's earliest row
  // become the largest finite value of their sign (NaN: +).  Rows that do
  // not see such a key are then exact; rows that see a non-finite value
  // there get that largest value in its place.
  const int wg_pos0 = base + R0 / G;  // position of the workgroup's earliest row
  // The test for a non-finite value comes first (a few instructions); the
  // clamp and its write run only where one was found.
  auto fixup = [&](int buf, int step) __attribute__((always_inline)) {
    const bool edge = step * kKeys + kKeys - 1 > wg_pos0;  // uniform
    const bool tail = step * kKeys + kKeys > Lc;           // uniform
    if (!edge && !tail) return;
#pragma unroll
    for (int u = 0; u < kDma; ++u) {
      const int kib = w * kDma + u;
      const int t = step * kKeys + row_w0 + u * kRowsPerKiB + lane / CPR;
      char* ks = lds_k + buf * LD::kBuf + kib * 1024 + lane * 16;
      char* vs = lds_v + buf * LD::kBuf + kib * 1024 + lane * 16;
      if (edge) {
        u32x4 vv = *reinterpret_cast<const u32x4*>(vs);
        const bool bad = nonfinite_any<DT>(vv) && t > wg_pos0;
        if (__builtin_amdgcn_ballot_w64(bad)) {
          if (bad) {
#pragma unroll
            for (int i = 0; i < 4; ++i) vv[i] = finite_pair<DT>(vv[i], true, true);
            *reinterpret_cast<u32x4*>(vs) = vv;
          }
        }
      }
      if (tail && t >= Lc) {
        const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(ks) = zero;
        *reinterpret_cast<u32x4*>(vs) = zero;
      }
    }
  };
  // Waits written out, so that no memory access moves across them: a
  // step's tiles have landed while the 2 kDma loads of the next step's
  // (issued after them) stay in flight; where no later loads were issued
  // (the last steps), all loads have landed.  A step's LDS writes are then
  // published by a barrier (lgkmcnt(0) first: this wave's LDS operations
  // done).
  auto wait_tiles = []() __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kDma) : "memory");
  };
  auto wait_loads = []() __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  auto publish = []() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // running max in log2 units, floored at -1e30 so that a row with nothing
  // visible yet keeps alpha = 1 and p = 0 (no infinity minus infinity)
  float m_run[kRB];
  float m_thr[kRB];  // m_run + kSlack
  floatx4 acc[kRB][NDB];
  float lsum[kRB];  // the lane's part of its row's sum of probabilities
  const float c2 = p.scale_log2;
  const int wave_pos0 = base + min(R0 + w * kRB * 16, rows - 1) / G;  // earliest row of the wave
  // the wave's latest row: steps that start past it are masked for all its
  // rows, and the wave only takes its part in their loads
  const int wave_pos1 = base + min(R0 + (w + 1) * kRB * 16 - 1, rows - 1) / G;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_run[rb] = -1e30f;
    m_thr[rb] = m_run[rb] + kSlack;
    lsum[rb] = 0.f;
#pragma unroll
    for (int j = 0; j < NDB; ++j) acc[rb][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // Three steps in flight, in three buffers: step s is computed from buffer
  // s % 3 while step s + 1's tiles land in the next and step s + 2's are
  // issued into the third (the one step s - 1 was computed from).
  int id_n = 0;  // block id of step s + 2, read during step s - 1
  // The loop is unrolled by the three buffers, so that each copy's buffer
  // offsets are constants (folded into the LDS instructions' offsets).
  auto body = [&](int step, auto phase) __attribute__((always_inline)) {
    constexpr int bcur = decltype(phase)::value;
    constexpr int bnxt = (bcur + 1) % 3;
    constexpr int bfar = (bcur + 2) % 3;
    const int id_nn = read_id(step + 3);
    // (no loads for steps past the last: a wave would wait for them before
    // it ends, and its workgroup's slot would stay taken meanwhile)
    const bool issue = step + 2 < nsteps;
    if (issue) dma(id_n, bfar);
    if (step * kKeys <= wave_pos1) {
      const char* kb = lds_k + bcur * LD::kBuf;
      const char* vb = lds_v + bcur * LD::kBuf;

      // S^T for both key blocks and both row blocks, one key block's
      // operands (read from LDS together) at a time
      floatx4 sc[kRB][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 ka[NKS];
        const int r = h * 16 + col;
#pragma unroll
        for (int m = 0; m < NKS; ++m)
          ka[m] = load16(kb + r * LD::kRowB + ((4 * m + grp) ^ LD::kswz(r)) * 16);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) sc[rb][h] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NKS; ++m) {
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) sc[rb][h] = mfma32<DT>(ka[m], q[rb][m], sc[rb][h]);
        }
      }

      // The value operands, read transposed: lane l gets dim 16j + l % 16 of
      // tokens 4(l/16) + 0..3 of each block (the probabilities' k order).
      // Dim block j = jl + kT jh sits at chunk 2 (jl ^ t) + 2 kT jh (+1 for
      // the lane's upper 8 dims): kT lane addresses, the rest offsets; the
      // second block's rows (16 on) have the same swizzle.  The first half is
      // read while the softmax runs, the second after the first half's
      // products (the registers of both halves at once would not leave room
      // for three waves per SIMD).
      u32x4 va[NDB];
      constexpr int kT = 4 / LD::kRowsPer256;  // distinct swizzles of the rows
      static_assert(NDB % kT == 0 && NDB % 2 == 0, "dim blocks in whole swizzle periods");
      const int r0 = 4 * grp + (col >> 2);
      const char* vrow =
          vb + r0 * LD::kRowB + (col & 1) * 8 + ((col & 3) >> 1) * 16;
      const int vt = LD::vswz(r0) / 2;
      auto read_v = [&](int j) __attribute__((always_inline)) {
        const char* a = vrow + 32 * ((j % kT) ^ vt) + 32 * kT * (j / kT);
        const uint2 lo = read_tr16(a);
        const uint2 hi = read_tr16(a + 16 * LD::kRowB);
        va[j] = u32x4{lo.x, lo.y, hi.x, hi.y};
      };
#pragma unroll
      for (int j = 0; j < NDB / 2; ++j) read_v(j);
      __builtin_amdgcn_sched_barrier(0);

      // online softmax per row; probabilities packed as the B operand of PV.
      // Steps that end at or before the wave's earliest row need no mask.
      const bool masked = step * kKeys + kKeys - 1 > wave_pos0;
      u32x4 pb[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        float x[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int i = 0; i < 4; ++i) x[h * 4 + i] = sc[rb][h][i];
        }
        if (masked) {
          // key e of the lane is token step kKeys + 4 grp + (e / 4) 16 + e % 4
          const int d = pos[rb] - 4 * grp - step * kKeys;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (e >> 2) * 16 + (e & 3) <= d ? x[e] : -INFINITY;
        }
        // The lane's own maximum decides whether its row's max may need
        // raising (the row's running max is the same in its four lanes); only
        // then is the row's maximum taken across them.
        float mt = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, x[e]);
        if (__builtin_amdgcn_ballot_w64(mt * c2 > m_thr[rb])) {  // rescale some rows
          const float m_tile = max4rows(mt) * c2;
          const bool grow = m_tile > m_thr[rb];
          const float m_new = grow ? m_tile : m_run[rb];
          const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
          m_run[rb] = m_new;
          m_thr[rb] = m_new + kSlack;
          lsum[rb] *= alpha;
#pragma unroll
          for (int j = 0; j < NDB; ++j) acc[rb][j] *= alpha;
        }
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(x[e], c2, -m_run[rb]));
#pragma unroll
        for (int e = 0; e < 4; ++e) pb[rb][e] = pack2<DT>(pe[2 * e], pe[2 * e + 1]);
      }

      // O^T += V^T P^T, one 16-dim block at a time
#pragma unroll
      for (int j = 0; j < NDB; ++j) {
        if (j == NDB / 2) {
#pragma unroll
          for (int jj = NDB / 2; jj < NDB; ++jj) read_v(jj);
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) acc[rb][j] = mfma32<DT>(va[j], pb[rb], acc[rb][j]);
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lsum[rb] = dot2_ones<DT>(pb[rb][e], lsum[rb]);
      }
    }

    // step + 1's tiles have landed (step + 2's, issued after them, stay in
    // flight); made safe where needed, then published
    __builtin_amdgcn_sched_barrier(0);
    if (issue)
      wait_tiles();
    else
      wait_loads();  // nothing issued after step + 1's tiles
    fixup(bnxt, step + 1);
    id_n = id_nn;
    publish();
  };

  if (nsteps > 0) {
    // steps 0 and 1 issued as the loop would, step 0's waited for
    const int id0 = read_id(0);
    const int id1 = read_id(1);
    dma(id0, 0);
    id_n = read_id(2);
    if (nsteps > 1) {
      dma(id1, 1);
      wait_tiles();
    } else {
      wait_loads();
    }
    fixup(0, 0);
  }
  // the queries have arrived (a wait the compiler sees, on either path, so
  // that it adds none for them inside the loop)
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  publish();
  int step = 0;
  for (; step + 3 <= nsteps; step += 3) {
    body(step, Phase<0>{});
    body(step + 1, Phase<1>{});
    body(step + 2, Phase<2>{});
  }
  if (step < nsteps) body(step, Phase<0>{});
  if (step + 1 < nsteps) body(step + 1, Phase<1>{});

  // normalize and store: lane l holds dims 16j + 4(l/16) .. +3 of its row
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float l = sum4rows(lsum[rb]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (row_ok[rb]) {
      char* dst = (char*)p.out + (row_off[rb] + 4 * grp) * 2;
#pragma unroll
      for (int j = 0; j < NDB; ++j) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const floatx4 o = acc[rb][j];
        const float o0 = o[0] * inv, o1 = o[1] * inv, o2 = o[2] * inv, o3 = o[3] * inv;
        *reinterpret_cast<u32x2*>(dst + 16 * j * 2) = u32x2{pack2<DT>(o0, o1), pack2<DT>(o2, o3)};
      }
    }
  }
}

template <int DT, int D>
static hipError_t launch(const Params& a, bool neg, unsigned grid, hipStream_t st) {
  if (neg)
    hipLaunchKernelGGL((paged_prefill_kernel<DT, D, true>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((paged_prefill_kernel<DT, D, false>), dim3(grid), dim3(kThreads), 0, st,
                       a);
  return hipGetLastError();
}

}  // namespace prefill
}  // namespace pkv

extern "C" int paged_attention_prefill(void* out, const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       const int32_t* context_lens,
                                       const int32_t* query_start_loc, float scale,
                                       int num_kv_heads, int num_seqs, int num_heads,
                                       int head_size, int block_size, int max_blocks_per_seq,
                                       int64_t num_blocks, int max_query_len, int dtype,
                                       void* stream) {
  using namespace pkv;
  using namespace pkv::prefill;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !query_start_loc)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || num_blocks > INT32_MAX || max_query_len < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (!(fabsf(scale) <= 3.402823466e38f)) return PKV_ERR_INVALID_ARG;  // NaN, +-inf
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PKV_ERR_UNSUPPORTED;
  if (((uintptr_t)query | (uintptr_t)key_cache | (uintptr_t)value_cache) & 15u)
    return PKV_ERR_INVALID_ARG;  // 16-byte loads
  if ((uintptr_t)out & 7u) return PKV_ERR_INVALID_ARG;  // 8-byte stores
  if (num_seqs == 0 || max_query_len == 0) return PKV_OK;
  const int64_t rows = (int64_t)max_query_len * (num_heads / num_kv_heads);
  const int64_t row_tiles = (rows + kRows - 1) / kRows;
  const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
  const int64_t per_xcd = (pairs + kXcds - 1) / kXcds;
  int64_t bundle = kBundleTiles / row_tiles;
  bundle = bundle < kMinBundle ? kMinBundle : bundle;
  bundle = bundle > per_xcd ? per_xcd : bundle;
  const int64_t grid = row_tiles * ((per_xcd + bundle - 1) / bundle) * bundle * kXcds;
  if (row_tiles > INT32_MAX || grid > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_query_len * num_heads > INT32_MAX / 2) return PKV_ERR_INVALID_ARG;
  if ((int64_t)num_kv_heads * kBlockSize * head_size * 2 > (int64_t)UINT32_MAX)
    return PKV_ERR_INVALID_ARG;  // bytes of one block, all kv heads
  Params a;
  a.out = out;
  a.query = (const char*)query;
  a.kcache = (const char*)key_cache;
  a.vcache = (const char*)value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  // exp(x) = 2^(x log2 e).  The kernel takes the scale's magnitude and its
  // sign apart (a negative scale flips the queries' signs); a zero scale is
  // taken as 1e-30, which weighs the visible tokens equally to float32
  // precision as zero does, while a masked score, -inf, still scales to -inf.
  const float scale_log2 = scale * 1.4426950408889634f;
  const bool neg = scale_log2 < 0.f;
  a.scale_log2 = fmaxf(fabsf(scale_log2), 1e-30f);
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.row_tiles = (int)row_tiles;
  a.bundle = (int)bundle;
  a.sort_seqs = num_seqs <= kMaxSortSeqs ? 1 : 0;
  (void)hipGetLastError();
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dtype == PKV_F16)
    e = head_size == 64 ? launch<PKV_F16, 64>(a, neg, (unsigned)grid, st)
                        : launch<PKV_F16, 128>(a, neg, (unsigned)grid, st);
  else
    e = head_size == 64 ? launch<PKV_BF16, 64>(a, neg, (unsigned)grid, st)
                        : launch<PKV_BF16, 128>(a, neg, (unsigned)grid, st);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
