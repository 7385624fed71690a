// Decode attention for batches whose sequences share prompt blocks, for
// gfx950 (MI355X).
//
// Sequences forked from one prompt (parallel samples, beams) map the
// prompt's full blocks to the same physical blocks: a forked table points
// at the parent's blocks and each block counts its sharers ([TEQ] "Paging's
// second gift: copy-on-write"; [AITJ] "How logical blocks, physical blocks
// and the block table work").  paged_attention_decode reads such a block
// once per sequence.  Here the caller names the groups of sequences that
// share leading blocks, and each shared tile (block, kv head) is read once
// for the query rows of every member of its group; each sequence's own
// blocks after the shared ones are read for that sequence alone.  The
// result is the same attention ([VAS] eq. 1 over each sequence's context),
// as an exact float32 merge of the pieces.
//
// Work items (a wave each, taken in turn by every wave of a persistent
// grid):
//   prefix item = (group j, kv head g, row set rs, chunk c): its rows are
//                 the (member, query head of g) pairs 16 rs .. 16 rs + 15 of
//                 the group (member-major), its tiles the shared blocks
//                 kChunk c .. kChunk (c + 1) - 1 of the group's first
//                 member's table;
//   suffix item = (sequence s, kv head g, row set rs, chunk c): its rows are
//                 the query heads 16 rs .. of g, its tiles the sequence's
//                 blocks after its group's shared ones, kChunk at a time.
// A group's shared blocks are the caller's count, clamped to the full
// blocks every member holds, so every shared tile is whole.  Each item
// leaves one float32 state per row (running max in log2 units, sum,
// unnormalized output) at (sequence, head, piece): the prefix chunks come
// first, then the suffix chunks.  The combine kernel merges each row's
// pieces into its output.
//
// Per tile, both products run on the matrix cores as in the decode
// kernel's grouped path: S^T = K Q^T with the key tile as loaded and the
// item's query rows on the 16 lane columns, a lane-local online softmax,
// and O^T += V^T P^T with the values staged as rows in LDS and read back
// transposed.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "pkv_device.h"

namespace pkv {
namespace shared_prefix {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxSeqs = 2048;            // sequences (and groups) per call
constexpr int kChunk = 8;                 // tiles per work item
constexpr int kRowsPerItem = 16;          // query rows per item (MFMA columns)
constexpr int kWavesPerSimd = 2;
constexpr float kSlack = 8.f;             // running max raised past this (log2 units)

struct Params {
  void* out;
  const char* query;
  const char* kcache;
  const char* vcache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* order;          // position -> sequence (NULL: the identity)
  const int32_t* group_start;
  const int32_t* prefix_blocks;
  int2* pieces;        // per sequence: (prefix pieces, suffix pieces)
  float* state_ml;     // [seq][head][piece][2]
  float* state_acc;    // [seq][head][piece][D]
  float scale_log2;    // softmax scale x log2 e
  int num_seqs, num_groups, num_heads, num_kv_heads, group, max_blocks, max_pieces;
  int64_t num_blocks;
};

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// The call's work plan, built in every workgroup's LDS from the lengths
// and the group description.
struct Plan {
  int gs[kMaxSeqs + 1];   // group starts, clamped into [0, num_seqs]
  int pb[kMaxSeqs];       // shared blocks per group (clamped)
  int gincl[kMaxSeqs];    // prefix items, inclusive running sum over groups
  int seq[kMaxSeqs];      // sequence at each position (the order, clamped)
  int len[kMaxSeqs];      // context lengths by position, clamped
  int grp[kMaxSeqs];      // group of each position, or -1
  int sincl[kMaxSeqs];    // suffix items, inclusive running sum over positions
  int scan[kThreads];
};

// Inclusive running sum of v[0..n) in place (every thread of the
// workgroup calls it).
__device__ void block_scan(int* v, int n, int* tmp) {
  const int tid = threadIdx.x;
  const int per = ceil_div(n, kThreads);
  const int b = tid * per, e = min(b + per, n);
  int sum = 0;
  for (int i = b; i < e; ++i) sum += v[i];
  tmp[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  int run = tid > 0 ? tmp[tid - 1] : 0;
  for (int i = b; i < e; ++i) {
    run += v[i];
    v[i] = run;
  }
  __syncthreads();
}

// Index of the entry x falls in: the first i with incl[i] > x.
__device__ __forceinline__ int search(const int* incl, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (incl[mid] > x) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

template <int D>
__device__ void build_plan(const Params& p, Plan& pl) {
  const int tid = threadIdx.x;
  const int ns = p.num_seqs, ng = p.num_groups;
  const int max_tokens = p.max_blocks * kBlockSize;
  for (int s = tid; s < ns; s += kThreads) {
    int q = p.order != nullptr ? p.order[s] : s;
    q = q < 0 ? 0 : (q >= ns ? ns - 1 : q);
    pl.seq[s] = q;
    const int L = p.context_lens[q];
    pl.len[s] = L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
  }
  for (int j = tid; j <= ng; j += kThreads) {
    const int g = p.group_start[j];
    pl.gs[j] = g < 0 ? 0 : (g > ns ? ns : g);
  }
  for (int j = tid; j < ng; j += kThreads) {
    const int b = p.prefix_blocks[j];
    pl.pb[j] = b < 0 ? 0 : (b > p.max_blocks ? p.max_blocks : b);
  }
  __syncthreads();
  // a sequence's group: the last j with gs[j] <= s, if s < gs[j + 1]; the
  // group's shared blocks at most the full blocks of each member
  for (int s = tid; s < ns; s += kThreads) {
    int j = -1;
    if (ng > 0) {
      int lo = 0, hi = ng - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pl.gs[mid] <= s) lo = mid;
        else hi = mid - 1;
      }
      if (pl.gs[lo] <= s && s < pl.gs[lo + 1]) j = lo;
    }
    pl.grp[s] = j;
    if (j >= 0) atomicMin(&pl.pb[j], pl.len[s] / kBlockSize);
  }
  __syncthreads();
  const int hkv = p.num_kv_heads, G = p.group;
  for (int j = tid; j < ng; j += kThreads) {
    const int members = max(pl.gs[j + 1] - pl.gs[j], 0);
    pl.gincl[j] = members > 0 && pl.pb[j] > 0
                      ? hkv * ceil_div(members * G, kRowsPerItem) * ceil_div(pl.pb[j], kChunk)
                      : 0;
  }
  for (int s = tid; s < ns; s += kThreads) {
    const int j = pl.grp[s];
    const int pb = j >= 0 ? pl.pb[j] : 0;
    const int suf = ceil_div(pl.len[s], kBlockSize) - pb;
    pl.sincl[s] = hkv * ceil_div(G, kRowsPerItem) * ceil_div(suf, kChunk);
    if (blockIdx.x == 0) p.pieces[pl.seq[s]] = int2{ceil_div(pb, kChunk), ceil_div(suf, kChunk)};
  }
  __syncthreads();
  if (ng > 0) block_scan(pl.gincl, ng, pl.scan);
  block_scan(pl.sincl, ns, pl.scan);
}

// One work item, as a wave sees it.
struct Item {
  int g;          // kv head
  int tseq;       // sequence whose table holds the tiles
  int n0, n1;     // blocks [n0, n1) of that table
  int last_valid; // tokens of block n1 - 1 (16 but in a sequence's last block)
  int piece;      // piece index of every row's state
  int nrows;      // rows (1..16)
  int seq_r, head_r;  // lane column's row (rows past nrows: row 0's)
};

__device__ __forceinline__ Item item_of(const Params& p, const Plan& pl, int x, int P, int col) {
  Item it;
  const int hkv = p.num_kv_heads, G = p.group;
  int r;  // this lane column's row within the item
  if (x < P) {
    const int j = search(pl.gincl, p.num_groups, x);
    const int local = x - (j > 0 ? pl.gincl[j - 1] : 0);
    const int members = pl.gs[j + 1] - pl.gs[j];
    const int rows = members * G;
    const int rsets = ceil_div(rows, kRowsPerItem);
    const int chunks = ceil_div(pl.pb[j], kChunk);
    it.g = local / (rsets * chunks);
    const int rem = local - it.g * rsets * chunks;
    const int rs = rem / chunks;
    const int c = rem - rs * chunks;
    it.tseq = pl.seq[pl.gs[j]];
    it.n0 = c * kChunk;
    it.n1 = min(it.n0 + kChunk, pl.pb[j]);
    it.last_valid = kBlockSize;
    it.piece = c;
    it.nrows = min(kRowsPerItem, rows - rs * kRowsPerItem);
    r = rs * kRowsPerItem + (col < it.nrows ? col : 0);
    it.seq_r = pl.seq[pl.gs[j] + r / G];
    it.head_r = it.g * G + r % G;
  } else {
    const int y = x - P;
    const int pos = search(pl.sincl, p.num_seqs, y);
    const int s = pl.seq[pos];
    const int local = y - (pos > 0 ? pl.sincl[pos - 1] : 0);
    const int j = pl.grp[pos];
    const int pb = j >= 0 ? pl.pb[j] : 0;
    const int nb = ceil_div(pl.len[pos], kBlockSize);
    const int rsets = ceil_div(G, kRowsPerItem);
    const int chunks = ceil_div(nb - pb, kChunk);
    it.g = local / (rsets * chunks);
    const int rem = local - it.g * rsets * chunks;
    const int rs = rem / chunks;
    const int c = rem - rs * chunks;
    it.tseq = s;
    it.n0 = pb + c * kChunk;
    it.n1 = min(it.n0 + kChunk, nb);
    it.last_valid = it.n1 == nb ? pl.len[pos] - (nb - 1) * kBlockSize : kBlockSize;
    it.piece = ceil_div(pb, kChunk) + c;
    it.nrows = min(kRowsPerItem, G - rs * kRowsPerItem);
    r = rs * kRowsPerItem + (col < it.nrows ? col : 0);
    it.seq_r = s;
    it.head_r = it.g * G + r;
  }
  // the same in every lane but the row: known uniform from here on
  it.g = __builtin_amdgcn_readfirstlane(it.g);
  it.tseq = __builtin_amdgcn_readfirstlane(it.tseq);
  it.n0 = __builtin_amdgcn_readfirstlane(it.n0);
  it.n1 = __builtin_amdgcn_readfirstlane(it.n1);
  it.last_valid = __builtin_amdgcn_readfirstlane(it.last_valid);
  it.piece = __builtin_amdgcn_readfirstlane(it.piece);
  it.nrows = __builtin_amdgcn_readfirstlane(it.nrows);
  return it;
}

template <int D>
struct Cfg {
  static constexpr int kRowB = D * 2;              // bytes per token row
  static constexpr int kTileB = kBlockSize * kRowB;
  static constexpr int kNld = kTileB / 1024;       // 16-B loads per lane per tile
  static constexpr int kNch = kRowB / 16;          // 16-B chunks per row
  static constexpr int kTpl = kWave / kNch;        // tokens per 1-KiB value load
  static constexpr int kNq = D / 32;               // MFMA k-steps per logit chain
  static constexpr int kNdb = D / 16;              // 16-dim output blocks
  static constexpr int kVS = D * 2 + 32;           // LDS value row stride
  static_assert(kNq == kNld, "one key chunk per k-step");
};

template <int D>
struct Tile {
  u32x4 k[Cfg<D>::kNld], v[Cfg<D>::kNld];
};

template <int DT, int D>
__global__ __launch_bounds__(kThreads, kWavesPerSimd) void shared_prefix_rows_kernel(
    const Params p) {
  using C = Cfg<D>;
  __shared__ Plan pl;
  __shared__ __attribute__((aligned(16))) char sm_v[kWaves][kBlockSize * C::kVS];
  build_plan<D>(p, pl);
  const int P = p.num_groups > 0 ? pl.gincl[p.num_groups - 1] : 0;
  const int total = P + pl.sincl[p.num_seqs - 1];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;   // lane column: the item's row
  const int jg = lane >> 4;    // lane group
  const int nwaves = gridDim.x * kWaves;
  char* const sv = sm_v[w];
  const int64_t block_stride = (int64_t)p.num_kv_heads * C::kTileB;
  const uint32_t koff = (uint32_t)(col * C::kRowB + jg * 16);
  const uint32_t voff = (uint32_t)(lane * 16);

  // tile n of the item: its block id sits in lane n - n0 of `ids`
  auto load_tile = [&](Tile<D>& t, const Item& it, int ids, int n) {
    const int64_t b = __builtin_amdgcn_readlane(ids, n - it.n0);
    const int64_t off = b * block_stride + (int64_t)it.g * C::kTileB;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.kcache + off, C::kTileB);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(p.vcache + off, C::kTileB);
#pragma unroll
    for (int m = 0; m < C::kNld; ++m) t.k[m] = load16_buffer<kCacheDefault>(kr, koff + m * 64);
#pragma unroll
    for (int m = 0; m < C::kNld; ++m) t.v[m] = load16_buffer<kCacheDefault>(vr, voff + m * 1024);
  };

  for (int x = blockIdx.x * kWaves + w; x < total; x += nwaves) {
    const Item it = item_of(p, pl, x, P, col);
    // the item's block ids (at most kChunk), one per lane, clamped into the pool
    int ids = 0;
    if (lane < it.n1 - it.n0) {
      const int b = p.block_tables[(int64_t)it.tseq * p.max_blocks + it.n0 + lane];
      ids = b < 0 ? 0 : (b >= p.num_blocks ? (int)(p.num_blocks - 1) : b);
    }
    // the lane column's query row: k-step m reads dims 32m + 8 jg .. +7
    u32x4 q[C::kNq];
    const char* qrow = p.query + ((int64_t)it.seq_r * p.num_heads + it.head_r) * C::kRowB;
#pragma unroll
    for (int m = 0; m < C::kNq; ++m) q[m] = load16(qrow + (jg + 4 * m) * 16);

    float om = -INFINITY, ol = 0.f;
    floatx4 oacc[C::kNdb];
#pragma unroll
    for (int b = 0; b < C::kNdb; ++b) oacc[b] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](Tile<D>& t, int n) __attribute__((always_inline)) {
      const int valid = n == it.n1 - 1 ? it.last_valid : kBlockSize;
      // S^T = K Q^T: lane l gets tokens 4 jg .. +3 of row col
      floatx4 rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < C::kNq; ++m) rr = mfma32<DT>(t.k[m], q[m], rr);
      float xs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[i] = 4 * jg + i < valid ? rr[i] * p.scale_log2 : -INFINITY;
      // the value tile into the wave's LDS rows, rows past the context zeroed
#pragma unroll
      for (int m = 0; m < C::kNld; ++m) {
        const int tok = m * C::kTpl + lane / C::kNch;
        const u32x4 vv = tok < valid ? t.v[m] : u32x4{0u, 0u, 0u, 0u};
        store16(sv + tok * C::kVS + (lane % C::kNch) * 16, vv);
      }
      __builtin_amdgcn_wave_barrier();
      const float m_tile = max4rows(fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3])));
      const bool grow = m_tile > om + kSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? m_tile : om;
        const float alpha = __builtin_amdgcn_exp2f(om - m_new);
        om = m_new;
        ol *= alpha;
#pragma unroll
        for (int b = 0; b < C::kNdb; ++b) oacc[b] *= alpha;
      }
      float pe[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pe[i] = __builtin_amdgcn_exp2f(xs[i] - om);
      ol += (pe[0] + pe[1]) + (pe[2] + pe[3]);
      const u32x4 pb = split_probs<DT>(pe);
      // O^T += V^T P^T: lane l reads dim 16b + col of tokens 4 jg .. +3
      const char* vsrc = sv + (4 * jg + (col >> 2)) * C::kVS + (col & 3) * 8;
#pragma unroll
      for (int b = 0; b < C::kNdb; ++b) {
        const uint2 va = read_tr16(vsrc + 32 * b);
        oacc[b] = mfma32<DT>(u32x4{va.x, va.y, va.x, va.y}, pb, oacc[b]);
      }
      __builtin_amdgcn_wave_barrier();
    };

    // two register tiles: the next tile's loads are in flight while the
    // current one is computed (past the item's last tile, its last tile
    // again, an L2 hit)
    Tile<D> ta, tb;
    load_tile(ta, it, ids, it.n0);
    for (int n = it.n0; n < it.n1; n += 2) {
      load_tile(tb, it, ids, n + 1 < it.n1 ? n + 1 : n);
      compute(ta, n);
      if (n + 1 < it.n1) {
        load_tile(ta, it, ids, n + 2 < it.n1 ? n + 2 : n + 1);
        compute(tb, n + 1);
      }
    }
    // every tile has a visible token, so the max is finite; the state of
    // lane column col's row: its sum over the four lane groups, and O^T
    // dims 16b + 4 jg .. +3
    const float l_tot = sum4rows(ol);
    if (col < it.nrows) {
      const int64_t slot =
          ((int64_t)it.seq_r * p.num_heads + it.head_r) * p.max_pieces + it.piece;
      float* dst = p.state_acc + slot * D + 4 * jg;
#pragma unroll
      for (int b = 0; b < C::kNdb; ++b)
        store16(dst + 16 * b, u32x4{bits_of(oacc[b][0]), bits_of(oacc[b][1]),
                                    bits_of(oacc[b][2]), bits_of(oacc[b][3])});
      if (jg == 0) {
        p.state_ml[slot * 2 + 0] = om;
        p.state_ml[slot * 2 + 1] = l_tot;
      }
    }
  }
}

// out[s, h] from the row's pieces: sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k,
// M = max_k m_k; zero for a sequence with no cached token.  A row takes D/4
// lanes, each holding 4 dims.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void shared_prefix_combine_kernel(const Params p) {
  constexpr int kLanesPerRow = D / 4;
  constexpr int kRowsPerWave = kWave / kLanesPerRow;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = (int)((blockIdx.x * (int64_t)kThreads + threadIdx.x) / kWave);
  const int64_t row = (int64_t)wave * kRowsPerWave + lane / kLanesPerRow;
  const int c = lane % kLanesPerRow;
  if (row >= (int64_t)p.num_seqs * p.num_heads) return;
  const int s = (int)(row / p.num_heads);
  const int2 pc = p.pieces[s];
  const int np = min(pc.x + pc.y, p.max_pieces);
  float M = -INFINITY, S = 0.f;
  floatx4 O = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < np; ++k) {
    const int64_t slot = row * p.max_pieces + k;
    const float mk = p.state_ml[slot * 2 + 0];
    const float lk = p.state_ml[slot * 2 + 1];
    const u32x4 a = load16(p.state_acc + slot * D + 4 * c);
    const float Mn = fmaxf(M, mk);
    const float wa = __builtin_amdgcn_exp2f(M - Mn);
    const float wb = __builtin_amdgcn_exp2f(mk - Mn);
    S = S * wa + lk * wb;
#pragma unroll
    for (int e = 0; e < 4; ++e) O[e] = fmaf(O[e], wa, wb * float_of(a[e]));
    M = Mn;
  }
  const float inv = np > 0 ? 1.f / S : 0.f;
  char* dst = (char*)p.out + (row * D + 4 * c) * Elt<DT>::kBytes;
  store4<DT>(dst, np > 0 ? O * inv : floatx4{0.f, 0.f, 0.f, 0.f});
}

// Workgroups the device holds at once (memoized per device and kernel).
static int resident_workgroups(const void* kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  struct Memo {
    int dev;
    const void* kernel;
    int wgs;
  };
  static std::mutex mu;
  static Memo memo[64];
  static int memo_n = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < memo_n; ++i)
    if (memo[i].dev == dev && memo[i].kernel == kernel) return memo[i].wgs;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess)
    return 0;
  // a workgroup puts one wave on each SIMD of its CU
  per_cu = per_cu < 1 ? 1 : (per_cu > kWavesPerSimd ? kWavesPerSimd : per_cu);
  const int n = cus * per_cu;
  if (memo_n < 64) memo[memo_n++] = Memo{dev, kernel, n};
  return n;
}

template <int DT, int D>
static hipError_t launch(const Params& a, hipStream_t st) {
  const void* k = reinterpret_cast<const void*>(&shared_prefix_rows_kernel<DT, D>);
  const int nwg = resident_workgroups(k);
  if (nwg <= 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL((shared_prefix_rows_kernel<DT, D>), dim3(nwg), dim3(kThreads), 0, st, a);
  const int64_t rows = (int64_t)a.num_seqs * a.num_heads;
  const int64_t rows_per_wg = (int64_t)kWaves * (kWave / (D / 4));
  const int64_t cwg = (rows + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((shared_prefix_combine_kernel<DT, D>), dim3((unsigned)cwg),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

struct Layout {
  size_t pieces, state_ml, state_acc, total;
};
static Layout layout_of(int num_seqs, int num_heads, int head_size, int max_pieces) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)num_seqs * num_heads * max_pieces;
  Layout l;
  l.pieces = 0;
  l.state_ml = up((size_t)num_seqs * sizeof(int2));
  l.state_acc = up(l.state_ml + rows * 2 * sizeof(float));
  l.total = up(l.state_acc + rows * head_size * sizeof(float));
  return l;
}
// pieces per row at most: the prefix chunks plus the suffix chunks
static int max_pieces_of(int max_blocks) { return ceil_div(max_blocks, kChunk) + 1; }

}  // namespace shared_prefix
}  // namespace pkv

extern "C" size_t paged_attention_shared_prefix_workspace_bytes(int num_seqs, int num_heads,
                                                                int head_size,
                                                                int max_blocks_per_seq) {
  using namespace pkv::shared_prefix;
  if (num_seqs <= 0 || num_seqs > kMaxSeqs || num_heads <= 0 || head_size <= 0 ||
      max_blocks_per_seq <= 0)
    return 0;
  return layout_of(num_seqs, num_heads, head_size, max_pieces_of(max_blocks_per_seq)).total;
}

extern "C" int paged_attention_decode_shared_prefix(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* order,
    const int32_t* group_start, const int32_t* prefix_blocks, int num_groups, float scale,
    int num_kv_heads, int num_seqs, int num_heads, int head_size, int block_size,
    int max_blocks_per_seq, int64_t num_blocks, void* workspace, size_t workspace_bytes,
    int dtype, void* stream) {
  using namespace pkv;
  using namespace pkv::shared_prefix;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (num_groups < 0 || (num_groups > 0 && (!group_start || !prefix_blocks)))
    return PKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || num_blocks > INT32_MAX || num_heads % num_kv_heads != 0)
    return PKV_ERR_INVALID_ARG;
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PKV_ERR_UNSUPPORTED;
  if (num_seqs > kMaxSeqs || num_groups > num_seqs) return PKV_ERR_UNSUPPORTED;
  if (((uintptr_t)query | (uintptr_t)key_cache | (uintptr_t)value_cache | (uintptr_t)out) &
      15u)
    return PKV_ERR_INVALID_ARG;  // rows are read and written 16 bytes at a time
  if (num_seqs == 0) return PKV_OK;
  // work items are counted in 32 bits: at most heads x pieces per row
  const int max_pieces = max_pieces_of(max_blocks_per_seq);
  if ((int64_t)num_seqs * num_heads * max_pieces > INT32_MAX) return PKV_ERR_INVALID_ARG;
  const size_t need = paged_attention_shared_prefix_workspace_bytes(num_seqs, num_heads,
                                                                    head_size, max_blocks_per_seq);
  if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 15u) return PKV_ERR_INVALID_ARG;

  const Layout l = layout_of(num_seqs, num_heads, head_size, max_pieces);
  Params a{};
  a.out = out;
  a.query = (const char*)query;
  a.kcache = (const char*)key_cache;
  a.vcache = (const char*)value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  // no groups: every sequence is a suffix of its own (the pointers are
  // never read)
  a.order = order;
  a.group_start = num_groups > 0 ? group_start : context_lens;
  a.prefix_blocks = num_groups > 0 ? prefix_blocks : context_lens;
  a.pieces = (int2*)((char*)workspace + l.pieces);
  a.state_ml = (float*)((char*)workspace + l.state_ml);
  a.state_acc = (float*)((char*)workspace + l.state_acc);
  a.scale_log2 = scale * 1.4426950408889634f;  // exp(x) = 2^(x log2 e)
  a.num_seqs = num_seqs;
  a.num_groups = num_groups;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_pieces = max_pieces;
  a.num_blocks = num_blocks;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();  // start from a clean error state
  hipError_t e;
  if (dtype == PKV_F16)
    e = head_size == 64 ? launch<PKV_F16, 64>(a, st) : launch<PKV_F16, 128>(a, st);
  else
    e = head_size == 64 ? launch<PKV_BF16, 64>(a, st) : launch<PKV_BF16, 128>(a, st);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
