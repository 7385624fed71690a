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
//   range     = qt consecutive tiles of that flattened order; the grid is
//               sized to what the chip holds resident and every wave takes
//               ranges v, v + NWV, ...  so each wave streams the same number
//               of bytes whatever the length mix (no empty or straggling
//               workgroups).
//   piece     = the part of one segment inside one range.  A wave keeps an
//               online softmax per piece; a piece that is a whole segment
//               writes the output directly, a piece of a split segment
//               writes float32 partials (running max, sum, unnormalized
//               accumulator).  The range holding a split segment's last
//               tile names that segment in a per-range descriptor, and a
//               second, light kernel merges the pieces of every segment a
//               descriptor names (one wave each).
//
// Per tile (one wave):
//   QK  = MFMA chain: the key tile is the B operand exactly as loaded (lane
//         l holds token l%16), the query rows are replicated so every lane
//         receives the logits of its own token for all heads of the group.
//   softmax = online, in log2 units; the running max per head is wave
//         uniform (DPP row reduction) and the accumulator is rescaled only
//         when it grows.
//   PV  = VALU FMA in float32 over value tiles loaded as contiguous 1 KiB
//         rows per instruction; probabilities reach the value layout through
//         a 16 x GC LDS buffer owned by the wave.
//   The next tile's K and V are loaded while the current one is computed.
//
// Masking: tokens at or beyond the context length in the last block are
// excluded by select (logit -inf, value zeroed), never by multiplying
// garbage by zero, so NaN-filled free slots cannot leak into the result.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "pkv_device.h"

namespace pkv {

constexpr int kWavesPerWG = 4;
constexpr int kThreads = kWavesPerWG * kWave;
constexpr int kMaxWGs = 2048;                   // at most 8192 resident waves
constexpr int kMaxWaves = kMaxWGs * kWavesPerWG;
constexpr int kMinTilesPerRange = 4;
constexpr int kMaxPartition = 4096;             // tokens per piece, when capped
constexpr int kSoloPieces = 8;                  // merged by one wave up to this many

template <int DT, int D, int GC>
struct DecodeCfg {
  static constexpr int kEsz = Elt<DT>::kBytes;
  static constexpr int kEpc = Elt<DT>::kPer16B;      // elements per 16-B chunk
  static constexpr int kRowB = D * kEsz;             // bytes per token row
  static constexpr int kNch = kRowB / 16;            // 16-B chunks per row
  static constexpr int kTileB = kBlockSize * kRowB;  // bytes per (block, kv head)
  static constexpr int kNld = kTileB / 1024;         // 16-B loads per lane per tile
  static constexpr int kTpl = kWave / kNch;          // tokens per 1-KiB value load
  static constexpr int kGcq = GC < 4 ? GC : 4;       // heads per MFMA chain
  static constexpr int kNqg = (GC + 3) / 4;          // MFMA chains per tile
  static_assert(kNch * 16 == kRowB, "row must be a whole number of 16-B chunks");
  static_assert(kNld * 4 == kNch, "key tile: 4 lane groups x kNld chunks per row");
  static_assert(kNch >= 8 && kNch <= 32, "lane-group reduction assumes 8..32 chunks");
  static_assert(GC == 1 || GC == 2 || GC == 4 || GC == 8, "heads per workgroup");
  // Waves per SIMD the register allocator must leave room for: 3 where the
  // kernel fits in 168 VGPRs without spilling (16-bit K/V up to 4 heads per
  // group, and 64-wide float32), otherwise whatever it needs.
  static constexpr int kMinWaves = (GC <= 4 && (kEsz == 2 || D == 64)) ? 3 : 1;
};

struct DecodeParams {
  void* out;
  const char* query;
  const char* kcache;
  const char* vcache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale_log2;
  int num_seqs, num_heads, num_kv_heads, max_blocks;
  int64_t num_blocks;
  int tile_cap;        // max tiles per range (0: no cap)
  int* header;         // [2]  ranges R, tiles per range qt (this call)
  int4* desc;          // [r_max]  split segment ending in range r: s, hg, P, nb
  float* part_ml;      // [r_max][2][GC][2]  running max (log2 units), sum
  float* part_acc;     // [r_max][2][GC][D]  unnormalized accumulator
};

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

// Tiles of every segment, summed over all sequences (wave-uniform).
__device__ int total_tiles(const DecodeParams& p, int head_groups, int lane) {
  const int max_tokens = p.max_blocks * kBlockSize;
  int acc = 0;
  for (int base = 0; base < p.num_seqs; base += kWave) {
    const int s = base + lane;
    if (s < p.num_seqs) acc += blocks_of(clamp_len(p.context_lens[s], max_tokens));
  }
  return sread(wave_sum_i(acc)) * head_groups;
}

// Tiles per range and number of ranges for T tiles over nwaves waves.
__device__ __forceinline__ void range_shape(int T, int nwaves, int cap, int& qt, int& R) {
  qt = (T + nwaves - 1) / nwaves;
  qt = qt < kMinTilesPerRange ? kMinTilesPerRange : qt;
  if (cap > 0 && qt > cap) qt = cap;
  R = T == 0 ? 0 : (T + qt - 1) / qt;
}

// Move (s, excl) forward to the sequence whose tiles contain flattened
// position x: excl = first flattened tile of sequence s.  Monotone: the
// search resumes from the caller's (s, excl).
__device__ void locate(const DecodeParams& p, int head_groups, int lane, int x, int& s_io,
                       int& excl_io) {
  const int max_tokens = p.max_blocks * kBlockSize;
  int base = s_io;
  int carry = excl_io;
  while (base < p.num_seqs) {
    const int s = base + lane;
    const int v = s < p.num_seqs
                      ? blocks_of(clamp_len(p.context_lens[s], max_tokens)) * head_groups
                      : 0;
    const int incl = wave_incl_scan_i(v, lane) + carry;
    const int excl = incl - v;
    const unsigned long long hit = __ballot(s < p.num_seqs && excl <= x && x < incl);
    if (hit) {
      // readlane keeps the results in scalar registers, so everything
      // derived from them (addresses included) stays wave-uniform
      const int l = __ffsll((long long)hit) - 1;
      s_io = base + l;
      excl_io = __builtin_amdgcn_readlane(excl, l);
      return;
    }
    carry = __builtin_amdgcn_readlane(incl, kWave - 1);
    base += kWave;
  }
  s_io = p.num_seqs;
  excl_io = carry;
}

template <int DT, int NLD>
__device__ __forceinline__ floatx4 qk_mfma(const u32x4 (&q)[NLD], const Tile& t) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < NLD; ++m) {
    if constexpr (DT == PKV_F16) {
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
template <int DT>
__device__ __forceinline__ void store4(char* dst, const floatx4& v) {
  if constexpr (DT == PKV_F32) {
    store16(dst, u32x4{bits_of(v[0]), bits_of(v[1]), bits_of(v[2]), bits_of(v[3])});
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2*>(dst) =
        u32x2{float_to_bits<DT>(v[0]) | (float_to_bits<DT>(v[1]) << 16),
              float_to_bits<DT>(v[2]) | (float_to_bits<DT>(v[3]) << 16)};
  }
}

// Merging the pieces k = 0..np-1 of a split segment (ranges rf..rf+np-1):
//   out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k,  M = max_k m_k.
// A wave folds a subset of the pieces into a running (max, sum, acc)
// state; every lane owns 16-byte chunks of the [GC][D] accumulator.
template <int D, int GC>
struct FoldState {
  static constexpr int kChunks = GC * D / 4;
  static constexpr int kCpl = (kChunks + kWave - 1) / kWave;
  float M[GC], S[GC];
  floatx4 O[kCpl];
};

struct Split {
  int s, hg, P, nb, rf, np;
  bool rf_tail;  // range rf's piece of this segment sits in its second slot
};

__device__ __forceinline__ Split split_of(const int4& d, int qt) {
  Split x;
  x.s = d.x;
  x.hg = d.y;
  x.P = d.z;
  x.nb = d.w;
  x.rf = x.P / qt;
  x.np = (x.P + x.nb - 1) / qt - x.rf + 1;
  x.rf_tail = x.P != x.rf * qt;
  return x;
}

template <int D, int GC>
__device__ void fold_pieces(const DecodeParams& p, const Split& sp, int k0, int kstep,
                            int lane, FoldState<D, GC>& st) {
  using F = FoldState<D, GC>;
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    st.M[g] = -INFINITY;
    st.S[g] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < F::kCpl; ++j) st.O[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = k0; k < sp.np; k += kstep) {
    const int64_t sl = (int64_t)(sp.rf + k) * 2 + ((k == 0 && sp.rf_tail) ? 1 : 0);
    float a[GC], b[GC];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const float mk = p.part_ml[(sl * GC + g) * 2 + 0];
      const float lk = p.part_ml[(sl * GC + g) * 2 + 1];
      const float Mn = fmaxf(st.M[g], mk);
      a[g] = __builtin_amdgcn_exp2f(st.M[g] - Mn);
      b[g] = __builtin_amdgcn_exp2f(mk - Mn);
      st.S[g] = st.S[g] * a[g] + lk * b[g];
      st.M[g] = Mn;
    }
#pragma unroll
    for (int j = 0; j < F::kCpl; ++j) {
      const int c = lane + j * kWave;
      if (c < F::kChunks) {
        const int g = c * 4 / D;
        float ag = a[0], bg = b[0];
#pragma unroll
        for (int gg = 1; gg < GC; ++gg) {
          ag = g == gg ? a[gg] : ag;
          bg = g == gg ? b[gg] : bg;
        }
        const u32x4 x = load16(p.part_acc + sl * GC * D + c * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) st.O[j][e] = fmaf(st.O[j][e], ag, bg * float_of(x[e]));
      }
    }
  }
}

template <int DT, int D, int GC>
__device__ __forceinline__ void store_merged(const DecodeParams& p, const Split& sp, int c,
                                             const floatx4& o, float inv) {
  char* dst = (char*)p.out +
              (((int64_t)sp.s * p.num_heads + sp.hg * GC) * D + c * 4) * Elt<DT>::kBytes;
  store4<DT>(dst, o * inv);
}

// A segment of few pieces: one wave folds them all and writes the output.
template <int DT, int D, int GC>
__device__ void merge_by_wave(const DecodeParams& p, const Split& sp, int lane) {
  using F = FoldState<D, GC>;
  F st;
  fold_pieces<D, GC>(p, sp, 0, 1, lane, st);
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

// ------------------------------------------------------------ main kernel --
template <int DT, int D, int GC>
__global__ __launch_bounds__(kThreads, (DecodeCfg<DT, D, GC>::kMinWaves)) void
paged_decode_kernel(const DecodeParams p) {
  using C = DecodeCfg<DT, D, GC>;
  constexpr int NLD = C::kNld;
  constexpr int EPC = C::kEpc;

  __shared__ float sm_p[kWavesPerWG][kBlockSize * GC];

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

  const int head_groups = p.num_heads / GC;
  const int group = p.num_heads / p.num_kv_heads;
  const int max_tokens = p.max_blocks * kBlockSize;
  const int T = total_tiles(p, head_groups, lane);

  // sequences with no cached token: their output is zero
  for (int base = 0; base < p.num_seqs; base += kWave) {
    const int s = base + lane;
    unsigned long long z = __ballot(s < p.num_seqs && s % nwaves == v &&
                                    clamp_len(p.context_lens[s], max_tokens) == 0);
    while (z) {
      const int l = __ffsll((long long)z) - 1;
      z &= z - 1;
      const int64_t row0 = (int64_t)(base + l) * p.num_heads * D;
      for (int i = lane; i < p.num_heads * D; i += kWave) store_elem<DT>(p.out, row0 + i, 0.f);
    }
  }

  int qt, R;
  range_shape(T, nwaves, p.tile_cap, qt, R);
  if (v == 0 && lane == 0) {
    p.header[0] = R;
    p.header[1] = qt;
  }
  if (v >= R) return;

  float* pw = sm_p[w];
  const int row = lane & 15;
  const int jg = lane >> 4;
  const uint32_t koff_lane = (uint32_t)(row * C::kRowB + jg * 16);
  const uint32_t voff_lane = (uint32_t)(lane * 16);
  const int64_t block_stride = (int64_t)p.num_kv_heads * C::kTileB;

  int ls = 0, lexcl = 0;  // locate cursor
  for (int r = v; r < R; r += nwaves) {
    const int x0 = r * qt;
    const int x1 = min(x0 + qt, T);
    locate(p, head_groups, lane, x0, ls, lexcl);
    int s = ls;
    int L = clamp_len(p.context_lens[s], max_tokens);
    int nb = blocks_of(L);
    int local = x0 - lexcl;
    int hg = local / nb;
    int n0 = local - hg * nb;
    int x = x0;
    bool first_piece = true;
    while (x < x1) {
      const int n1 = min(nb, n0 + (x1 - x));
      const int cnt = n1 - n0;
      const bool complete = n0 == 0 && n1 == nb;
      const int h0 = hg * GC;
      const int kvh = h0 / group;
      if (first_piece && lane == 0) {
        // a range's first piece is the last piece of a split segment exactly
        // when the segment began in an earlier range and ends in this one
        p.desc[r] = (n0 > 0 && n1 == nb) ? int4{s, hg, x - n0, nb} : int4{-1, 0, 0, 0};
      }

      // query rows as MFMA A operands: row r of chain c is head c*4 + r % kGcq
      u32x4 qa[C::kNqg][NLD];
#pragma unroll
      for (int c = 0; c < C::kNqg; ++c) {
        const int head = h0 + c * 4 + (row % C::kGcq);
        const char* qrow = p.query + ((int64_t)s * p.num_heads + head) * C::kRowB;
#pragma unroll
        for (int m = 0; m < NLD; ++m) qa[c][m] = load16(qrow + (jg + 4 * m) * 16);
      }

      float m_run[GC], l_run[GC], acc[GC][EPC];
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        m_run[g] = -INFINITY;
        l_run[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[g][e] = 0.f;
      }

      const int32_t* bt_row = p.block_tables + (int64_t)s * p.max_blocks;
      const char* kbase = p.kcache + (int64_t)kvh * C::kTileB;
      const char* vbase = p.vcache + (int64_t)kvh * C::kTileB;

      // the piece's tiles in windows of 64 (one block id per lane)
      for (int c0 = 0; c0 < cnt; c0 += kWave) {
        const int wcnt = min(kWave, cnt - c0);
        int my_id = 0;
        if (lane < wcnt) {
          int64_t b = bt_row[n0 + c0 + lane];
          b = b < 0 ? 0 : (b >= p.num_blocks ? p.num_blocks - 1 : b);
          my_id = (int)b;
        }
        auto load_tile = [&](Tile& t, int i) {
          const int64_t off = (int64_t)__builtin_amdgcn_readlane(my_id, i) * block_stride;
          const char* kb = kbase + off;
          const char* vb = vbase + off;
#pragma unroll
          for (int m = 0; m < NLD; ++m) t.k[m] = load16(kb + koff_lane + m * 64);
#pragma unroll
          for (int m = 0; m < NLD; ++m) t.v[m] = load16(vb + voff_lane + m * 1024);
        };
        auto compute_tile = [&](const Tile& t, int i) {
          const int valid = L - (n0 + c0 + i) * kBlockSize;  // >= 1; < 16 only last block
          float sc[GC];
#pragma unroll
          for (int c = 0; c < C::kNqg; ++c) {
            const floatx4 rr = qk_mfma<DT, NLD>(qa[c], t);
#pragma unroll
            for (int j = 0; j < C::kGcq; ++j) sc[c * 4 + j] = rr[j] * p.scale_log2;
          }
          if (row >= valid) {
#pragma unroll
            for (int g = 0; g < GC; ++g) sc[g] = -INFINITY;
          }
          float pr[GC];
#pragma unroll
          for (int g = 0; g < GC; ++g) {
            const float tmax = uniform(row_max16(sc[g]));
            if (tmax > m_run[g]) {
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
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int ld = 0; ld < NLD; ++ld) {
            const int tok = ld * C::kTpl + lane / C::kNch;
            float pv[GC];
#pragma unroll
            for (int g = 0; g < GC; ++g) pv[g] = pw[tok * GC + g];
            u32x4 vv = t.v[ld];
            if (valid < kBlockSize && tok >= valid) vv = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
              const float f = elem_to_float<DT>(vv, e);
#pragma unroll
              for (int g = 0; g < GC; ++g) acc[g][e] = fmaf(pv[g], f, acc[g][e]);
            }
          }
          __builtin_amdgcn_wave_barrier();
        };

        // two register tiles, alternating: load i+1 while computing i
        Tile ta, tb;
        load_tile(ta, 0);
        for (int i = 0; i < wcnt; i += 2) {
          if (i + 1 < wcnt) load_tile(tb, i + 1);
          compute_tile(ta, i);
          if (i + 1 < wcnt) {
            if (i + 2 < wcnt) load_tile(ta, i + 2);
            compute_tile(tb, i + 1);
          }
        }
      }

      // piece totals: l over the 16 token lanes; acc over lanes sharing a chunk
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        l_run[g] = row_sum16(l_run[g]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[g][e] = sum_over_lane_groups<C::kNch>(acc[g][e]);
      }
      if (complete) {
        if (lane < C::kNch) {
#pragma unroll
          for (int g = 0; g < GC; ++g) {
            const float inv = 1.f / l_run[g];
            float o[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[e] = acc[g][e] * inv;
            char* dst = (char*)p.out +
                        (((int64_t)s * p.num_heads + h0 + g) * D + lane * EPC) * C::kEsz;
            store_chunk<DT>(dst, o);
          }
        }
      } else {
        const int64_t slot = (int64_t)r * 2 + (first_piece ? 0 : 1);
        if (lane < C::kNch) {
#pragma unroll
          for (int g = 0; g < GC; ++g) {
            float* dst = p.part_acc + (slot * GC + g) * D + lane * EPC;
#pragma unroll
            for (int e = 0; e < EPC; e += 4)
              store16(dst + e, u32x4{bits_of(acc[g][e]), bits_of(acc[g][e + 1]),
                                     bits_of(acc[g][e + 2]), bits_of(acc[g][e + 3])});
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

      // next piece: the next segment (next head group, or next sequence
      // that has a cached token)
      x += cnt;
      first_piece = false;
      n0 = 0;
      if (x < x1) {
        if (++hg == head_groups) {
          hg = 0;
          do {
            ++s;
            L = clamp_len(p.context_lens[s], max_tokens);
          } while (L == 0);
          nb = blocks_of(L);
        }
      }
    }
  }
}

// ----------------------------------------------------------- merge kernel --
// Workgroups take four ranges at a time; a range whose descriptor names a
// split segment gets that segment's pieces merged into its output.
template <int DT, int D, int GC>
__global__ __launch_bounds__(kThreads) void paged_decode_merge_kernel(const DecodeParams p) {
  __shared__ MergeSmem<D, GC> sm;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = sread(threadIdx.x >> 6);
  const int R = p.header[0];
  const int qt = p.header[1];
  for (int base = blockIdx.x * kWavesPerWG; base < R; base += gridDim.x * kWavesPerWG) {
    // each wave merges its own range's segment if it has few pieces ...
    const int r = base + w;
    if (r < R) {
      const int4 d = p.desc[r];
      if (d.x >= 0) {
        const Split sp = split_of(d, qt);
        if (sp.np <= kSoloPieces) merge_by_wave<DT, D, GC>(p, sp, lane);
      }
    }
    // ... and the four waves together take those with many
    for (int v = 0; v < kWavesPerWG && base + v < R; ++v) {
      const int4 d = p.desc[base + v];
      if (d.x < 0) continue;
      const Split sp = split_of(d, qt);
      if (sp.np > kSoloPieces) merge_by_workgroup<DT, D, GC>(p, sp, lane, w, sm);
    }
  }
}

// ------------------------------------------------------------------ host --
// Resident workgroups of a kernel on the current device (memoized: the
// answer depends only on the device and the kernel's resources).
static int resident_workgroups(const void* kernel) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static std::vector<std::pair<std::pair<int, const void*>, int>> memo;
  std::lock_guard<std::mutex> lock(mu);
  for (auto& e : memo)
    if (e.first.first == dev && e.first.second == kernel) return e.second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess)
    return 0;
  int n = cus * (per_cu > 0 ? per_cu : 1);
  n = n > kMaxWGs ? kMaxWGs : n;
  memo.push_back({{dev, kernel}, n});
  return n;
}

template <int DT, int D, int GC>
static hipError_t launch_decode(const DecodeParams& a, hipStream_t st) {
  const void* k = reinterpret_cast<const void*>(&paged_decode_kernel<DT, D, GC>);
  const int nwg = resident_workgroups(k);
  if (nwg <= 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL((paged_decode_kernel<DT, D, GC>), dim3(nwg), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((paged_decode_merge_kernel<DT, D, GC>), dim3(nwg), dim3(kThreads), 0, st,
                     a);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t dispatch_gc(const DecodeParams& a, int gc, hipStream_t st) {
  switch (gc) {
    case 1: return launch_decode<DT, D, 1>(a, st);
    case 2: return launch_decode<DT, D, 2>(a, st);
    case 4: return launch_decode<DT, D, 4>(a, st);
    default: return launch_decode<DT, D, 8>(a, st);
  }
}

template <int DT>
static hipError_t dispatch_d(const DecodeParams& a, int d, int gc, hipStream_t st) {
  return d == 64 ? dispatch_gc<DT, 64>(a, gc, st) : dispatch_gc<DT, 128>(a, gc, st);
}

static int heads_per_wg(int num_heads, int num_kv_heads) {
  const int group = num_heads / num_kv_heads;
  return group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
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

// Workspace: header [2 ints], range descriptors [r][4 ints], then (max,
// sum) [r][2][gc][2] and accumulators [r][2][gc][head_size] in float32;
// each part 256-B aligned.  Every call writes what it reads.
struct WorkspaceLayout {
  size_t header, desc, part_ml, part_acc, total;
};
static WorkspaceLayout workspace_layout(int64_t r, int gc, int head_size) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WorkspaceLayout l;
  l.header = 0;
  l.desc = 256;
  l.part_ml = up(l.desc + (size_t)r * 16);
  l.part_acc = up(l.part_ml + (size_t)r * 2 * gc * 2 * sizeof(float));
  l.total = up(l.part_acc + (size_t)r * 2 * gc * head_size * sizeof(float));
  return l;
}

static bool partition_ok(int ps) {
  return ps == 0 || (ps >= kBlockSize && ps <= kMaxPartition && ps % kBlockSize == 0);
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
  const int gc = heads_per_wg(num_heads, num_kv_heads);
  const int64_t max_tiles = (int64_t)num_seqs * max_blocks_per_seq * (num_heads / gc);
  const int64_t r = max_ranges(max_tiles, partition_size / kBlockSize);
  return workspace_layout(r, gc, head_size).total;
}

extern "C" int paged_attention_decode(void* out, const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, float scale,
                                      int num_kv_heads, int num_seqs, int num_heads,
                                      int head_size, int block_size, int max_blocks_per_seq,
                                      int64_t num_blocks, int partition_size, void* workspace,
                                      size_t workspace_bytes, int dtype, void* stream) {
  using namespace pkv;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || num_blocks > INT32_MAX)
    return PKV_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PKV_ERR_UNSUPPORTED;
  if (!partition_ok(partition_size)) return PKV_ERR_INVALID_ARG;
  if (((uintptr_t)query | (uintptr_t)key_cache | (uintptr_t)value_cache | (uintptr_t)out) &
      15u)
    return PKV_ERR_INVALID_ARG;  // rows are read and written 16 bytes at a time
  const int gc = heads_per_wg(num_heads, num_kv_heads);
  // flattened tile positions are 32-bit
  if ((int64_t)num_seqs * max_blocks_per_seq * (num_heads / gc) > INT32_MAX)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  const size_t need = paged_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads,
                                                      head_size, max_blocks_per_seq,
                                                      block_size, partition_size);
  if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 15u) return PKV_ERR_INVALID_ARG;

  DecodeParams a{};
  a.out = out;
  a.query = (const char*)query;
  a.kcache = (const char*)key_cache;
  a.vcache = (const char*)value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale_log2 = scale * 1.4426950408889634f;  // exp(x) = 2^(x log2 e)
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.tile_cap = partition_size / kBlockSize;
  const int64_t r = max_ranges((int64_t)num_seqs * max_blocks_per_seq * (num_heads / gc),
                               a.tile_cap);
  const WorkspaceLayout wl = workspace_layout(r, gc, head_size);
  a.header = (int*)((char*)workspace + wl.header);
  a.desc = (int4*)((char*)workspace + wl.desc);
  a.part_ml = (float*)((char*)workspace + wl.part_ml);
  a.part_acc = (float*)((char*)workspace + wl.part_acc);
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();  // start from a clean error state
  hipError_t e;
  switch (dtype) {
    case PKV_F32: e = dispatch_d<PKV_F32>(a, head_size, gc, st); break;
    case PKV_F16: e = dispatch_d<PKV_F16>(a, head_size, gc, st); break;
    default: e = dispatch_d<PKV_BF16>(a, head_size, gc, st); break;
  }
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
