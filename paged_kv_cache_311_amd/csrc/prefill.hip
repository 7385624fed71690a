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
//   rows      = (new token, query head of the group) pairs of one
//               (sequence, kv head), token-major: row r is token r / G,
//               head r % G of the group (G = Hq / Hkv).
//   workgroup = 128 rows of one (sequence, kv head): 4 waves x 2 blocks
//               of 16 rows.  It walks the keys 32 at a time (two pool
//               blocks), from token 0 to the last position its rows see.
//   per step  = the 256 threads load the two blocks' K and V tiles
//               (16-B chunks, through the table) into registers, then into
//               one of two LDS buffers; the step after computes from that
//               buffer while the next step's loads are in flight.
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
//                transposed from LDS (2-byte reads).  Lane l holds output
//                dims 16j + 4(l/16) .. +3 of row l % 16, so the rescale by
//                the row's running max and the final 1/sum are lane-local.
//
// Precision: products accumulate in float32; the probabilities enter the
// second product rounded to the input type (as the values are), and the
// row sums are taken over the rounded probabilities, so the output is an
// exact weighted mean of the values under weights perturbed by at most one
// rounding each.

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

// LDS: two buffers of K [32 tokens][D] and V [32 tokens][D], rows padded so
// that the 16-lane groups of a 16-B key read and of a transposed 2-B value
// read fall on distinct banks.
template <int D>
struct Lds {
  static constexpr int kKS = D * 2 + 16;    // key row stride (bytes), 16-B aligned
  static constexpr int kVS = D * 2 + 8;     // value row stride (bytes), 8-B aligned
  static constexpr int kKBuf = kKeys * kKS;
  static constexpr int kVBuf = kKeys * kVS;
  static constexpr int kBytes = 2 * kKBuf + 2 * kVBuf;
};

struct Params {
  void* out;
  const char* query;
  const char* kcache;
  const char* vcache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  float scale_log2;  // softmax scale x log2 e
  int num_seqs, num_heads, num_kv_heads, max_blocks;
  int64_t num_blocks;
  int row_tiles;     // 128-row tiles per (sequence, kv head) the grid covers
};

template <int DT>
__device__ __forceinline__ floatx4 mfma32(const u32x4& a, const u32x4& b, const floatx4& c) {
  if constexpr (DT == PKV_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Round a float to the 16-bit type and give its bits, and back (exact).
template <int DT>
__device__ __forceinline__ uint32_t to16(float x) {
  return float_to_bits<DT>(x);
}
template <int DT>
__device__ __forceinline__ float from16(uint32_t h) {
  if constexpr (DT == PKV_F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  else
    return float_of(h << 16);
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads, 2) void paged_prefill_kernel(const Params p) {
  using LD = Lds<D>;
  constexpr int NKS = D / 32;                    // QK k-steps of 32 dims
  constexpr int NDB = D / 16;                    // output blocks of 16 dims
  constexpr int CPR = D / 8;                     // 16-B chunks per token row
  constexpr int NCH = kKeys * CPR / kThreads;    // chunks per thread per tensor
  static_assert(NCH * kThreads == kKeys * CPR, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) char lds[LD::kBytes];

  // workgroup -> (row tile, sequence, kv head); the latest (heaviest) row
  // tiles of every (sequence, kv head) are dispatched first
  const int per_tile = p.num_seqs * p.num_kv_heads;
  const int rank = blockIdx.x / per_tile;
  const int sg = blockIdx.x - rank * per_tile;
  const int s = sg / p.num_kv_heads;
  const int g = sg - s * p.num_kv_heads;
  const int tile = p.row_tiles - 1 - rank;

  const int G = p.num_heads / p.num_kv_heads;
  const int q0 = p.query_start_loc[s];
  const int n = p.query_start_loc[s + 1] - q0;
  const int rows = n * G;
  const int R0 = tile * kRows;
  if (n <= 0 || R0 >= rows) return;  // uniform per workgroup
  const int max_tokens = p.max_blocks * kBlockSize;
  int Lc = p.context_lens[s];
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

  // this lane's rows (one per 16-row block) and their query operands
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
      q[rb][m] = row_ok[rb] ? load16(p.query + (row_off[rb] + 32 * m + 8 * grp) * 2)
                            : u32x4{0u, 0u, 0u, 0u};
  }

  // cooperative tile loads: chunk c = tid + 256u is 16 B of token c / CPR
  const int64_t blk_bytes = (int64_t)p.num_kv_heads * kBlockSize * D * 2;
  const int64_t head_bytes = (int64_t)g * kBlockSize * D * 2;
  const int32_t* table = p.block_tables + (int64_t)s * p.max_blocks;
  u32x4 kst[NCH], vst[NCH];
  auto gload = [&](int step) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + u * kThreads;
      const int tk = c / CPR;
      const int t = step * kKeys + tk;
      kst[u] = u32x4{0u, 0u, 0u, 0u};  // tokens past the context: zero
      vst[u] = u32x4{0u, 0u, 0u, 0u};
      if (t < Lc) {
        int64_t b = table[t / kBlockSize];
        b = b < 0 ? 0 : (b >= p.num_blocks ? p.num_blocks - 1 : b);
        const int64_t off = b * blk_bytes + head_bytes + (int64_t)(t % kBlockSize) * D * 2 +
                            (c - tk * CPR) * 16;
        kst[u] = load16(p.kcache + off);
        vst[u] = load16(p.vcache + off);
      }
    }
  };
  auto lstore = [&](int buf) {
    char* kb = lds + buf * LD::kKBuf;
    char* vb = lds + 2 * LD::kKBuf + buf * LD::kVBuf;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + u * kThreads;
      const int tk = c / CPR;
      const int dc = c - tk * CPR;
      store16(kb + tk * LD::kKS + dc * 16, kst[u]);
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const uint32_t v0 = vst[u][0], v1 = vst[u][1], v2 = vst[u][2], v3 = vst[u][3];
      *reinterpret_cast<u32x2*>(vb + tk * LD::kVS + dc * 16) = u32x2{v0, v1};
      *reinterpret_cast<u32x2*>(vb + tk * LD::kVS + dc * 16 + 8) = u32x2{v2, v3};
    }
  };

  float m_run[kRB], l_run[kRB];
  floatx4 acc[kRB][NDB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int j = 0; j < NDB; ++j) acc[rb][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  if (nsteps > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) gload(step + 1);
    const char* kb = lds + buf * LD::kKBuf;
    const char* vb = lds + 2 * LD::kKBuf + buf * LD::kVBuf;

    // S^T for both key blocks and both row blocks
    floatx4 sc[kRB][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) sc[rb][h] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < NKS; ++m) {
        const u32x4 a = load16(kb + (h * 16 + col) * LD::kKS + (32 * m + 8 * grp) * 2);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) sc[rb][h] = mfma32<DT>(a, q[rb][m], sc[rb][h]);
      }
    }

    // online softmax per row; probabilities packed as the B operand of PV
    u32x4 pb[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float x[8];
      float mt = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = step * kKeys + h * 16 + 4 * grp + i;
          const float v = sc[rb][h][i] * p.scale_log2;
          x[h * 4 + i] = (t <= pos[rb] && t < Lc) ? v : -INFINITY;
          mt = fmaxf(mt, x[h * 4 + i]);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
      mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
      const float m_new = fmaxf(m_run[rb], mt);
      const bool none = m_new == -INFINITY;  // nothing visible to this row yet
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
      m_run[rb] = m_new;
      uint32_t hbits[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = none ? 0.f : __builtin_amdgcn_exp2f(x[e] - m_new);
        hbits[e] = to16<DT>(pe);
        psum += from16<DT>(hbits[e]);
      }
      l_run[rb] = l_run[rb] * alpha + psum;
#pragma unroll
      for (int j = 0; j < NDB; ++j) acc[rb][j] *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[rb][e] = hbits[2 * e] | (hbits[2 * e + 1] << 16);
    }

    // O^T += V^T P^T, one 16-dim block at a time
#pragma unroll
    for (int j = 0; j < NDB; ++j) {
      uint32_t vh[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vh[h * 4 + i] = *reinterpret_cast<const uint16_t*>(
              vb + (h * 16 + 4 * grp + i) * LD::kVS + (16 * j + col) * 2);
      }
      const u32x4 a = {vh[0] | (vh[1] << 16), vh[2] | (vh[3] << 16), vh[4] | (vh[5] << 16),
                       vh[6] | (vh[7] << 16)};
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) acc[rb][j] = mfma32<DT>(a, pb[rb], acc[rb][j]);
    }

    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

  // normalize and store: lane l holds dims 16j + 4(l/16) .. +3 of its row
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    float l = l_run[rb];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (row_ok[rb]) {
      char* dst = (char*)p.out + (row_off[rb] + 4 * grp) * 2;
#pragma unroll
      for (int j = 0; j < NDB; ++j) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const floatx4 o = acc[rb][j];
        const float o0 = o[0] * inv, o1 = o[1] * inv, o2 = o[2] * inv, o3 = o[3] * inv;
        *reinterpret_cast<u32x2*>(dst + 16 * j * 2) =
            u32x2{to16<DT>(o0) | (to16<DT>(o1) << 16), to16<DT>(o2) | (to16<DT>(o3) << 16)};
      }
    }
  }
}

template <int DT, int D>
static hipError_t launch(const Params& a, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((paged_prefill_kernel<DT, D>), dim3(grid), dim3(kThreads), 0, st, a);
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
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PKV_ERR_UNSUPPORTED;
  if (((uintptr_t)query | (uintptr_t)key_cache | (uintptr_t)value_cache) & 15u)
    return PKV_ERR_INVALID_ARG;  // 16-byte loads
  if ((uintptr_t)out & 7u) return PKV_ERR_INVALID_ARG;  // 8-byte stores
  if (num_seqs == 0 || max_query_len == 0) return PKV_OK;
  const int64_t rows = (int64_t)max_query_len * (num_heads / num_kv_heads);
  const int64_t row_tiles = (rows + kRows - 1) / kRows;
  const int64_t grid = row_tiles * num_seqs * num_kv_heads;
  if (row_tiles > INT32_MAX || grid > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_query_len * num_heads > INT32_MAX / 2) return PKV_ERR_INVALID_ARG;
  Params a;
  a.out = out;
  a.query = (const char*)query;
  a.kcache = (const char*)key_cache;
  a.vcache = (const char*)value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.row_tiles = (int)row_tiles;
  (void)hipGetLastError();
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dtype == PKV_F16)
    e = head_size == 64 ? launch<PKV_F16, 64>(a, (unsigned)grid, st)
                        : launch<PKV_F16, 128>(a, (unsigned)grid, st);
  else
    e = head_size == 64 ? launch<PKV_BF16, 64>(a, (unsigned)grid, st)
                        : launch<PKV_BF16, 128>(a, (unsigned)grid, st);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
