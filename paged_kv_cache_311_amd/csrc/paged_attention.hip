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
// Work decomposition
//   workgroup  = (sequence, group of GC query heads sharing one kv head,
//                 partition of `partition_size` logical tokens); 4 waves.
//   wave       = every 4th block of the partition; per block it loads the
//                 (block, kv head) key tile and value tile (16 x head_size
//                 contiguous elements each), prefetching the next block's
//                 tiles while it computes on the current ones.
//   QK         = one MFMA chain per tile: the key tile is the B operand as
//                 loaded (lane l holds token l%16), the query rows are
//                 replicated so every lane receives the logits of its own
//                 token for all heads of the group.
//   softmax    = online, in log2 units, wave-uniform running max per head
//                 (DPP row reduction), rescaling the accumulator only when
//                 the max grows.
//   PV         = VALU FMA in float32 over value tiles loaded as contiguous
//                 1 KiB rows per instruction; the probabilities reach the
//                 value layout through a 16 x GC LDS buffer per wave.
//   merge      = the 4 waves' (max, sum, acc) through LDS; a sequence that
//                 fits in one partition writes its output directly, longer
//                 ones write float32 partials merged by a second kernel.
//
// Masking: tokens at or beyond the context length in the last block are
// excluded by select (logit -inf, value zeroed), never by multiplying
// garbage by zero, so NaN-filled free slots cannot leak into the result.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * kWave;
constexpr int kDefaultPartition = 512;
constexpr int kMaxPartition = 4096;   // 256 blocks: 64 per wave, one id per lane

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
};

struct Tile {
  // K in MFMA-B layout (lane l: token l%16, chunks (l/16) + 4m), V as
  // contiguous 1-KiB slices (lane l: bytes ld*1024 + 16l of the tile).
  u32x4 k[8];
  u32x4 v[8];
};

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
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_float(q[m], e),
                                                   lane_float(t.k[m], e), acc, 0, 0, 0);
    }
  }
  return acc;
}

template <int DT, int D, int GC>
__global__ __launch_bounds__(kDecodeThreads) void paged_decode_kernel(
    void* __restrict__ out, const char* __restrict__ query,
    const char* __restrict__ kcache, const char* __restrict__ vcache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    float scale_log2, int num_kv_heads, int num_heads, int max_blocks,
    int64_t num_blocks, int partition_size, int num_parts,
    float* __restrict__ part_acc, float* __restrict__ part_m, float* __restrict__ part_s) {
  using C = DecodeCfg<DT, D, GC>;
  constexpr int NLD = C::kNld;

  __shared__ float sm_p[kDecodeWaves][kBlockSize * GC];
  __shared__ float sm_m[kDecodeWaves][GC];
  __shared__ float sm_s[kDecodeWaves][GC];
  __shared__ float sm_acc[kDecodeWaves][GC][D];

  const int head_groups = num_heads / GC;
  const int wg = blockIdx.x;
  const int p = wg % num_parts;
  const int hg = (wg / num_parts) % head_groups;
  const int s = wg / (num_parts * head_groups);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid >> 6;
  const int h0 = hg * GC;
  const int kvh = h0 / (num_heads / num_kv_heads);

  int L = context_lens[s];
  L = L < 0 ? 0 : (L > max_blocks * kBlockSize ? max_blocks * kBlockSize : L);
  const int tok0 = p * partition_size;
  if (tok0 >= L) {
    if (p == 0) {  // empty sequence: the output is zero
      for (int i = tid; i < GC * D; i += kDecodeThreads)
        store_elem<DT>(out, ((int64_t)s * num_heads + h0) * D + i, 0.f);
    }
    return;
  }
  const int tok1 = min(L, tok0 + partition_size);
  const int blk0 = tok0 / kBlockSize;
  const int nblk = (tok1 - tok0 + kBlockSize - 1) / kBlockSize;
  const int cnt = nblk > w ? (nblk - w + kDecodeWaves - 1) / kDecodeWaves : 0;

  // physical ids of this wave's blocks: lane i holds block blk0 + w + 4i
  int my_id = 0;
  if (lane < cnt) {
    int64_t b = block_tables[(int64_t)s * max_blocks + blk0 + w + kDecodeWaves * lane];
    b = b < 0 ? 0 : (b >= num_blocks ? num_blocks - 1 : b);
    my_id = (int)b;
  }

  // query rows as MFMA A operands: row r of chain c is head c*4 + r % kGcq
  const int row = lane & 15;
  const int jg = lane >> 4;
  u32x4 qa[C::kNqg][NLD];
#pragma unroll
  for (int c = 0; c < C::kNqg; ++c) {
    const int head = h0 + c * 4 + (row % C::kGcq);
    const char* qrow = query + ((int64_t)s * num_heads + head) * C::kRowB;
#pragma unroll
    for (int m = 0; m < NLD; ++m) qa[c][m] = load16(qrow + (jg + 4 * m) * 16);
  }

  const int64_t head_stride = (int64_t)C::kTileB;               // bytes per kv head
  const int64_t block_stride = (int64_t)num_kv_heads * C::kTileB;
  const uint32_t koff_lane = (uint32_t)(row * C::kRowB + jg * 16);
  const uint32_t voff_lane = (uint32_t)(lane * 16);

  auto load_tile = [&](Tile& t, int n) {
    const int id = __builtin_amdgcn_readlane(my_id, n);
    const char* kb = kcache + (int64_t)id * block_stride + kvh * head_stride;
    const char* vb = vcache + (int64_t)id * block_stride + kvh * head_stride;
#pragma unroll
    for (int m = 0; m < NLD; ++m) t.k[m] = load16(kb + koff_lane + m * 64);
#pragma unroll
    for (int m = 0; m < NLD; ++m) t.v[m] = load16(vb + voff_lane + m * 1024);
  };

  float m_run[GC], l_run[GC], acc[GC][C::kEpc];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < C::kEpc; ++e) acc[g][e] = 0.f;
  }
  float* pw = sm_p[w];

  auto compute_tile = [&](const Tile& t, int n) {
    const int lb = blk0 + w + kDecodeWaves * n;
    const int valid = L - lb * kBlockSize;  // >= 1; < 16 only in the last block
    float sc[GC];
#pragma unroll
    for (int c = 0; c < C::kNqg; ++c) {
      floatx4 r = qk_mfma<DT, NLD>(qa[c], t);
#pragma unroll
      for (int i = 0; i < C::kGcq; ++i) sc[c * 4 + i] = r[i] * scale_log2;
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
        for (int e = 0; e < C::kEpc; ++e) acc[g][e] *= alpha;
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
      for (int e = 0; e < C::kEpc; ++e) {
        const float f = elem_to_float<DT>(vv, e);
#pragma unroll
        for (int g = 0; g < GC; ++g) acc[g][e] = fmaf(pv[g], f, acc[g][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // two register tiles, alternating: load n+1 while computing n
  Tile ta, tb;
  if (cnt > 0) load_tile(ta, 0);
  for (int n = 0; n < cnt; n += 2) {
    if (n + 1 < cnt) load_tile(tb, n + 1);
    compute_tile(ta, n);
    if (n + 1 < cnt) {
      if (n + 2 < cnt) load_tile(ta, n + 2);
      compute_tile(tb, n + 1);
    }
  }

  // wave totals: sum over the 16 token lanes; acc over lanes sharing a chunk
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    l_run[g] = row_sum16(l_run[g]);
#pragma unroll
    for (int e = 0; e < C::kEpc; ++e) acc[g][e] = sum_over_lane_groups<C::kNch>(acc[g][e]);
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      sm_m[w][g] = m_run[g];
      sm_s[w][g] = l_run[g];
    }
  }
  if (lane < C::kNch) {
#pragma unroll
    for (int g = 0; g < GC; ++g)
#pragma unroll
      for (int e = 0; e < C::kEpc; ++e) sm_acc[w][g][lane * C::kEpc + e] = acc[g][e];
  }
  __syncthreads();

  const bool single = L <= partition_size;
  for (int i = tid; i < GC * D; i += kDecodeThreads) {
    const int g = i / D;
    const int d = i % D;
    float M = sm_m[0][g];
#pragma unroll
    for (int v = 1; v < kDecodeWaves; ++v) M = fmaxf(M, sm_m[v][g]);
    float S = 0.f, O = 0.f;
#pragma unroll
    for (int v = 0; v < kDecodeWaves; ++v) {
      const float wt = __builtin_amdgcn_exp2f(sm_m[v][g] - M);  // idle wave: 0
      S = fmaf(sm_s[v][g], wt, S);
      O = fmaf(sm_acc[v][g][d], wt, O);
    }
    const int h = h0 + g;
    if (single) {
      store_elem<DT>(out, ((int64_t)s * num_heads + h) * D + d, O / S);
    } else {
      const int64_t slot = ((int64_t)s * num_heads + h) * num_parts + p;
      part_acc[slot * D + d] = O;
      if (d == 0) {
        part_m[slot] = M;
        part_s[slot] = S;
      }
    }
  }
}

// Merge of the per-partition float32 states of sequences longer than one
// partition: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) s_p.
template <int DT, int D>
__global__ __launch_bounds__(kWave) void paged_decode_reduce_kernel(
    void* __restrict__ out, const int32_t* __restrict__ context_lens, int num_heads,
    int max_blocks, int partition_size, int num_parts, const float* __restrict__ part_acc,
    const float* __restrict__ part_m, const float* __restrict__ part_s) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int L = context_lens[s];
  L = L < 0 ? 0 : (L > max_blocks * kBlockSize ? max_blocks * kBlockSize : L);
  const int np = (L + partition_size - 1) / partition_size;
  if (np <= 1) return;
  const int64_t base = ((int64_t)s * num_heads + h) * num_parts;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, part_m[base + p]);
  constexpr int DPL = D / kWave;
  float O[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) O[i] = 0.f;
  float S = 0.f;
  for (int p = 0; p < np; ++p) {
    const float wt = __builtin_amdgcn_exp2f(part_m[base + p] - M);
    S = fmaf(wt, part_s[base + p], S);
    const float* a = part_acc + (base + p) * D;
#pragma unroll
    for (int i = 0; i < DPL; ++i) O[i] = fmaf(wt, a[threadIdx.x + i * kWave], O[i]);
  }
  const float inv = 1.f / S;
#pragma unroll
  for (int i = 0; i < DPL; ++i)
    store_elem<DT>(out, ((int64_t)s * num_heads + h) * D + threadIdx.x + i * kWave, O[i] * inv);
}

struct DecodeArgs {
  void* out;
  const void* query;
  const void* kcache;
  const void* vcache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale_log2;
  int num_kv_heads, num_seqs, num_heads, max_blocks;
  int64_t num_blocks;
  int partition_size, num_parts;
  float *part_acc, *part_m, *part_s;
};

template <int DT, int D, int GC>
static hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const int64_t nwg = (int64_t)a.num_parts * (a.num_heads / GC) * a.num_seqs;
  hipLaunchKernelGGL((paged_decode_kernel<DT, D, GC>), dim3((unsigned)nwg),
                     dim3(kDecodeThreads), 0, st, a.out, (const char*)a.query,
                     (const char*)a.kcache, (const char*)a.vcache, a.block_tables,
                     a.context_lens, a.scale_log2, a.num_kv_heads, a.num_heads,
                     a.max_blocks, a.num_blocks, a.partition_size, a.num_parts,
                     a.part_acc, a.part_m, a.part_s);
  if (a.num_parts > 1) {
    hipLaunchKernelGGL((paged_decode_reduce_kernel<DT, D>),
                       dim3(a.num_heads, a.num_seqs), dim3(kWave), 0, st, a.out,
                       a.context_lens, a.num_heads, a.max_blocks, a.partition_size,
                       a.num_parts, a.part_acc, a.part_m, a.part_s);
  }
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t dispatch_gc(const DecodeArgs& a, int gc, hipStream_t st) {
  switch (gc) {
    case 1: return launch_decode<DT, D, 1>(a, st);
    case 2: return launch_decode<DT, D, 2>(a, st);
    case 4: return launch_decode<DT, D, 4>(a, st);
    default: return launch_decode<DT, D, 8>(a, st);
  }
}

template <int DT>
static hipError_t dispatch_d(const DecodeArgs& a, int d, int gc, hipStream_t st) {
  return d == 64 ? dispatch_gc<DT, 64>(a, gc, st) : dispatch_gc<DT, 128>(a, gc, st);
}

static int resolve_partition(int partition_size) {
  return partition_size == 0 ? kDefaultPartition : partition_size;
}

static int num_partitions(int max_blocks_per_seq, int partition) {
  const int64_t max_tokens = (int64_t)max_blocks_per_seq * kBlockSize;
  return (int)((max_tokens + partition - 1) / partition);
}

static bool partition_ok(int ps) {
  return ps >= kBlockSize && ps <= kMaxPartition && ps % kBlockSize == 0;
}

}  // namespace pkv

extern "C" size_t paged_attention_workspace_bytes(int num_seqs, int num_heads,
                                                  int head_size, int max_blocks_per_seq,
                                                  int block_size, int partition_size) {
  using namespace pkv;
  if (num_seqs <= 0 || num_heads <= 0 || head_size <= 0 || max_blocks_per_seq <= 0 ||
      block_size != kBlockSize)
    return 0;
  const int ps = resolve_partition(partition_size);
  if (!partition_ok(ps)) return 0;
  const int np = num_partitions(max_blocks_per_seq, ps);
  if (np <= 1) return 0;
  return (size_t)num_seqs * num_heads * np * (head_size + 2) * sizeof(float);
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
  const int ps = resolve_partition(partition_size);
  if (!partition_ok(ps)) return PKV_ERR_INVALID_ARG;
  if (((uintptr_t)query | (uintptr_t)key_cache | (uintptr_t)value_cache) & 15u)
    return PKV_ERR_INVALID_ARG;  // tiles and query rows are read 16 bytes at a time
  if ((int64_t)max_blocks_per_seq * kBlockSize > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;

  const int np = num_partitions(max_blocks_per_seq, ps);
  const int group = num_heads / num_kv_heads;
  const int gc = group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
  // grid.x * block must fit in 32 bits
  if ((int64_t)np * (num_heads / gc) * num_seqs > (int64_t)(UINT32_MAX / kDecodeThreads))
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)num_seqs > 65535 && np > 1) return PKV_ERR_INVALID_ARG;  // merge grid.y

  DecodeArgs a{};
  a.out = out;
  a.query = query;
  a.kcache = key_cache;
  a.vcache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale_log2 = scale * 1.4426950408889634f;  // exp(x) = 2^(x log2 e)
  a.num_kv_heads = num_kv_heads;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.partition_size = ps;
  a.num_parts = np;
  if (np > 1) {
    const size_t need = paged_attention_workspace_bytes(num_seqs, num_heads, head_size,
                                                        max_blocks_per_seq, block_size, ps);
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    float* ws = (float*)workspace;
    const size_t rows = (size_t)num_seqs * num_heads * np;
    a.part_acc = ws;
    a.part_m = ws + rows * head_size;
    a.part_s = a.part_m + rows;
  }
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
