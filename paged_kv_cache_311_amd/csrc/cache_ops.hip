// Pool maintenance kernels for gfx950: reshape_and_cache and copy_blocks.
//
// reshape_and_cache writes each new token's key and value rows into the
// slot the runtime assigned to it: prefill fills the blocks given to the
// prompt and every decode step appends one token, a fresh block being
// taken from the pool when the current one is full ("PagedAttention KV
// cache memory management" [AITJ], "A request lifecycle: allocation,
// growth, sharing and release").  copy_blocks is the copy half of
// block-level copy-on-write: a sequence about to write into a block that
// others still reference gets its own copy first ("Your GPU was mostly
// empty..." [TEQ], "Paging's second gift: copy-on-write").
//
// Both are pure data movement (bit-exact, dtype-agnostic): every thread
// moves 16-byte chunks with dwordx4 loads and stores.  reshape_and_cache_fp8
// writes into pools of 8-bit float (E4M3) codes: each new element becomes
// the code of its float32 quotient by the pool's scale ("PagedAttention KV
// cache memory management" [AITJ], "PagedAttention vs KV-cache quantization
// vs prefix caching").

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {

constexpr int kCopyThreads = 256;

// One thread per (token, kv head, 16-B chunk of the row); K and V both.
__global__ __launch_bounds__(kCopyThreads) void reshape_and_cache_kernel(
    const char* __restrict__ key, const char* __restrict__ value,
    const int64_t* __restrict__ slot_mapping, char* __restrict__ kcache,
    char* __restrict__ vcache, int64_t total_chunks, int num_kv_heads, int row_bytes,
    int64_t num_slots) {
  const int64_t idx = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x;
  if (idx >= total_chunks) return;
  const int nch = row_bytes >> 4;
  const int c = (int)(idx % nch);
  const int64_t th = idx / nch;  // token * num_kv_heads + head
  const int g = (int)(th % num_kv_heads);
  const int64_t i = th / num_kv_heads;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;  // padding / out of the pool
  const int64_t blk = slot / kBlockSize;
  const int off = (int)(slot % kBlockSize);
  const int64_t src = th * row_bytes + c * 16;
  const int64_t dst = ((blk * num_kv_heads + g) * kBlockSize + off) * row_bytes + c * 16;
  store16(kcache + dst, load16(key + src));
  store16(vcache + dst, load16(value + src));
}

// One thread per (token, kv head, 4 elements of the row): 4 input elements
// (8 or 16 bytes) become 4 E4M3 codes (4 bytes).  The encode is a chain of
// dependent float operations per element, so few elements per thread keep
// the kernel short when only one token per sequence is written.
constexpr int kFp8Group = 4;

template <int DT>
__device__ __forceinline__ u32x4 load_group4(const char* p) {
  if constexpr (Elt<DT>::kBytes == 4) {
    return load16(p);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return u32x4{w.x, w.y, 0u, 0u};
  }
}

template <int DT>
__global__ __launch_bounds__(kCopyThreads) void reshape_and_cache_fp8_kernel(
    const char* __restrict__ key, const char* __restrict__ value,
    const int64_t* __restrict__ slot_mapping, char* __restrict__ kcache,
    char* __restrict__ vcache, float k_scale, float v_scale, int64_t total_groups,
    int num_kv_heads, int head_size, int64_t num_slots) {
  const int64_t idx = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x;
  if (idx >= total_groups) return;
  const int ngr = head_size / kFp8Group;
  const int c = (int)(idx % ngr);
  const int64_t th = idx / ngr;  // token * num_kv_heads + head
  const int g = (int)(th % num_kv_heads);
  const int64_t i = th / num_kv_heads;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;  // padding / out of the pool
  const int64_t blk = slot / kBlockSize;
  const int off = (int)(slot % kBlockSize);
  const int64_t src = (th * head_size + c * kFp8Group) * Elt<DT>::kBytes;
  const int64_t dst = ((blk * num_kv_heads + g) * kBlockSize + off) * head_size + c * kFp8Group;
  auto quantize = [&](const char* in, float scale) {
    const u32x4 x = load_group4<DT>(in);
    uint32_t codes = 0u;
#pragma unroll
    for (int e = 0; e < kFp8Group; ++e)
      codes |= e4m3_code(elem_to_float<DT>(x, e) / scale) << (8 * e);
    return codes;
  };
  *reinterpret_cast<uint32_t*>(kcache + dst) = quantize(key + src, k_scale);
  *reinterpret_cast<uint32_t*>(vcache + dst) = quantize(value + src, v_scale);
}

// grid.x = pair, grid.y = slice of the block; each thread copies kUnroll
// 16-B chunks of K and of V, consecutive threads on consecutive chunks.
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    char* __restrict__ kcache, char* __restrict__ vcache, const int64_t* __restrict__ pairs,
    int64_t block_bytes, int64_t num_blocks) {
  const int64_t src = pairs[2 * (int64_t)blockIdx.x];
  const int64_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t chunks = block_bytes >> 4;
  const int64_t c0 = (int64_t)blockIdx.y * kCopyThreads * kCopyUnroll + threadIdx.x;
  const char* ks = kcache + src * block_bytes;
  const char* vs = vcache + src * block_bytes;
  char* kd = kcache + dst * block_bytes;
  char* vd = vcache + dst * block_bytes;
  u32x4 kr[kCopyUnroll], vr[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t c = c0 + (int64_t)u * kCopyThreads;
    if (c < chunks) {
      kr[u] = load16(ks + c * 16);
      vr[u] = load16(vs + c * 16);
    }
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t c = c0 + (int64_t)u * kCopyThreads;
    if (c < chunks) {
      store16(kd + c * 16, kr[u]);
      store16(vd + c * 16, vr[u]);
    }
  }
}

static int elem_bytes(int dtype) {
  return dtype == PKV_F32 ? 4 : (dtype == PKV_F16 || dtype == PKV_BF16) ? 2
                                                                        : dtype == PKV_FP8_E4M3 ? 1 : 0;
}

}  // namespace pkv

extern "C" int reshape_and_cache(const void* key, const void* value,
                                 const int64_t* slot_mapping, void* key_cache,
                                 void* value_cache, int num_tokens, int num_kv_heads,
                                 int head_size, int block_size, int64_t num_blocks, int dtype,
                                 void* stream) {
  using namespace pkv;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_INVALID_ARG;
  if (!key_cache || !value_cache) return PKV_ERR_INVALID_ARG;
  if (num_tokens > 0 && (!key || !value || !slot_mapping)) return PKV_ERR_INVALID_ARG;
  const int eb = elem_bytes(dtype);
  if (eb == 0 || dtype == PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;  // fp8: the _fp8 call
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PKV_ERR_UNSUPPORTED;
  if (((uintptr_t)key | (uintptr_t)value | (uintptr_t)key_cache | (uintptr_t)value_cache) &
      15u)
    return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return PKV_OK;
  const int row_bytes = head_size * eb;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * (row_bytes / 16);
  const int64_t grid = (total + kCopyThreads - 1) / kCopyThreads;
  if (grid > (int64_t)(UINT32_MAX / kCopyThreads)) return PKV_ERR_INVALID_ARG;
  (void)hipGetLastError();
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0,
                     (hipStream_t)stream, (const char*)key, (const char*)value, slot_mapping,
                     (char*)key_cache, (char*)value_cache, total, num_kv_heads, row_bytes,
                     num_blocks * kBlockSize);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int copy_blocks(void* key_cache, void* value_cache, const int64_t* src_dst_pairs,
                           int num_pairs, int num_kv_heads, int head_size, int block_size,
                           int64_t num_blocks, int dtype, void* stream) {
  using namespace pkv;
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_INVALID_ARG;
  if (!key_cache || !value_cache) return PKV_ERR_INVALID_ARG;
  if (num_pairs > 0 && !src_dst_pairs) return PKV_ERR_INVALID_ARG;
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PKV_ERR_UNSUPPORTED;
  if (((uintptr_t)key_cache | (uintptr_t)value_cache) & 15u) return PKV_ERR_INVALID_ARG;
  if (num_pairs == 0) return PKV_OK;
  const int64_t block_bytes = (int64_t)num_kv_heads * kBlockSize * head_size * eb;
  const int64_t per_wg = (int64_t)kCopyThreads * kCopyUnroll * 16;
  const int64_t slices = (block_bytes + per_wg - 1) / per_wg;
  if (slices > 65535) return PKV_ERR_INVALID_ARG;
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, (unsigned)slices),
                     dim3(kCopyThreads), 0, (hipStream_t)stream, (char*)key_cache,
                     (char*)value_cache, src_dst_pairs, block_bytes, num_blocks);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int reshape_and_cache_fp8(const void* key, const void* value,
                                     const int64_t* slot_mapping, void* key_cache,
                                     void* value_cache, float k_scale, float v_scale,
                                     int num_tokens, int num_kv_heads, int head_size,
                                     int block_size, int64_t num_blocks, int dtype,
                                     void* stream) {
  using namespace pkv;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_INVALID_ARG;
  if (!key_cache || !value_cache) return PKV_ERR_INVALID_ARG;
  if (num_tokens > 0 && (!key || !value || !slot_mapping)) return PKV_ERR_INVALID_ARG;
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale > 3.0e38f || v_scale > 3.0e38f)
    return PKV_ERR_INVALID_ARG;  // finite and positive (NaN fails both tests)
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PKV_ERR_UNSUPPORTED;
  if (((uintptr_t)key | (uintptr_t)value | (uintptr_t)key_cache | (uintptr_t)value_cache) &
      15u)
    return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return PKV_OK;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * (head_size / kFp8Group);
  const int64_t grid = (total + kCopyThreads - 1) / kCopyThreads;
  if (grid > (int64_t)(UINT32_MAX / kCopyThreads)) return PKV_ERR_INVALID_ARG;
  (void)hipGetLastError();
  const dim3 g3((unsigned)grid), b3(kCopyThreads);
  hipStream_t st = (hipStream_t)stream;
  const int64_t slots = num_blocks * kBlockSize;
  switch (dtype) {
    case PKV_F32:
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<PKV_F32>, g3, b3, 0, st, (const char*)key,
                         (const char*)value, slot_mapping, (char*)key_cache, (char*)value_cache,
                         k_scale, v_scale, total, num_kv_heads, head_size, slots);
      break;
    case PKV_F16:
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<PKV_F16>, g3, b3, 0, st, (const char*)key,
                         (const char*)value, slot_mapping, (char*)key_cache, (char*)value_cache,
                         k_scale, v_scale, total, num_kv_heads, head_size, slots);
      break;
    default:
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<PKV_BF16>, g3, b3, 0, st, (const char*)key,
                         (const char*)value, slot_mapping, (char*)key_cache, (char*)value_cache,
                         k_scale, v_scale, total, num_kv_heads, head_size, slots);
      break;
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

#ifndef PKV_BUILD_ID
#define PKV_BUILD_ID "unstamped"
#endif

extern "C" int pkv_abi_version(void) { return 9; }

extern "C" const char* pkv_build_id(void) { return PKV_BUILD_ID; }

extern "C" const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}
