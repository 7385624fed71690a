// Virtually contiguous KV pool (host code, HIP virtual-memory API).
//
// The pages weigh paging against the alternative that keeps each request's
// cache contiguous in virtual memory and lets the driver's virtual-memory
// interface map physical pages behind it on demand (vAttention; [TEQ] "The
// tradeoff: you just wrote a virtual memory subsystem in userspace").
// This pool gives the attention kernels exactly
// that: one reserved virtual range per tensor (keys, values) with the
// paged pool's layout [num_blocks][num_kv_heads][16][head_size], physical
// memory mapped in granules of the device's allocation granularity (one
// hipMemCreate allocation each, so their physical placement is the
// driver's) only where blocks are in use.  A caller that hands each
// sequence a run of consecutive virtual blocks gets a block table
// base, base+1, ...: the same kernels then read a virtually contiguous
// cache, and the difference from the paged layout is the cost of
// translation through block tables.
//
// The pool keeps, per granule, whether it is mapped; pkv_vpool_covers
// lets the caller check that every block a launch will read is backed
// before launching (a read of an unmapped address is a GPU memory fault).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>
#include <vector>

#include "pagedkv.h"
#include "pkv_vpool.h"

struct pkv_vpool {
  int device;
  int64_t num_blocks;
  int64_t block_bytes;
  size_t gran;                 // physical granule (allocation granularity)
  size_t bytes;                // reserved bytes per tensor (whole granules)
  void* base[2];               // keys, values
  std::vector<hipMemGenericAllocationHandle_t> h[2];
  std::vector<uint8_t> mapped;  // per granule, both tensors alike
  int64_t mapped_granules;
};

namespace {

constexpr size_t kMinGranule = size_t(2) << 20;

hipMemAllocationProp device_prop(int device) {
  hipMemAllocationProp prop = {};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

void release_all(pkv_vpool* p) {
  for (int t = 0; t < 2; ++t) {
    if (!p->base[t]) continue;
    for (size_t g = 0; g < p->mapped.size(); ++g) {
      if (!p->mapped[g]) continue;
      (void)hipMemUnmap((char*)p->base[t] + g * p->gran, p->gran);
      (void)hipMemRelease(p->h[t][g]);
    }
    (void)hipMemAddressFree(p->base[t], p->bytes);
    p->base[t] = nullptr;
  }
}

}  // namespace

extern "C" int pkv_vpool_create(int64_t num_blocks, int64_t block_bytes, pkv_vpool** out) {
  if (!out) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks <= 0 || block_bytes <= 0 || block_bytes % 256 != 0) return PKV_ERR_INVALID_ARG;
  if (num_blocks > INT64_MAX / block_bytes) return PKV_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  const hipMemAllocationProp prop = device_prop(dev);
  // granule: the recommended granularity, at least 2 MiB (a multiple of
  // the minimum), so that a pool of gigabytes needs a few thousand maps
  size_t gmin = 0, grec = 0;
  if (hipMemGetAllocationGranularity(&gmin, &prop, hipMemAllocationGranularityMinimum) !=
          hipSuccess ||
      gmin == 0)
    return PKV_ERR_HIP;
  if (hipMemGetAllocationGranularity(&grec, &prop, hipMemAllocationGranularityRecommended) !=
      hipSuccess)
    grec = gmin;
  size_t gran = grec > kMinGranule ? grec : kMinGranule;
  gran = (gran + gmin - 1) / gmin * gmin;
  pkv_vpool* p = new (std::nothrow) pkv_vpool();
  if (!p) return PKV_ERR_INVALID_ARG;
  p->device = dev;
  p->num_blocks = num_blocks;
  p->block_bytes = block_bytes;
  p->gran = gran;
  const int64_t want = num_blocks * block_bytes;
  const int64_t granules = (want + (int64_t)gran - 1) / (int64_t)gran;
  p->bytes = (size_t)granules * gran;
  p->mapped.assign((size_t)granules, 0);
  p->mapped_granules = 0;
  for (int t = 0; t < 2; ++t) {
    p->base[t] = nullptr;
    p->h[t].assign((size_t)granules, hipMemGenericAllocationHandle_t{});
  }
  for (int t = 0; t < 2; ++t) {
    if (hipMemAddressReserve(&p->base[t], p->bytes, gran, nullptr, 0) != hipSuccess) {
      p->base[t] = nullptr;
      release_all(p);
      delete p;
      return PKV_ERR_HIP;
    }
  }
  // the first granule is always backed, so the base addresses are valid
  // device memory for pointer queries
  const int rc = pkv_vpool_map(p, 0, 1);
  if (rc != PKV_OK) {
    release_all(p);
    delete p;
    return rc;
  }
  *out = p;
  return PKV_OK;
}

extern "C" int pkv_vpool_map(pkv_vpool* p, int64_t first_block, int64_t count) {
  if (!p || first_block < 0 || count < 0 || first_block > p->num_blocks - count)
    return PKV_ERR_INVALID_ARG;
  if (count == 0) return PKV_OK;
  const int64_t g0 = first_block * p->block_bytes / (int64_t)p->gran;
  const int64_t g1 = ((first_block + count) * p->block_bytes - 1) / (int64_t)p->gran;
  const hipMemAllocationProp prop = device_prop(p->device);
  hipMemAccessDesc acc = {};
  acc.location.type = hipMemLocationTypeDevice;
  acc.location.id = p->device;
  acc.flags = hipMemAccessFlagsProtReadWrite;
  for (int64_t g = g0; g <= g1; ++g) {
    if (p->mapped[(size_t)g]) continue;
    hipMemGenericAllocationHandle_t hh[2];
    int made = 0;
    bool ok = true;
    for (int t = 0; t < 2 && ok; ++t) {
      char* va = (char*)p->base[t] + (size_t)g * p->gran;
      ok = hipMemCreate(&hh[t], p->gran, &prop, 0) == hipSuccess;
      if (!ok) break;
      ok = hipMemMap(va, p->gran, 0, hh[t], 0) == hipSuccess;
      if (!ok) {
        (void)hipMemRelease(hh[t]);
        break;
      }
      ++made;
      ok = hipMemSetAccess(va, p->gran, &acc, 1) == hipSuccess;
    }
    if (!ok) {  // undo this granule's tensors; earlier granules stay mapped
      for (int t = 0; t < made; ++t) {
        (void)hipMemUnmap((char*)p->base[t] + (size_t)g * p->gran, p->gran);
        (void)hipMemRelease(hh[t]);
      }
      return PKV_ERR_HIP;
    }
    p->h[0][(size_t)g] = hh[0];
    p->h[1][(size_t)g] = hh[1];
    p->mapped[(size_t)g] = 1;
    ++p->mapped_granules;
  }
  return PKV_OK;
}

extern "C" int pkv_vpool_covers(const pkv_vpool* p, int64_t first_block, int64_t count) {
  if (!p || first_block < 0 || count < 0 || first_block > p->num_blocks - count) return 0;
  if (count == 0) return 1;
  const int64_t g0 = first_block * p->block_bytes / (int64_t)p->gran;
  const int64_t g1 = ((first_block + count) * p->block_bytes - 1) / (int64_t)p->gran;
  for (int64_t g = g0; g <= g1; ++g)
    if (!p->mapped[(size_t)g]) return 0;
  return 1;
}

extern "C" void* pkv_vpool_keys(const pkv_vpool* p) { return p ? p->base[0] : nullptr; }
extern "C" void* pkv_vpool_values(const pkv_vpool* p) { return p ? p->base[1] : nullptr; }
extern "C" int64_t pkv_vpool_granularity(const pkv_vpool* p) {
  return p ? (int64_t)p->gran : 0;
}
extern "C" int64_t pkv_vpool_mapped_bytes(const pkv_vpool* p) {
  return p ? 2 * p->mapped_granules * (int64_t)p->gran : 0;
}

extern "C" void pkv_vpool_destroy(pkv_vpool* p) {
  if (!p) return;
  release_all(p);
  delete p;
}
