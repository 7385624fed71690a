/*
 * pkv_vpool.h -- a virtually contiguous KV pool on the HIP virtual-memory
 * interface, for comparing paged and virtually contiguous caches with the
 * same attention kernels.
 *
 * The pages contrast block tables inside the attention kernel with keeping
 * each request's cache contiguous in virtual memory and backing it with
 * physical pages on demand through the driver's virtual-memory interface
 * (vAttention; [TEQ] "The tradeoff: you just wrote a virtual memory
 * subsystem in userspace").  A pkv_vpool reserves one virtual range per
 * tensor (keys, values) laid out like a paged pool,
 *     [num_blocks][num_kv_heads][16][head_size],
 * and maps physical memory behind it in granules (one allocation each)
 * only where asked.
 * Giving sequence s the virtual blocks base_s, base_s + 1, ... makes its
 * cache virtually contiguous; paged_attention_decode and the other calls
 * of pagedkv.h then run on it unchanged (key_cache = pkv_vpool_keys(p),
 * value_cache = pkv_vpool_values(p), num_blocks as created).
 *
 * Host-side calls, on the current device; not thread-safe per pool.
 * Reading a block that is not mapped is a GPU memory fault: check
 * pkv_vpool_covers for every block a launch will read.
 *
 * Statuses are those of pagedkv.h (PKV_OK, PKV_ERR_INVALID_ARG,
 * PKV_ERR_HIP when the virtual-memory interface refuses).
 */
#ifndef PKV_VPOOL_H_
#define PKV_VPOOL_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_vpool pkv_vpool;

/* Reserve num_blocks blocks of block_bytes bytes (a multiple of 256) for
 * keys and the same for values, and map the first granule of each (so the
 * base addresses are backed).  Granule = the device's recommended
 * allocation granularity, at least 2 MiB.  *out receives the pool (NULL on
 * error).  The caller owns it: pkv_vpool_destroy. */
int pkv_vpool_create(int64_t num_blocks, int64_t block_bytes, pkv_vpool** out);

/* Back blocks [first_block, first_block + count) of both tensors with
 * physical memory (whole granules; already mapped granules are kept, and
 * their contents too).  On PKV_ERR_HIP the granules mapped before the
 * failure stay mapped. */
int pkv_vpool_map(pkv_vpool* pool, int64_t first_block, int64_t count);

/* 1 if every granule holding blocks [first_block, first_block + count) is
 * mapped, else 0 (also 0 for a range outside the pool). */
int pkv_vpool_covers(const pkv_vpool* pool, int64_t first_block, int64_t count);

/* Device addresses of the two reserved ranges. */
void* pkv_vpool_keys(const pkv_vpool* pool);
void* pkv_vpool_values(const pkv_vpool* pool);

/* Granule size in bytes, and physical bytes mapped (both tensors). */
int64_t pkv_vpool_granularity(const pkv_vpool* pool);
int64_t pkv_vpool_mapped_bytes(const pkv_vpool* pool);

/* Unmap, release and unreserve everything (NULL is a no-op).  No launch
 * that reads the pool may still be running. */
void pkv_vpool_destroy(pkv_vpool* pool);

#ifdef __cplusplus
}
#endif

#endif /* PKV_VPOOL_H_ */
