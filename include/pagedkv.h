/*
 * pagedkv.h -- C ABI of the paged KV-cache decode library for MI355X (gfx950).
 *
 * Three operations on a shared pool of fixed 16-token key/value blocks:
 *
 *   paged_attention_decode  one decode step of attention per (sequence,
 *                           query head), reading keys and values through
 *                           each sequence's block table;
 *   reshape_and_cache       scatter new tokens' keys/values to their slots;
 *   copy_blocks             block-level copy-on-write of shared blocks;
 * the first two again for pools of 8-bit float (E4M3) codes with one
 * scale per pool (paged_attention_decode_fp8, reshape_and_cache_fp8);
 *   paged_attention_decode_append  the first two fused for a decode step
 *                           in which every sequence appends one token; and
 *   paged_attention_prefill causal attention of a chunk of new tokens per
 *                           sequence (a whole prompt, or the next part of
 *                           one) over the cached tokens, on the same pools;
 *   paged_attention_decode_shared_prefix  decode for batches whose
 *                           sequences share leading blocks (samples, beams
 *                           of one prompt), each shared block read once.
 *
 * Sources (titles of the pages this library follows):
 *   [TEQ]  "Your GPU was mostly empty: how PagedAttention turned KV-cache
 *          waste into 2-4x throughput" (blog.teqners.com)
 *   [IV]   "vLLM and PagedAttention" (interviewsvector.com)
 *   [AITJ] "PagedAttention KV cache memory management" (aitechjournal.org)
 *   [VAS]  Vaswani et al., "Attention Is All You Need" (2017), eq. (1)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer argument is device memory owned by the caller
 * (the library allocates nothing and keeps no state beyond a per-device
 * memo of kernel occupancy and, for paged_attention_decode_noalloc only,
 * its fixed scratch array; calls are reentrant).
 * All tensors are dense, row-major, with no padding between rows.
 *
 * Element types (`dtype`): PKV_F32, PKV_F16 (IEEE binary16), PKV_BF16.
 * Queries, outputs, keys, values and both pools share one element type.
 *
 * Pool layout.  key_cache and value_cache are each
 *     [num_blocks][num_kv_heads][block_size][head_size]
 * so the 16 slots of one (block, kv head) are 16*head_size contiguous
 * elements.  Token t of a sequence lives in physical block
 * block_tables[s][t / 16] at slot t % 16.  The pages fix the block size
 * at 16 tokens ([TEQ] "The OS already solved this in the 1960s") and the
 * logical-to-physical block table ([AITJ] "How logical blocks, physical
 * blocks and the block table work"); the element layout inside the pool
 * is this library's choice.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Work is enqueued asynchronously; nothing synchronizes the host.
 *
 * Errors.  Every entry point returns PKV_OK (0) or a negative status, and
 * validates its scalar arguments before touching the device: on a nonzero
 * status nothing has been enqueued unless the status is PKV_ERR_HIP (the
 * launch itself failed).  Device-side contents are not validated on the
 * hot path; the kernels clamp what could address memory outside the
 * arguments (block ids, slots, pair entries) and skip those entries, so a
 * bad index gives wrong numbers for that sequence, never an out-of-bounds
 * access.  pkv_status_string() names a status.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats.  PKV_FP8_E4M3 is a KV-pool format only (the OCP 8-bit
 * float E4M3: bias 7, 3 mantissa bits, largest finite 448, S.1111.111 =
 * NaN): pools in it go with the _fp8 entry points and copy_blocks. */
enum pkv_dtype { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_FP8_E4M3 = 3 };

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,  /* null pointer, size <= 0, Hq % Hkv != 0 ... */
  PKV_ERR_UNSUPPORTED = -2,  /* block_size != 16, head_size not 64/128, dtype */
  PKV_ERR_WORKSPACE = -3,    /* split-context workspace missing or too small */
  PKV_ERR_HIP = -4           /* the HIP runtime reported a launch error */
};

/* ABI version of this header (bumped on any signature change). */
int pkv_abi_version(void);  /* 9 */

/* Human-readable name of a status code (static storage, never NULL). */
const char* pkv_status_string(int status);

/* Identifier of the sources this library was built from (a sha256 in hex,
 * static storage).  A binding compares it with its own sources to refuse a
 * library left over from older ones. */
const char* pkv_build_id(void);

/*
 * paged_attention_decode
 *
 * For every sequence s and query head h, with L = context_lens[s] and
 * kv head g = h / (num_heads / num_kv_heads):
 *     out[s][h] = sum_t softmax_t(scale * q[s][h] . k_t) v_t,  t = 0..L-1,
 * where k_t, v_t are token t's key and value in kv head g, read from the
 * pools through block_tables[s] ([VAS] eq. (1); keys and values are
 * read through the sequence's table, [IV] "Architecture, step by step",
 * step 3).  L counts every cached token, including the one written
 * this step.  L = 0 gives out[s][h] = 0.  Slots at or past L and blocks
 * past ceil(L/16) are never used, whatever they hold (NaN included).
 *
 *   out           [num_seqs][num_heads][head_size]     written
 *   query         [num_seqs][num_heads][head_size]
 *   key_cache     [num_blocks][num_kv_heads][16][head_size]
 *   value_cache   same layout as key_cache
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entries at
 *                 n >= ceil(L/16) are ignored (any value)
 *   context_lens  int32 [num_seqs]; values are clamped to
 *                 [0, 16*max_blocks_per_seq]
 *   scale         the softmax scale (typically 1/sqrt(head_size); any finite
 *                 float: a negative one weighs the smallest logits most,
 *                 zero weighs the visible tokens equally)
 *   num_kv_heads  kv heads; num_heads must be a multiple of it
 *   num_blocks    pool size in blocks; block ids outside [0, num_blocks)
 *                 are clamped into it (wrong output, no fault)
 *   partition_size  0 (default): every sequence's context is split wherever
 *                 the load balance puts it; otherwise the most tokens one
 *                 piece of a split context may hold, a multiple of 16 in
 *                 [16, 4096].  Pieces are computed in float32 (running max,
 *                 sum, unnormalized output) and merged exactly as one
 *                 softmax over the whole context.
 *   workspace     device scratch of at least
 *                 paged_attention_workspace_bytes(...) bytes, 16-byte
 *                 aligned; caller-owned, contents need no initialization.
 *                 Calls that use one workspace must not overlap (one
 *                 stream, or ordered).
 *   block_shared  optional (NULL allowed): uint8 [num_blocks], device
 *                 memory, nonzero for a block that more than one sequence
 *                 of the batch maps -- the runtime's reference count above
 *                 one ([TEQ] "Paging's second gift: copy-on-write").  It
 *                 only chooses how tiles are cached: a shared block's tiles
 *                 are kept in L2 for its other readers, every other tile is
 *                 streamed past the cache.  With flags, a batch of at most
 *                 512 sequences is also worked through sorted by each
 *                 sequence's first block, so siblings (samples, beams of
 *                 one request), which share it, are read together wherever
 *                 they sit in the batch.  The flags' values never change
 *                 the result; a call with flags may cut the contexts into
 *                 pieces elsewhere than one without, so the two can differ
 *                 by rounding (both within the stated accuracy).  NULL: the
 *                 batch order is kept, and a block counts as shared when
 *                 the previous or the next sequence maps it at the same
 *                 index, so siblings must sit side by side to keep their
 *                 prompt blocks in cache.
 *
 * Work is balanced over the GPU: the grid holds two waves per SIMD, each
 * streaming an equal share of all (block, kv head) tiles of the batch,
 * whatever the mix of context lengths.  Batches of more than 2048
 * sequences run as consecutive launches of 2048.
 *
 * Accumulation is float32 for every dtype; the output is rounded to
 * nearest-even into `dtype`.  With 16-bit queries and four or more query
 * heads per kv head, both products run on the matrix cores: the
 * probabilities enter the second one as their 16-bit rounding plus the
 * remainder of that rounding, so it keeps float32 accuracy.
 * num_seqs * max_blocks_per_seq * (num_heads / heads per workgroup) must be
 * below 2^31.
 */
int paged_attention_decode(void* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           const int32_t* context_lens, float scale,
                           int num_kv_heads, int num_seqs, int num_heads,
                           int head_size, int block_size, int max_blocks_per_seq,
                           int64_t num_blocks, int partition_size,
                           void* workspace, size_t workspace_bytes, int dtype,
                           const uint8_t* block_shared, void* stream);

/*
 * paged_attention_decode_noalloc: paged_attention_decode without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The split-context workspace is a fixed device array of
 * PKV_NOALLOC_SCRATCH_BYTES inside the library, one per device the library
 * runs on, held until the process ends; the call allocates nothing (no
 * hipMalloc, no allocating library routine).  Its first call on a device
 * looks up that device's copy (with the device current).
 *
 * Arguments, results and errors are those of paged_attention_decode (16-
 * and 32-bit pools, no new-token rows, no block_shared flags: the
 * neighbour rule decides the cache policy), with one more: sizes whose
 * workspace would not fit the array -- ranges = max(waves of this device's
 * grid, tiles of one launch / (partition_size / 16)), laid out as the
 * workspace above for the head-group size this dtype uses -- return
 * PKV_ERR_WORKSPACE before anything is enqueued.
 *
 * Every call on one device shares that device's array, and the array keeps
 * the last call's contents (each call writes everything it reads, so
 * nothing needs clearing).  Calls that overlap on one device -- on two
 * streams, or from two threads without ordering -- race on it: order them.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, float scale,
                                   int num_kv_heads, int num_seqs, int num_heads,
                                   int head_size, int block_size, int max_blocks_per_seq,
                                   int64_t num_blocks, int partition_size, int dtype,
                                   void* stream);

/*
 * Bytes of workspace paged_attention_decode needs for these sizes.  One
 * launch (at most 2048 sequences) splits its (block, kv head) tiles into at
 * most ranges = max(4096, tiles / (partition_size / 16)) equal ranges; the
 * workspace holds a 256-byte header, two 16-byte descriptors per range and
 * two float32 partial states per range (head_size + 2 floats for each query
 * head of a group: up to 16 heads with 16-bit queries when a kv head serves
 * more than 8, else up to 8), each part rounded up to 256 bytes.  Depends only on the
 * arguments (no device query).  Returns 0 for invalid sizes, which
 * paged_attention_decode then rejects.
 */
size_t paged_attention_workspace_bytes(int num_seqs, int num_heads,
                                       int num_kv_heads, int head_size,
                                       int max_blocks_per_seq, int block_size,
                                       int partition_size);

/*
 * reshape_and_cache
 *
 * Writes new tokens' keys and values into their slots of the pools: for
 * each i with slot = slot_mapping[i] >= 0,
 *     key_cache[slot / 16][g][slot % 16][:] = key[i][g][:]   for every g,
 * and the same for value.  This is the write that prefill performs for the
 * prompt and every decode step performs for its new token ([AITJ] "A
 * request lifecycle: allocation, growth, sharing and release"); choosing
 * the slot (and allocating a fresh block when the current one is full) is
 * the caller's.  The copy is bit-exact.  A negative slot skips the token;
 * a slot >= 16*num_blocks is skipped as well.  Two tokens with the same
 * slot race (undefined which one lands).
 *
 *   key, value    [num_tokens][num_kv_heads][head_size]
 *   slot_mapping  int64 [num_tokens]
 *   key_cache, value_cache  pools as above (modified in place)
 *
 * num_tokens = 0 is a valid no-op (key, value and slot_mapping may then be
 * NULL).
 */
int reshape_and_cache(const void* key, const void* value,
                      const int64_t* slot_mapping, void* key_cache,
                      void* value_cache, int num_tokens, int num_kv_heads,
                      int head_size, int block_size, int64_t num_blocks,
                      int dtype, void* stream);

/*
 * copy_blocks
 *
 * Block-level copy-on-write ([TEQ] "Paging's second gift: copy-on-write"):
 * for each pair (src, dst) = (src_dst_pairs[2i], src_dst_pairs[2i+1]) the
 * whole block -- all kv heads, all 16 slots -- is copied, bit-exact, in both
 * pools:  key_cache[dst] = key_cache[src], value_cache[dst] = value_cache[src].
 * Pairs are applied as if at once: destinations must be distinct and no
 * destination may also be a source (else the result is undefined).  A pair
 * with an entry outside [0, num_blocks) is skipped.  Deciding which block
 * to copy (the reference count) is the caller's.
 *
 *   src_dst_pairs  int64 [num_pairs][2], device memory
 *
 * num_pairs = 0 is a valid no-op (src_dst_pairs may then be NULL).
 */
int copy_blocks(void* key_cache, void* value_cache, const int64_t* src_dst_pairs,
                int num_pairs, int num_kv_heads, int head_size, int block_size,
                int64_t num_blocks, int dtype, void* stream);

/*
 * fp8 KV pools.  A pool may hold E4M3 codes (one byte per element, same
 * [num_blocks][num_kv_heads][16][head_size] layout) with one float32 scale
 * per pool: the key element a code stands for is e4m3(code) * k_scale, the
 * value element e4m3(code) * v_scale.  Half the bytes of a 16-bit pool per
 * token, so twice the tokens per byte of HBM ([AITJ] "PagedAttention vs
 * KV-cache quantization vs prefix caching": quantization changes how
 * densely cached tensors are stored, paging where they are stored).
 * copy_blocks moves such pools with dtype = PKV_FP8_E4M3.
 *
 * reshape_and_cache_fp8: as reshape_and_cache, but each element x of
 * key[i] (of `dtype`, 16- or 32-bit) is stored as the code nearest to the
 * float32 quotient x / k_scale (values: / v_scale), ties to the even
 * mantissa; quotients of magnitude >= 448 (inf included) saturate to
 * +-448, NaN becomes 0x7F.  Scales must be finite and > 0.
 */
int reshape_and_cache_fp8(const void* key, const void* value,
                          const int64_t* slot_mapping, void* key_cache,
                          void* value_cache, float k_scale, float v_scale,
                          int num_tokens, int num_kv_heads, int head_size,
                          int block_size, int64_t num_blocks, int dtype,
                          void* stream);

/*
 * paged_attention_decode_append: one decode step that also caches the
 * step's token -- reshape_and_cache followed by paged_attention_decode, in
 * one launch.  For every sequence s with L = context_lens[s] >= 1, token
 * L - 1 is the new one: its key and value rows new_key[s], new_value[s]
 * ([num_seqs][num_kv_heads][head_size], `dtype`, 16-byte aligned) are
 * written into its slot, block_tables[s][(L-1)/16] * 16 + (L-1) % 16
 * ([TEQ] "The OS already solved this in the 1960s": a token's slot comes
 * from the table), and the attention over tokens 0 .. L-1 uses them.  The
 * result equals reshape_and_cache of those rows to those slots followed by
 * paged_attention_decode (same arguments otherwise).  The block holding a
 * new token must not be shared (copy it first, as for reshape_and_cache).
 * Pools in `dtype` (E4M3 pools: paged_attention_decode_append_fp8).
 * Sequences with L = 0 write nothing.
 */
int paged_attention_decode_append(void* out, const void* query, void* key_cache,
                                  void* value_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, const void* new_key,
                                  const void* new_value, float scale, int num_kv_heads,
                                  int num_seqs, int num_heads, int head_size,
                                  int block_size, int max_blocks_per_seq,
                                  int64_t num_blocks, int partition_size,
                                  void* workspace, size_t workspace_bytes, int dtype,
                                  const uint8_t* block_shared, void* stream);

/*
 * paged_attention_decode_fp8: paged_attention_decode over E4M3 pools, the
 * keys and values being the codes' values times k_scale and v_scale.
 * query and out are `dtype` (PKV_F16 or PKV_BF16); every other argument,
 * the workspace (paged_attention_workspace_bytes with the same sizes) and
 * the error behaviour are those of paged_attention_decode.  Codes widen
 * exactly to `dtype` for the QK products (float32 accumulation); the
 * scales are applied in float32.
 */
int paged_attention_decode_fp8(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               const int32_t* context_lens, float scale, float k_scale,
                               float v_scale, int num_kv_heads, int num_seqs,
                               int num_heads, int head_size, int block_size,
                               int max_blocks_per_seq, int64_t num_blocks,
                               int partition_size, void* workspace,
                               size_t workspace_bytes, int dtype,
                               const uint8_t* block_shared, void* stream);

/*
 * paged_attention_decode_append_fp8: the appending decode step over E4M3
 * pools -- reshape_and_cache_fp8 of each sequence's newest token followed
 * by paged_attention_decode_fp8, in one launch.  For every sequence s with
 * L = context_lens[s] >= 1, token L - 1 is the new one: its key and value
 * rows new_key[s], new_value[s] ([num_seqs][num_kv_heads][head_size],
 * `dtype`, PKV_F16 or PKV_BF16) are encoded as reshape_and_cache_fp8
 * encodes them (the code nearest to the float32 quotient by k_scale /
 * v_scale, ties to even, saturating at +-448, NaN to 0x7F), the codes are
 * written to the token's slot, block_tables[s][(L-1)/16] * 16 + (L-1) % 16
 * ([TEQ] "The OS already solved this in the 1960s"), and the attention
 * over tokens 0 .. L-1 uses them.  The result -- pools and outputs -- equals
 * reshape_and_cache_fp8 of those rows to those slots followed by
 * paged_attention_decode_fp8 with the same arguments.  The block holding a
 * new token must not be shared.  Sequences with L = 0 write nothing.
 * Other arguments, workspace and errors as for paged_attention_decode_fp8.
 */
int paged_attention_decode_append_fp8(void* out, const void* query, void* key_cache,
                                      void* value_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, const void* new_key,
                                      const void* new_value, float scale, float k_scale,
                                      float v_scale, int num_kv_heads, int num_seqs,
                                      int num_heads, int head_size, int block_size,
                                      int max_blocks_per_seq, int64_t num_blocks,
                                      int partition_size, void* workspace,
                                      size_t workspace_bytes, int dtype,
                                      const uint8_t* block_shared, void* stream);

/*
 * paged_attention_prefill
 *
 * The new tokens of each sequence attend causally to its cached tokens:
 * the prompt (or the next chunk of it) has been written into the blocks
 * the runtime assigned ([AITJ] "A request lifecycle: allocation, growth,
 * sharing and release"), and each new token sees every token up to its
 * own position, the decoder's masked self-attention ([VAS] section 3.2.3,
 * eq. (1)); keys and values are read through the block table as in
 * decoding ([IV] "Architecture, step by step", step 3).
 *
 * Sequence s owns the n_s = query_start_loc[s+1] - query_start_loc[s]
 * rows query_start_loc[s] .. +n_s-1 of `query` and `out`.  With
 * L = context_lens[s] (clamped to [0, 16*max_blocks_per_seq]), those rows
 * are the sequence's last n_s tokens, whose keys and values are already in
 * the pools: row i sits at position L - n_s + i and, for every query head
 * h with kv head g = h / (num_heads / num_kv_heads),
 *     out[row][h] = sum_t softmax_t(scale * q[row][h] . k_t) v_t,
 *     t = 0 .. L - n_s + i.
 * n_s = L is a whole prompt; n_s < L a chunk after a cached prefix.
 *
 *   out, query       [total rows][num_heads][head_size], `dtype`
 *                    (PKV_F16 or PKV_BF16); query 16-byte aligned, out
 *                    8-byte aligned
 *   key_cache, value_cache, block_tables, num_blocks, scale: as for
 *                    paged_attention_decode (pools in `dtype`)
 *   query_start_loc  int32 [num_seqs + 1], non-decreasing from 0
 *   max_query_len    at least every n_s (sizes the grid; rows of a
 *                    sequence beyond it are not written); n_s <= L
 *
 * Work: one workgroup per 128 rows of one (sequence, kv head), rows being
 * (new token, query head of the group) pairs; keys are walked 32 at a
 * time through LDS and both products run on MFMA with float32
 * accumulation.  The probabilities enter the second product rounded to
 * `dtype`.  No workspace.
 *
 * Masking: keys past a row's position get probability 0 by selection, and
 * tokens past the context are read as zeros, so whatever the pools hold
 * there never reaches a result.  In the 32-key steps that mask keys for
 * some rows of a workgroup, the values of the keys past its earliest row
 * are made finite before the second product (an infinity or NaN becomes
 * the largest finite value of its sign, NaN: +): rows that do not see such
 * a key are exact, rows that do see a non-finite value there get that
 * largest value in its place rather than an infinity or NaN.
 *
 * The scale may be any finite float: a negative one is applied by
 * flipping the queries' signs, and zero weighs the visible tokens equally
 * (it is taken as 1e-30 / log2 e, equal weights to float32 precision).
 *
 * Errors: INVALID_ARG for null pointers, sizes
 * out of range, Hq % Hkv != 0, misalignment or a non-finite scale;
 * UNSUPPORTED for other dtypes, block_size != 16 or head_size not 64/128.
 * Device-side contents
 * (tables, lengths, query_start_loc) are not validated; every read stays
 * inside the buffers whatever they hold, provided query_start_loc
 * describes rows of `query`.
 */
int paged_attention_prefill(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* query_start_loc,
                            float scale, int num_kv_heads, int num_seqs, int num_heads,
                            int head_size, int block_size, int max_blocks_per_seq,
                            int64_t num_blocks, int max_query_len, int dtype,
                            void* stream);

/*
 * paged_attention_decode_shared_prefix -- paged_attention_decode for a
 * batch whose sequences share leading blocks, reading each shared block
 * once for all the sequences that map it.
 *
 * Sequences forked from one prompt (parallel samples, beams) map the
 * prompt's blocks to the same physical blocks, each block counting its
 * sharers, until one of them writes into a block and gets a private copy
 * ([TEQ] "Paging's second gift: copy-on-write"; [AITJ] "A request
 * lifecycle: allocation, growth, sharing and release").  The caller, which
 * keeps those reference counts, names the groups:
 *
 *   order          int32 [num_seqs], device, or NULL (the identity): a
 *                  permutation of the sequences; groups are runs of
 *                  consecutive positions in it, so the members of a group
 *                  need not sit side by side in the batch
 *   group_start    int32 [num_groups + 1], device: group j is the
 *                  sequences at positions group_start[j] ..
 *                  group_start[j+1] - 1 of `order`; increasing from 0 to
 *                  num_seqs (so every sequence is in one group; a
 *                  sequence that shares nothing is a group of its own)
 *   prefix_blocks  int32 [num_groups], device: every member of group j
 *                  holds the same block ids in its first prefix_blocks[j]
 *                  table entries.  The library uses at most the full
 *                  blocks of the group's shortest member (so a shared
 *                  block holds 16 cached tokens of every member)
 *   num_groups     0 .. num_seqs; 0: nothing is shared (both pointers may
 *                  be NULL)
 *
 * The other arguments are as for paged_attention_decode; the result is
 * the same attention, merged exactly in float32 from pieces of at most 128
 * tokens.  Each (shared block, kv head) is read once for the query rows
 * of every member of its group (up to 16 rows per read, member-major);
 * each sequence's blocks after its group's shared ones are read for it
 * alone.  A first kernel leaves a float32 state (max, sum, unnormalized
 * output) per (sequence, head, piece) in the workspace, a second merges
 * each row's pieces into `out`.
 *
 *   dtype        PKV_F16 or PKV_BF16 (pools in `dtype`)
 *   num_seqs     at most 2048
 *   workspace    at least paged_attention_shared_prefix_workspace_bytes()
 *                bytes, 16-byte aligned, caller-owned, contents need no
 *                initialization; calls that use one workspace must not
 *                overlap
 *
 * Errors: INVALID_ARG for null pointers (group pointers only when
 * num_groups > 0), sizes out of range, Hq % Hkv != 0 or misalignment;
 * UNSUPPORTED for other dtypes, block_size != 16, head_size not 64/128,
 * more than 2048 sequences or more groups than sequences; WORKSPACE when
 * the workspace is missing or too small.  Device-side contents are not
 * validated: order entries are clamped into [0, num_seqs), group starts
 * into [0, num_seqs], shared counts into [0, max_blocks_per_seq] and block
 * ids into the pool, so a wrong description (or an order that is not a
 * permutation) gives wrong numbers, never an access outside the buffers.
 */
int paged_attention_decode_shared_prefix(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* order,
    const int32_t* group_start, const int32_t* prefix_blocks, int num_groups, float scale,
    int num_kv_heads, int num_seqs, int num_heads, int head_size, int block_size,
    int max_blocks_per_seq, int64_t num_blocks, void* workspace, size_t workspace_bytes,
    int dtype, void* stream);

/* Workspace bytes paged_attention_decode_shared_prefix needs for these
 * sizes (0 when they are out of range: num_seqs outside 1..2048 or a size
 * <= 0).  No device access. */
size_t paged_attention_shared_prefix_workspace_bytes(int num_seqs, int num_heads,
                                                     int head_size, int max_blocks_per_seq);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
