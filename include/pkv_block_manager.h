/*
 * pkv_block_manager.h -- host-side management of a paged KV-cache pool.
 *
 * The runtime side of paging: a pool of fixed-size blocks (16 token slots
 * each), a free list, one block table per sequence, reference counts for
 * blocks that several sequences share, copy-on-write when a sequence writes
 * into a shared block, and release when sequences finish.  Blocks are
 * taken on demand, one when a sequence's last block is full ("Your GPU was
 * mostly empty..." [TEQ], "The OS already solved this in the 1960s" and
 * "Paging's second gift: copy-on-write"; "PagedAttention KV cache memory
 * management" [AITJ], "A request lifecycle: allocation, growth, sharing and
 * release").
 *
 * The manager only does the bookkeeping: the slot it hands out for a token
 * is what reshape_and_cache writes, its block tables are what
 * paged_attention_decode reads, and its copy-on-write pairs are what
 * copy_blocks copies (pagedkv.h).  Host memory only; no GPU call.
 *
 * Also: a decode-loop simulator that serves a seeded stream of requests
 * under a fixed KV memory budget, once with this paged allocation and once
 * with per-request reservations of the maximum length, and reports how
 * much of the reserved memory held tokens.
 *
 * Error behaviour: every call returns a status (0 = OK, negative = error)
 * or a documented value; an operation that fails changes nothing.  Handles
 * are not thread-safe: one thread per manager, or external locking.
 */
#ifndef PKV_BLOCK_MANAGER_H
#define PKV_BLOCK_MANAGER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_bm_status {
  PKV_BM_OK = 0,
  PKV_BM_INVALID = -1,    /* bad argument, unknown or duplicate sequence id */
  PKV_BM_NO_BLOCKS = -5,  /* the pool has too few free blocks; nothing changed */
};

typedef struct pkv_bm pkv_bm; /* opaque */

/* ABI version of this header (bumped on any signature change). */
int pkv_bm_abi_version(void);

/*
 * A pool of num_blocks blocks of block_size token slots (block_size > 0).
 * Free blocks are handed out last-freed first; initially block 0 first.
 * Returns NULL on invalid sizes or allocation failure.
 */
pkv_bm* pkv_bm_create(int32_t num_blocks, int32_t block_size);
void pkv_bm_destroy(pkv_bm* bm);

int32_t pkv_bm_num_blocks(const pkv_bm* bm);
int32_t pkv_bm_block_size(const pkv_bm* bm);
int32_t pkv_bm_num_free(const pkv_bm* bm);
int32_t pkv_bm_num_sequences(const pkv_bm* bm);
/* References to a block (0 = free); -1 for an id outside the pool. */
int32_t pkv_bm_refcount(const pkv_bm* bm, int32_t block);
/* flags[b] = 1 where block b has more than one reference, else 0, for every
 * block of the pool (the block_shared argument of the decode calls of
 * pagedkv.h, once copied to the device).  n is the capacity of flags (at
 * least num_blocks).  Returns num_blocks, or PKV_BM_INVALID. */
int32_t pkv_bm_shared_flags(const pkv_bm* bm, uint8_t* flags, int32_t n);

/*
 * The group description of paged_attention_decode_shared_prefix (pagedkv.h)
 * for a batch of n sequences (positions 0..n-1 = seq_ids[0..n-1]):
 * sequences whose first block is a full block held by more than one
 * reference, and the same for all of them, form a group; order[0..n) is a
 * stable permutation of the positions putting each group's members side
 * by side (ordered by that first block, sequences without one last), group
 * j is positions group_start[j] .. group_start[j+1] - 1 of order, and
 * prefix_blocks[j] is the number of leading blocks every member holds in
 * common, full blocks only (0 for a group of one).  order and
 * prefix_blocks need room for n entries, group_start for n + 1;
 * *num_groups receives the count.  PKV_BM_INVALID for null pointers or an
 * unknown sequence (nothing written).
 */
int pkv_bm_prefix_groups(const pkv_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* order,
                         int32_t* group_start, int32_t* prefix_blocks, int32_t* num_groups);

/*
 * A new sequence seq_id holding num_tokens tokens (its prompt): takes
 * ceil(num_tokens / block_size) blocks.  PKV_BM_INVALID if seq_id exists or
 * num_tokens < 0; PKV_BM_NO_BLOCKS if the pool has too few free blocks.
 */
int pkv_bm_add_sequence(pkv_bm* bm, int64_t seq_id, int64_t num_tokens);

/*
 * A new sequence child that shares every block of parent (each block's
 * reference count goes up by one) and has parent's length.  No block is
 * taken.  PKV_BM_INVALID if parent is unknown or child exists.
 */
int pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child);

/*
 * Reserve the slot of sequence seq_id's next token and grow its length by
 * one.  *slot = physical block * block_size + offset in the block.
 *   - last block full (or none): a free block is appended to the table;
 *   - last block shared (reference count > 1) and the token would land in
 *     it: copy-on-write -- a free block replaces it in this sequence's
 *     table, its reference count drops by one, and *cow_src / *cow_dst
 *     receive the (old, new) pair for copy_blocks; otherwise both are -1.
 * PKV_BM_NO_BLOCKS (nothing changed) when a block is needed and none is
 * free; PKV_BM_INVALID for an unknown sequence or null pointers.
 */
int pkv_bm_append_slot(pkv_bm* bm, int64_t seq_id, int64_t* slot, int32_t* cow_src,
                       int32_t* cow_dst);

/*
 * append_slot for n sequences in order; slots[i] for seq_ids[i].  The
 * copy-on-write pairs are written to cow_pairs[2k], cow_pairs[2k+1] (room
 * for n pairs) and their count to *num_pairs.  On an error at sequence i,
 * sequences 0..i-1 keep their new slots and *num_done = i.
 */
int pkv_bm_append_slots(pkv_bm* bm, const int64_t* seq_ids, int32_t n, int64_t* slots,
                        int64_t* cow_pairs, int32_t* num_pairs, int32_t* num_done);

/*
 * Release a finished sequence: every block's reference count drops by one,
 * and blocks that reach zero return to the free list.
 */
int pkv_bm_free_sequence(pkv_bm* bm, int64_t seq_id);

/* Tokens of seq_id, or -1 if unknown. */
int64_t pkv_bm_seq_len(const pkv_bm* bm, int64_t seq_id);

/*
 * Block table of seq_id into table[0..width): its blocks in logical order,
 * -1 past the last.  Returns the number of blocks, -1 if seq_id is unknown
 * or the table is wider than width.
 */
int32_t pkv_bm_block_table(const pkv_bm* bm, int64_t seq_id, int32_t* table, int32_t width);

/*
 * Block tables [n][width] int32 and lengths [n] int32 of n sequences (the
 * decode kernel's inputs).  PKV_BM_INVALID if a sequence is unknown, a
 * table is wider than width or a length exceeds 2^31 - 1.
 */
int pkv_bm_block_tables(const pkv_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* tables,
                        int32_t width, int32_t* lens);

/*
 * Decode-loop simulator.
 *
 * A seeded stream of num_requests requests (splitmix64 from `seed`).
 * Request i has a final length L_i (prompt + generated tokens) drawn from
 * `lengths` and a prompt of P_i = clip(round(prompt_fraction * L_i), 1,
 * L_i - 1) tokens.  It is admitted (its prompt cached in one step, which
 * also yields its first new token), then gains one token per step until it
 * holds L_i tokens, and is released.  Both allocators serve the same stream
 * under the same budget of pool_tokens slots, admitting in arrival order
 * while the next request fits (continuous batching):
 *   paged -- blocks of block_size taken on demand through this manager; a
 *            request is admitted when its prompt's blocks plus one more,
 *            plus a watermark of 1% of the pool's blocks, are free (no
 *            watermark while nothing runs).  When a running sequence needs
 *            a block and none is free, the most recently admitted one is
 *            preempted: its blocks are released and it rejoins the head of
 *            the queue, to have everything it held computed again.
 *   slab  -- each admitted request reserves max_len slots (the maximum
 *            length) until it finishes; equal slabs, so no external
 *            fragmentation is counted.
 * Utilization = (token slots holding tokens) / (slots reserved), summed
 * over every step; waste = 1 - utilization.
 */
enum pkv_sim_lengths {
  PKV_SIM_UNIFORM = 0,   /* L ~ U{min_len .. max_len} */
  PKV_SIM_LOGNORMAL = 1, /* L = clip(rint(exp(N(ln median, sigma^2))), min_len, max_len) */
};

typedef struct {
  int64_t num_requests;
  int32_t lengths;        /* pkv_sim_lengths */
  int32_t min_len, max_len;  /* 2 <= min_len <= max_len */
  double median, sigma;   /* lognormal only */
  double prompt_fraction; /* in [0, 1] */
  int64_t pool_tokens;    /* memory budget in token slots, at least
                             (ceil(max_len / block_size) + 1) * block_size */
  int32_t block_size;
  uint64_t seed;
} pkv_sim_config;

typedef struct {
  int64_t steps;             /* decode steps until every request finished */
  int64_t tokens_generated;  /* sum over requests of L_i - P_i */
  double utilization;        /* slots holding tokens / slots reserved, over all steps */
  double mean_batch;         /* running sequences per step */
  int32_t max_batch;
  int64_t preemptions;       /* paged only: sequences sent back to the queue */
  int64_t recomputed_tokens; /* paged only: tokens cached again after a preemption */
  int32_t max_tail_waste;    /* paged: most empty slots in one sequence's last block, any step */
} pkv_sim_result;

/*
 * Run both allocators; PKV_BM_INVALID for an inconsistent configuration
 * (a request that cannot fit the budget alone, sizes out of range).
 */
int pkv_sim_decode(const pkv_sim_config* cfg, pkv_sim_result* paged, pkv_sim_result* slab);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H */
