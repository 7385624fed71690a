"""Seeded synthetic inputs for the paged decode path (no method arithmetic).

This module only draws inputs: sequence lengths, the physical placement of
blocks, reference-counted sharing with copy-on-write pairs, slot numbers
for new tokens, and N(0,1) query/key/value values.  It computes no
attention and no cache update; it is the one module that both the GPU
path's tests and the CPU oracle's tests draw their inputs from.

Workloads (the shapes the pages' discussion is about: OPT-13B's 40 heads of
128 and its 2,048-token reservation, conversational lengths, parallel
sampling over a shared prompt, long contexts):

  tiny           4 seqs, 4 heads of 64, fp32, lengths U{1..100}, a 64-block
                 pool, random placement.
  opt13b         one OPT-13B-shaped layer: 40 heads of 128, fp16, 64 seqs,
                 lengths U{1..2048}, pool 1.25x the need, random placement.
  llama13b_conv  40 heads of 128, fp16, 256 seqs, lognormal lengths
                 (median 600, sigma 0.8, capped at 4096); one new token per
                 sequence is appended (slot mapping) before decoding.
  sampling_cow   32 prompts x 8 samples, 40 heads of 128, fp16, prompt
                 lengths U{64..1024} shared through reference-counted
                 blocks, 1..64 private tokens per sample; a shared, partly
                 filled last block is copied before a sample writes to it.
  long_gqa       32 query heads over 8 kv heads of 128, bf16, 16 seqs of
                 32,768 tokens, pool 1.25x the need; contexts are split
                 into pieces merged through float32 (max, sum) states.
  long_gqa_p512  long_gqa with the contexts split into partitions of 512
                 tokens (64 pieces per sequence and kv head).
  opt13b_fp8,    the same shapes and lengths with pools of OCP E4M3 codes
  long_gqa_fp8   and one scale per pool (keys 1/64, values 3/128); queries,
                 outputs and new tokens stay fp16 / bf16.
  sampling_cow_shuffled, beam_shuffled
                 the same batches with the sequences in a random order, so
                 the siblings of a request are no longer neighbours.
  beam           beam search: 16 requests x 4 beams, 40 heads of 128, fp16,
                 prompts U{256..1024} shared by their beams; 24 steps of
                 appends (copy-on-write of shared partial blocks) with beams
                 dying and survivors forking in their place, then one more
                 append of every beam (its copy_blocks pairs and slots) and
                 the decode.
  prefill_chunk  chunked prefill: 16 seqs, 40 heads of 128, fp16, a cached
                 prefix of U{0..1536} tokens and a new chunk of 512 tokens
                 each (written by reshape_and_cache, then attended).
  prefill_gqa    whole prompts: 8 seqs of 2048 new tokens, 32 query heads
                 over 8 kv heads of 128, bf16.
  prefill_tiny   4 seqs, 4 query / 2 kv heads of 64, fp16, prefixes
                 U{0..40}, chunks U{1..24}, a 64-block pool.

An E4M3 pool is drawn as codes: N(0,1) values divided by the pool's scale,
clamped to the format's range and converted by torch's float8_e4m3fn cast
(a library conversion used only to draw codes with that spread; both the
oracle and the GPU path read the codes as given).  Its free slots hold the
NaN code 0x7F.

Every slot that holds no token -- unused blocks and the tail of each
sequence's last block -- is filled with NaN, so any stray read shows up in
the output.  Lengths and placement come from numpy's PCG64 seeded with the
workload's seed; values come from torch's generator seeded the same way on
the device that will hold them.
"""

from collections import deque
from dataclasses import dataclass

import numpy as np

BLOCK_SIZE = 16
FP8_K_SCALE = 1.0 / 64     # N(0,1) / scale stays below the E4M3 maximum 448
FP8_V_SCALE = 3.0 / 128
E4M3_NAN = 0x7F


@dataclass(frozen=True)
class Workload:
    key: str
    index: int              # seeds the workload; an fp8 variant shares its base's,
                            # so lengths, placement and values match
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    dtype: str              # "f32" | "f16" | "bf16"
    lengths: tuple          # see draw_context_lens
    pool: tuple             # ("blocks", n) | ("factor", f)
    step: str               # "decode" | "append" | "cow" | "beam" | "prefill"
    max_len: int            # longest possible context (sets the table width)
    partition_size: int = 0   # cap on tokens per piece of a split context (0: none)
    prompts: int = 0
    samples: int = 0
    kv_dtype: str = ""      # "" (pools in `dtype`) | "e4m3" (pools of E4M3 codes)
    k_scale: float = 1.0    # per-pool scales of an E4M3 pool
    v_scale: float = 1.0
    shuffle: bool = False   # (cow / beam) sequences in a random order instead of
                            # each request's siblings side by side

    @property
    def max_query_len(self):
        """Most new tokens of one sequence in a prefill step."""
        return int(self.lengths[4]) if self.step == "prefill" else 1

    @property
    def fp8(self):
        return self.kv_dtype == "e4m3"

    @property
    def kv_elem_bytes(self):
        return 1 if self.fp8 else (4 if self.dtype == "f32" else 2)

    @property
    def table_width(self):
        return -(-self.max_len // BLOCK_SIZE)

    @property
    def scale(self):
        return np.float32(1.0 / np.sqrt(self.head_size))

    @property
    def default_seed(self):
        return 311000 + self.index

    def seeds(self):
        """The workload's seed plus two more used by the parity tests."""
        s = self.default_seed
        return (s, s + 100, s + 200)


WORKLOADS = {
    w.key: w for w in (
        Workload("tiny", 1, 4, 4, 4, 64, "f32", ("uniform", 1, 100),
                 ("blocks", 64), "decode", 100),
        Workload("opt13b", 2, 64, 40, 40, 128, "f16", ("uniform", 1, 2048),
                 ("factor", 1.25), "decode", 2048),
        Workload("llama13b_conv", 3, 256, 40, 40, 128, "f16",
                 ("lognormal", 600.0, 0.8, 4096), ("factor", 1.25), "append",
                 4096),
        Workload("sampling_cow", 4, 256, 40, 40, 128, "f16",
                 ("cow", 64, 1024, 1, 64), ("factor", 1.25), "cow", 1088,
                 prompts=32, samples=8),
        Workload("long_gqa", 5, 16, 32, 8, 128, "bf16", ("fixed", 32768),
                 ("factor", 1.25), "decode", 32768),
        # the same, split into the configured context partitions of 512
        # tokens (32 blocks): 64 pieces per (sequence, kv head)
        Workload("long_gqa_p512", 5, 16, 32, 8, 128, "bf16", ("fixed", 32768),
                 ("factor", 1.25), "decode", 32768, partition_size=512),
        Workload("opt13b_fp8", 2, 64, 40, 40, 128, "f16", ("uniform", 1, 2048),
                 ("factor", 1.25), "decode", 2048, kv_dtype="e4m3",
                 k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE),
        Workload("long_gqa_fp8", 5, 16, 32, 8, 128, "bf16", ("fixed", 32768),
                 ("factor", 1.25), "decode", 32768, kv_dtype="e4m3",
                 k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE),
        # wider grouped-query shapes than long_gqa's 4 query heads per kv
        # head, at its lengths: 8 per kv head, and 16 per kv head
        Workload("gqa8_long", 12, 16, 64, 8, 128, "bf16", ("fixed", 32768),
                 ("factor", 1.25), "decode", 32768),
        Workload("gqa16_long", 13, 16, 32, 2, 128, "bf16", ("fixed", 32768),
                 ("factor", 1.25), "decode", 32768),
        Workload("beam", 11, 64, 40, 40, 128, "f16", ("beam", 256, 1024, 24),
                 ("factor", 1.25), "beam", 1056, prompts=16, samples=4),
        # the same two batches with their sequences in a random order (the
        # siblings of a request no longer side by side)
        Workload("sampling_cow_shuffled", 4, 256, 40, 40, 128, "f16",
                 ("cow", 64, 1024, 1, 64), ("factor", 1.25), "cow", 1088,
                 prompts=32, samples=8, shuffle=True),
        Workload("beam_shuffled", 11, 64, 40, 40, 128, "f16", ("beam", 256, 1024, 24),
                 ("factor", 1.25), "beam", 1056, prompts=16, samples=4, shuffle=True),
        Workload("prefill_chunk", 8, 16, 40, 40, 128, "f16", ("prefill", 0, 1536, 512, 512),
                 ("factor", 1.25), "prefill", 2048),
        Workload("prefill_gqa", 9, 8, 32, 8, 128, "bf16", ("prefill", 0, 0, 2048, 2048),
                 ("factor", 1.25), "prefill", 2048),
        Workload("prefill_tiny", 10, 4, 4, 2, 64, "f16", ("prefill", 0, 40, 1, 24),
                 ("blocks", 64), "prefill", 64),
    )
}


def draw_context_lens(w, rng, n=None):
    """Context lengths of a workload (integer ranges are inclusive)."""
    n = w.num_seqs if n is None else n
    kind = w.lengths[0]
    if kind == "uniform":
        lo, hi = w.lengths[1:]
        return rng.integers(lo, hi + 1, size=n).astype(np.int64)
    if kind == "lognormal":
        median, sigma, cap = w.lengths[1:]
        x = np.exp(rng.normal(np.log(median), sigma, size=n))
        return np.clip(np.rint(x), 1, cap).astype(np.int64)
    if kind == "fixed":
        return np.full(n, w.lengths[1], dtype=np.int64)
    if kind == "list":  # explicit lengths, for edge-case tests
        return np.asarray(w.lengths[1], dtype=np.int64)
    raise ValueError(f"no plain length draw for {kind!r}")


class BlockManager:
    """Host-side owner of the physical block pool (caller's side of the API).

    Hands out free blocks in a random order (so placement is scattered),
    keeps a reference count per block, shares blocks on fork and asks for a
    copy when a sequence is about to write into a block someone else still
    references.  Releasing a table returns unreferenced blocks to the pool.
    """

    def __init__(self, num_blocks, rng, block_size=BLOCK_SIZE):
        self.num_blocks = int(num_blocks)
        self.block_size = block_size
        self.free = deque(int(b) for b in rng.permutation(self.num_blocks))
        self.ref = np.zeros(self.num_blocks, dtype=np.int64)

    def allocate(self):
        if not self.free:
            raise MemoryError("block pool exhausted")
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def allocate_for(self, n_tokens):
        return [self.allocate() for _ in range(-(-n_tokens // self.block_size))]

    def fork(self, table):
        for b in table:
            self.ref[b] += 1
        return list(table)

    def release(self, table):
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
            elif self.ref[b] < 0:
                raise RuntimeError("block released twice")

    def append_slot(self, table, position):
        """Slot for the token at logical `position`, growing/copying as needed.

        Returns (slot, cow_pair); cow_pair is (src, dst) when the block that
        receives the token was shared and has just been replaced by a copy.
        """
        bs = self.block_size
        n, off = divmod(position, bs)
        pair = None
        if n == len(table):
            table.append(self.allocate())
        elif n > len(table):
            raise ValueError("append beyond the end of the table")
        elif self.ref[table[n]] > 1:
            src = table[n]
            dst = self.allocate()
            self.ref[src] -= 1
            table[n] = dst
            pair = (src, dst)
        return table[n] * bs + off, pair


def _pool_blocks(w, need):
    if w.pool[0] == "blocks":
        if w.pool[1] < need:
            raise ValueError("fixed pool too small for the drawn lengths")
        return int(w.pool[1])
    return max(1, int(np.ceil(w.pool[1] * need)))


def _table_array(tables, width):
    bt = np.full((len(tables), width), -1, dtype=np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    return bt


def _live_slot_mask(num_blocks, tables, filled, block_size=BLOCK_SIZE):
    """[NB, bs] bool: slots that hold a token (filled[s] tokens of table s)."""
    live = np.zeros((num_blocks, block_size), dtype=bool)
    for t, n in zip(tables, filled):
        full, rem = divmod(int(n), block_size)
        live[t[:full], :] = True
        if rem:
            live[t[full], :rem] = True
    return live


def draw_metadata(w, seed):
    """Integer side of a workload: lengths, tables, slots, CoW pairs.

    Returns a dict of numpy arrays:
      context_lens  int32 [S]      tokens each sequence attends to
      block_tables  int32 [S, W]   -1 past each sequence's last block
      num_blocks    int            pool size in blocks
      live_slots    bool [NB, bs]  slots holding a token before the step
      slot_mapping  int64 [T]      (append / cow) slots of the new tokens
      token_seq     int64 [T]      (append / cow) sequence of each new token
      cow_pairs     int64 [N, 2]   (cow) blocks to copy before the writes
      shared_blocks int            (cow) blocks referenced by > 1 sequence
      query_start_loc int32 [S+1]  (prefill) rows of each sequence's chunk
    """
    rng = np.random.default_rng(seed)
    bs = BLOCK_SIZE
    md = {}
    if w.step == "prefill":
        # a cached prefix of P tokens and a chunk of n new ones per sequence:
        # the chunk's slots are assigned (blocks taken for all P + n tokens)
        # but hold no token until the step writes them
        if w.lengths[0] == "prefill":
            plo, phi, nlo, nhi = w.lengths[1:]
            P = rng.integers(plo, phi + 1, size=w.num_seqs)
            n = rng.integers(nlo, nhi + 1, size=w.num_seqs)
        else:  # ("prefill_list", prefixes, chunks), for edge-case tests
            P = np.asarray(w.lengths[1], dtype=np.int64)
            n = np.asarray(w.lengths[2], dtype=np.int64)
        lens = (P + n).astype(np.int64)
        need = int(sum(-(-int(L) // bs) for L in lens))
        nb = _pool_blocks(w, need)
        mgr = BlockManager(nb, rng)
        tables, slots, token_seq = [], [], []
        for s_, L in enumerate(lens):
            t = mgr.allocate_for(int(L))
            tables.append(t)
            for pos in range(int(P[s_]), int(L)):
                slots.append(t[pos // bs] * bs + pos % bs)
                token_seq.append(s_)
        md["context_lens"] = lens.astype(np.int32)
        md["block_tables"] = _table_array(tables, w.table_width)
        md["num_blocks"] = nb
        md["live_slots"] = _live_slot_mask(nb, tables, P)
        md["slot_mapping"] = np.asarray(slots, dtype=np.int64)
        md["token_seq"] = np.asarray(token_seq, dtype=np.int64)
        md["query_start_loc"] = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        return md
    if w.step in ("decode", "append"):
        lens = draw_context_lens(w, rng)
        need = int(sum(-(-int(L) // bs) for L in lens))
        nb = _pool_blocks(w, need)
        mgr = BlockManager(nb, rng)
        tables, filled, slots = [], [], []
        for L in lens:
            L = int(L)
            cached = L if w.step == "decode" else max(L - 1, 0)
            t = mgr.allocate_for(cached)
            if w.step == "append":
                slot, pair = mgr.append_slot(t, cached)
                assert pair is None
                slots.append(slot)
            tables.append(t)
            filled.append(cached)
        md["context_lens"] = lens.astype(np.int32)
        md["block_tables"] = _table_array(tables, w.table_width)
        md["num_blocks"] = nb
        md["live_slots"] = _live_slot_mask(nb, tables, filled)
        if w.step == "append":
            md["slot_mapping"] = np.asarray(slots, dtype=np.int64)
            md["token_seq"] = np.arange(len(lens), dtype=np.int64)
        return md

    if w.step == "cow":
        plo, phi, nlo, nhi = w.lengths[1:]
        P = rng.integers(plo, phi + 1, size=w.prompts)
        n = rng.integers(nlo, nhi + 1, size=(w.prompts, w.samples))
        need = 0
        for i in range(w.prompts):
            p = int(P[i])
            need += -(-p // bs)
            rem_cap = (bs - p % bs) % bs
            for k in range(w.samples):
                if p % bs and k < w.samples - 1:
                    need += 1  # private copy of the shared partial block
                need += -(-max(int(n[i, k]) - rem_cap, 0) // bs)
        nb = _pool_blocks(w, need)
        mgr = BlockManager(nb, rng)
        prompt_tables = [mgr.allocate_for(int(p)) for p in P]
        live = _live_slot_mask(nb, prompt_tables, P)
        tables, lens, slots, token_seq, pairs = [], [], [], [], []
        for i in range(w.prompts):
            p = int(P[i])
            shared = [mgr.fork(prompt_tables[i]) for _ in range(w.samples)]
            mgr.release(prompt_tables[i])  # the prompt itself is done
            for k in range(w.samples):
                t = shared[k]
                for pos in range(p, p + int(n[i, k])):
                    slot, pair = mgr.append_slot(t, pos)
                    if pair is not None:
                        pairs.append(pair)
                    slots.append(slot)
                    token_seq.append(len(tables))
                tables.append(t)
                lens.append(p + int(n[i, k]))
        md["context_lens"] = np.asarray(lens, dtype=np.int32)
        md["block_tables"] = _table_array(tables, w.table_width)
        md["num_blocks"] = nb
        md["live_slots"] = live
        md["slot_mapping"] = np.asarray(slots, dtype=np.int64)
        md["token_seq"] = np.asarray(token_seq, dtype=np.int64)
        md["cow_pairs"] = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
        md["shared_blocks"] = int((mgr.ref > 1).sum())
        md["block_shared"] = (mgr.ref > 1).astype(np.uint8)
        md["prompt_lens"] = P.astype(np.int64)
        return _shuffled(md, seed) if w.shuffle else md

    if w.step == "beam":
        # beam search: each request's beams share its prompt; every step each
        # beam appends a token (copying a shared partial last block first),
        # and between steps some beams die and surviving ones fork to take
        # their place.  The state after `history` such steps is cached; the
        # step drawn here is one more append of every beam.
        plo, phi, history = w.lengths[1:]
        R, B = w.prompts, w.samples
        P = rng.integers(plo, phi + 1, size=R)
        need = int(sum(-(-int(p) // bs) for p in P)) + R * B * (history + 2)
        nb = _pool_blocks(w, need)
        mgr = BlockManager(nb, rng)
        beams = []  # (request, table, length)
        for i in range(R):
            prompt = mgr.allocate_for(int(P[i]))
            beams.extend((i, mgr.fork(prompt), int(P[i])) for _ in range(B))
            mgr.release(prompt)
        forks = kills = 0
        for step in range(history):
            for k, (i, t, L) in enumerate(beams):
                mgr.append_slot(t, L)
                beams[k] = (i, t, L + 1)
            for i in range(R):  # some beams die, survivors fork in their place
                mine = [k for k, b in enumerate(beams) if b[0] == i]
                dead = rng.choice(mine, size=int(rng.integers(0, B // 2 + 1)), replace=False)
                alive = [k for k in mine if k not in set(dead.tolist())]
                for k in dead:
                    mgr.release(beams[k][1])
                    src = beams[int(rng.choice(alive))]
                    beams[k] = (i, mgr.fork(src[1]), src[2])
                    forks += 1
                    kills += 1
        tables = [t for _, t, _ in beams]
        lens = [L for _, _, L in beams]
        live = _live_slot_mask(nb, tables, lens)
        slots, pairs = [], []
        for k, (i, t, L) in enumerate(beams):
            slot, pair = mgr.append_slot(t, L)
            if pair is not None:
                pairs.append(pair)
            slots.append(slot)
        md["context_lens"] = np.asarray([L + 1 for L in lens], dtype=np.int32)
        md["block_tables"] = _table_array(tables, w.table_width)
        md["num_blocks"] = nb
        md["live_slots"] = live
        md["slot_mapping"] = np.asarray(slots, dtype=np.int64)
        md["token_seq"] = np.arange(len(beams), dtype=np.int64)
        md["cow_pairs"] = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
        md["shared_blocks"] = int((mgr.ref > 1).sum())
        md["block_shared"] = (mgr.ref > 1).astype(np.uint8)
        md["prompt_lens"] = P.astype(np.int64)
        md["forks"] = forks
        return _shuffled(md, seed) if w.shuffle else md
    raise ValueError(w.step)


def _shuffled(md, seed):
    """The same batch with its sequences in a seeded random order: rows of
    the tables and lengths permuted, each new token moved with its sequence
    (tokens stay grouped by sequence, in the new order); blocks, slots and
    copy pairs are unchanged."""
    perm = np.random.default_rng(seed + 7777).permutation(len(md["context_lens"]))
    new_of_old = np.empty_like(perm)
    new_of_old[perm] = np.arange(len(perm))
    md = dict(md)
    md["context_lens"] = md["context_lens"][perm]
    md["block_tables"] = md["block_tables"][perm]
    ts = new_of_old[md["token_seq"]]
    order = np.argsort(ts, kind="stable")
    md["token_seq"] = ts[order].astype(np.int64)
    md["slot_mapping"] = md["slot_mapping"][order]
    md["sequence_order"] = perm.astype(np.int64)
    return md


_TORCH_DTYPES = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def torch_dtype(dtype):
    import torch
    return getattr(torch, _TORCH_DTYPES[dtype])


def _randn(shape, gen, device, dtype):
    import torch
    return torch.randn(shape, generator=gen, device=device,
                       dtype=torch.float32).to(torch_dtype(dtype))


def make_batch(w, seed=None, device="cpu", chunk_blocks=2048):
    """A full seeded batch: metadata (numpy) plus value tensors (torch).

    Values: query [S, Hq, D]; key_cache / value_cache [NB, Hkv, bs, D] with
    N(0,1) in live slots and NaN everywhere else; for append/cow steps the
    new tokens' key / value [T, Hkv, D].
    """
    import torch
    seed = w.default_seed if seed is None else int(seed)
    md = draw_metadata(w, seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    td = torch_dtype(w.dtype)
    S, Hq, Hkv, D = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size
    nb = md["num_blocks"]
    live = md["live_slots"]
    used = np.flatnonzero(live.any(axis=1))
    caches = []
    for pool_scale in (w.k_scale, w.v_scale):
        shape = (nb, Hkv, BLOCK_SIZE, D)
        if w.fp8:
            cache = torch.full(shape, E4M3_NAN, dtype=torch.uint8, device=device)
        else:
            cache = torch.full(shape, float("nan"), dtype=td, device=device)
        for c0 in range(0, len(used), chunk_blocks):
            ids = used[c0:c0 + chunk_blocks]
            dead = torch.from_numpy(~live[ids]).to(device)[:, None, :, None]
            if w.fp8:
                vals = torch.randn((len(ids), Hkv, BLOCK_SIZE, D), generator=gen,
                                   device=device, dtype=torch.float32)
                vals = (vals / pool_scale).clamp_(-448.0, 448.0)
                vals = vals.to(torch.float8_e4m3fn).view(torch.uint8)
                vals.masked_fill_(dead, E4M3_NAN)
            else:
                vals = _randn((len(ids), Hkv, BLOCK_SIZE, D), gen, device, w.dtype)
                vals.masked_fill_(dead, float("nan"))
            cache[torch.from_numpy(ids).to(device)] = vals
        caches.append(cache)
    batch = dict(md)
    nq = int(md["query_start_loc"][-1]) if w.step == "prefill" else S
    batch.update(
        workload=w, seed=seed, scale=w.scale,
        query=_randn((nq, Hq, D), gen, device, w.dtype),
        key_cache=caches[0], value_cache=caches[1],
    )
    if "slot_mapping" in md:
        T = len(md["slot_mapping"])
        batch["key"] = _randn((T, Hkv, D), gen, device, w.dtype)
        batch["value"] = _randn((T, Hkv, D), gen, device, w.dtype)
    return batch


def to_host(t):
    """Host numpy array holding a tensor's bits (bf16 as uint16)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def kv_token_count(md):
    """Tokens attended in one decode step (sum of context lengths)."""
    return int(np.asarray(md["context_lens"], dtype=np.int64).sum())


def custom_prefill(prefixes, chunks, num_heads, num_kv_heads, head_size, dtype,
                   pool_factor=1.25):
    """A prefill workload with explicit prefix and chunk lengths."""
    prefixes = tuple(int(x) for x in prefixes)
    chunks = tuple(int(x) for x in chunks)
    max_len = max(max(p + c for p, c in zip(prefixes, chunks)), 1)
    return Workload("custom_prefill", 0, len(chunks), num_heads, num_kv_heads, head_size,
                    dtype, ("prefill_list", prefixes, chunks, 0, max(chunks)),
                    ("factor", pool_factor), "prefill", max_len)


def custom(lens, num_heads, num_kv_heads, head_size, dtype, max_len=None,
           pool_factor=1.25, partition_size=512, kv_dtype="", k_scale=1.0, v_scale=1.0):
    """A decode workload with explicit context lengths (edge-case tests)."""
    lens = tuple(int(x) for x in lens)
    max_len = max(max(lens), 1) if max_len is None else max_len
    return Workload("custom", 0, len(lens), num_heads, num_kv_heads, head_size,
                    dtype, ("list", lens), ("factor", pool_factor), "decode",
                    max_len, partition_size, kv_dtype=kv_dtype, k_scale=k_scale,
                    v_scale=v_scale)
