"""Invariants of the seeded input generators (CPU only)."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_311_amd import workloads as wl

BS = wl.BLOCK_SIZE


@pytest.mark.parametrize("key", list(wl.WORKLOADS))
def test_metadata_invariants(key):
    w = wl.WORKLOADS[key]
    md = wl.draw_metadata(w, w.default_seed)
    lens = md["context_lens"].astype(np.int64)
    bt = md["block_tables"]
    nb = md["num_blocks"]
    assert bt.shape == (w.num_seqs, w.table_width)
    assert lens.min() >= 1 and lens.max() <= w.max_len
    used = []
    for s, L in enumerate(lens):
        n = -(-int(L) // BS)
        row = bt[s]
        assert (row[:n] >= 0).all() and (row[:n] < nb).all()
        assert (row[n:] == -1).all()
        used.extend(row[:n].tolist())
    counts = np.bincount(np.asarray(used), minlength=nb)
    if w.step in ("cow", "beam"):
        # blocks are shared only among one prompt's samples / beams
        assert counts.max() <= w.samples
        assert (counts > 1).sum() == md["shared_blocks"]
    else:
        assert counts.max() == 1          # every block has one owner
    # at most 15 empty slots per sequence; under 4% of the pool on every
    # workload of realistic lengths (the 4-sequence tiny case is too short)
    assert max(oracle.empty_slots(int(L)) for L in lens) <= BS - 1
    if key not in ("tiny", "prefill_tiny"):
        assert oracle.waste_fraction(lens) < 0.04
    if w.pool[0] == "factor":
        need = len(set(used))
        assert nb == int(np.ceil(w.pool[1] * need)) or w.step in ("cow", "beam")


def test_tiny_pool_and_lengths():
    w = wl.WORKLOADS["tiny"]
    md = wl.draw_metadata(w, w.default_seed)
    assert md["num_blocks"] == 64 and md["block_tables"].shape == (4, 7)
    L = wl.draw_context_lens(w, np.random.default_rng(0), n=20000)
    assert L.min() == 1 and L.max() == 100


def test_lognormal_lengths():
    w = wl.WORKLOADS["llama13b_conv"]
    L = wl.draw_context_lens(w, np.random.default_rng(1), n=200000)
    assert abs(np.median(L) - 600) < 10
    assert L.max() == 4096 and L.min() >= 1
    assert 0.004 < (L == 4096).mean() < 0.012


def test_append_slots():
    w = wl.WORKLOADS["llama13b_conv"]
    md = wl.draw_metadata(w, w.default_seed)
    lens, bt, slots = md["context_lens"], md["block_tables"], md["slot_mapping"]
    assert len(np.unique(slots)) == len(slots)
    for s in range(len(lens)):
        pos = int(lens[s]) - 1
        assert slots[s] == bt[s, pos // BS] * BS + pos % BS
        blk, off = divmod(int(slots[s]), BS)
        # the new token's slot is empty before the step, earlier ones full
        assert not md["live_slots"][blk, off]
        assert md["live_slots"][blk, :off].all()


def test_cow_pairs_follow_reference_counts():
    w = wl.WORKLOADS["sampling_cow"]
    md = wl.draw_metadata(w, w.default_seed)
    P = md["prompt_lens"]
    pairs = md["cow_pairs"]
    # samples 0..6 copy a shared partial last block, the 8th writes in place
    assert len(pairs) == (w.samples - 1) * int((P % BS != 0).sum())
    assert len(np.unique(pairs[:, 1])) == len(pairs)
    assert not np.intersect1d(pairs[:, 0], pairs[:, 1]).size
    # every private token's slot is distinct and not in a shared block
    slots = md["slot_mapping"]
    assert len(np.unique(slots)) == len(slots)
    lens = md["context_lens"]
    bt = md["block_tables"]
    seq = md["token_seq"]
    assert len(slots) == int(sum(lens[s] - P[s // w.samples]
                                 for s in range(w.num_seqs)))
    counts = np.bincount(bt[bt >= 0].ravel(), minlength=md["num_blocks"])
    assert (counts[slots // BS] == 1).all()
    for s in (0, 7, 100, 255):
        first = int(np.flatnonzero(seq == s)[0])
        pos = int(P[s // w.samples])
        assert slots[first] == bt[s, pos // BS] * BS + pos % BS


def test_tiny_batch_values_poisoned():
    w = wl.WORKLOADS["tiny"]
    b = wl.make_batch(w, device="cpu")
    live = torch.from_numpy(b["live_slots"])
    kc = b["key_cache"]
    assert torch.isfinite(kc[live[:, None, :].expand(-1, w.num_kv_heads, -1)]).all()
    assert torch.isnan(kc[(~live)[:, None, :].expand(-1, w.num_kv_heads, -1)]).all()
    assert b["query"].shape == (4, 4, 64) and b["query"].dtype == torch.float32
    # the same seed gives the same batch
    b2 = wl.make_batch(w, device="cpu")
    assert torch.equal(b["query"], b2["query"])
    assert np.array_equal(wl.to_host(kc).view(np.uint32),
                          wl.to_host(b2["key_cache"]).view(np.uint32))


def test_bf16_to_host_bits():
    t = torch.tensor([1.0, -2.0, float("inf")], dtype=torch.bfloat16)
    h = wl.to_host(t)
    assert h.dtype == np.uint16
    assert h.tolist() == [0x3F80, 0xC000, 0x7F80]


@pytest.mark.parametrize("base", ["opt13b", "long_gqa"])
def test_fp8_variant_shares_metadata(base):
    """An E4M3 workload draws the same lengths and placement as its base."""
    w, w8 = wl.WORKLOADS[base], wl.WORKLOADS[base + "_fp8"]
    assert w8.fp8 and not w.fp8 and w8.kv_elem_bytes == 1 and w.kv_elem_bytes == 2
    a, b = wl.draw_metadata(w, w.default_seed), wl.draw_metadata(w8, w8.default_seed)
    assert (a["context_lens"] == b["context_lens"]).all()
    assert (a["block_tables"] == b["block_tables"]).all()


def test_fp8_pool_codes():
    """E4M3 pools hold codes: the NaN code in free slots, finite codes with
    the pool's scale in live ones."""
    w = wl.custom([5, 33, 16], 4, 2, 64, "f16", kv_dtype="e4m3", k_scale=1 / 64,
                  v_scale=3 / 128)
    b = wl.make_batch(w, 3)
    live = b["live_slots"]
    for cache, scale in ((b["key_cache"], w.k_scale), (b["value_cache"], w.v_scale)):
        assert cache.dtype == torch.uint8
        codes = cache.numpy()
        dead = ~live[:, None, :, None].repeat(w.num_kv_heads, 1).repeat(w.head_size, 3)
        assert (codes[dead] == wl.E4M3_NAN).all()
        vals = oracle.e4m3_decode(codes[~dead])
        assert np.isfinite(vals).all()
        # N(0,1) in the pool's units: the spread comes back after scaling
        assert 0.8 < np.std(vals * scale) < 1.2
    assert b["query"].dtype == torch.float16


@pytest.mark.parametrize("key", ["prefill_chunk", "prefill_gqa", "prefill_tiny"])
def test_prefill_metadata(key):
    """A prefill step's chunk: n new rows per sequence at positions L - n ..
    L - 1, whose slots are in the sequence's blocks and empty before the
    step; the prefix slots are live."""
    w = wl.WORKLOADS[key]
    md = wl.draw_metadata(w, w.default_seed)
    qsl = md["query_start_loc"]
    n = np.diff(qsl)
    lens = md["context_lens"].astype(np.int64)
    assert qsl[0] == 0 and (n >= 1).all() and (n <= lens).all() and n.max() <= w.max_query_len
    assert len(md["slot_mapping"]) == qsl[-1]
    live = md["live_slots"]
    bt = md["block_tables"]
    for s in range(w.num_seqs):
        L, k = int(lens[s]), int(n[s])
        slots = md["slot_mapping"][qsl[s]:qsl[s + 1]]
        want = [bt[s, t // BS] * BS + t % BS for t in range(L - k, L)]
        assert slots.tolist() == want
        assert not live.reshape(-1)[slots].any()
        prefix = [bt[s, t // BS] * BS + t % BS for t in range(L - k)]
        assert live.reshape(-1)[prefix].all()
    b = wl.make_batch(wl.WORKLOADS["prefill_tiny"], 5)
    assert b["query"].shape[0] == b["query_start_loc"][-1] == b["key"].shape[0]


def test_beam_step_copies_shared_partial_blocks():
    """The beam workload's step: every beam appends one token; a pair is
    drawn exactly where a beam's last block was shared and partly filled,
    its destination is that beam's own block now, and the new token lands
    in it.  Beams of one request share their prompt's full blocks."""
    w = wl.WORKLOADS["beam"]
    md = wl.draw_metadata(w, w.default_seed)
    bt, lens, slots = md["block_tables"], md["context_lens"], md["slot_mapping"]
    assert len(slots) == w.num_seqs == w.prompts * w.samples
    assert md["forks"] > 0 and len(md["cow_pairs"]) > 0
    refs = np.bincount(bt[bt >= 0], minlength=md["num_blocks"])
    dsts = {int(d): int(sv) for sv, d in md["cow_pairs"]}
    for s_ in range(w.num_seqs):
        L = int(lens[s_])
        last = int(bt[s_, (L - 1) // BS])
        assert slots[s_] == last * BS + (L - 1) % BS
        if last in dsts:
            assert refs[last] == 1 and (L - 1) % BS != 0
            assert md["live_slots"][dsts[last], :(L - 1) % BS].all()
    # the first prompt block of a request is shared by all its beams
    first = bt[:, 0].reshape(w.prompts, w.samples)
    assert (first == first[:, :1]).all()


@pytest.mark.parametrize("base", ["sampling_cow", "beam"])
def test_shuffled_batches_are_the_same_batch_reordered(base):
    """The shuffled sibling workloads hold the ordered batch's sequences in
    another order: the same rows, every new token still in a block of its
    own sequence's table at that sequence's next position, and the same
    blocks flagged as shared (reference count above one)."""
    w0 = wl.WORKLOADS[base]
    w1 = wl.WORKLOADS[base + "_shuffled"]
    a = wl.draw_metadata(w0, w0.default_seed)
    b = wl.draw_metadata(w1, w1.default_seed)
    perm = b["sequence_order"]
    assert not np.array_equal(perm, np.arange(len(perm)))
    assert np.array_equal(b["context_lens"], a["context_lens"][perm])
    assert np.array_equal(b["block_tables"], a["block_tables"][perm])
    assert np.array_equal(np.sort(b["slot_mapping"]), np.sort(a["slot_mapping"]))
    assert (np.diff(b["token_seq"]) >= 0).all()
    for slot, s in zip(b["slot_mapping"], b["token_seq"]):
        assert slot // 16 in set(b["block_tables"][s].tolist())
    assert np.array_equal(b["block_shared"], a["block_shared"])
    assert np.array_equal(b["cow_pairs"], a["cow_pairs"])
    # flags = blocks that more than one sequence's table maps
    counts = np.zeros(a["num_blocks"], np.int64)
    for s, L in enumerate(a["context_lens"]):
        for x in a["block_tables"][s, :-(-int(L) // 16)]:
            counts[x] += 1
    assert np.array_equal(a["block_shared"], (counts > 1).astype(np.uint8))
