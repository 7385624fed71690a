"""Oracle for the two pool-maintenance operations (bit-exact data movement).

TEST INFRASTRUCTURE: see the package docstring.

reshape_and_cache.  Prefill writes the prompt's keys and values into the
blocks assigned to the request, and each decode step appends the new
token's state into the current block, a fresh block being allocated when
the current one fills ([AITJ] "A request lifecycle: allocation, growth,
sharing and release"; [TEQ] "The OS already solved this in the 1960s").
The runtime hands the write as one slot number per new token, slot =
physical_block * block_size + offset (a reading: the pages give the block
mapping, not the encoding).  Token i's key [Hkv, D] goes to
key_cache[slot // bs, :, slot % bs, :], likewise its value.  A negative
slot means "no write" (padding).

copy_blocks.  Sequences that share a block keep a reference count on it;
a sequence that writes into a shared block first gets its own copy:
block-level copy-on-write as in fork() ([TEQ] "Paging's second gift:
copy-on-write"; [IV] "Production takeaways").  For each (src, dst) pair
the whole block -- every kv head, every slot -- is copied in both pools.
Pairs are applied as if simultaneously, so a destination may not repeat
and may not also be a source.

Both operate on integer views so every bit (NaN payloads included) is
preserved, and return new arrays instead of writing in place.

Parity: pinned (tests check hand-built cases against an element-by-element
loop, that untouched slots keep their bits, that writing then gathering
through the table returns the written token, and the rejection rules).
"""

import numpy as np

from .formats import bits_view


def reshape_and_cache(key, value, slot_mapping, key_cache, value_cache,
                      block_size=16):
    """Return (new_key_cache, new_value_cache) with token rows scattered in.

    key, value    [T, Hkv, D]  any element format (bits are copied)
    slot_mapping  [T] integer, -1 (or any negative) = skip
    key_cache     [NB, Hkv, bs, D]
    """
    kc = bits_view(key_cache).copy()
    vc = bits_view(value_cache).copy()
    kb = bits_view(key)
    vb = bits_view(value)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = slots[slots >= 0]
    if len(np.unique(live)) != len(live):
        raise ValueError("duplicate destination slot")
    if len(live) and live.max() >= kc.shape[0] * block_size:
        raise ValueError("slot outside the pool")
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), block_size)
        kc[block, :, offset, :] = kb[i]
        vc[block, :, offset, :] = vb[i]
    return (kc.view(np.asarray(key_cache).dtype),
            vc.view(np.asarray(value_cache).dtype))


def copy_blocks(key_cache, value_cache, src_dst_pairs):
    """Return (new_key_cache, new_value_cache) after block copy-on-write."""
    kc = bits_view(key_cache).copy()
    vc = bits_view(value_cache).copy()
    pairs = np.asarray(src_dst_pairs, dtype=np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0], pairs[:, 1]
    if len(np.unique(dst)) != len(dst):
        raise ValueError("a destination block appears twice")
    if np.intersect1d(src, dst).size:
        raise ValueError("a destination block is also a source")
    nb = kc.shape[0]
    if len(pairs) and (pairs.min() < 0 or pairs.max() >= nb):
        raise ValueError("block id outside the pool")
    k_src = bits_view(key_cache)
    v_src = bits_view(value_cache)
    for s, d in pairs:
        kc[d] = k_src[s]
        vc[d] = v_src[s]
    return (kc.view(np.asarray(key_cache).dtype),
            vc.view(np.asarray(value_cache).dtype))


def reshape_and_cache_fp8(key, value, slot_mapping, key_cache, value_cache, k_scale,
                          v_scale, dtype, block_size=16):
    """reshape_and_cache into e4m3 pools (uint8 codes): each new key
    element is stored as the code of key / k_scale (values: / v_scale),
    quantized as in oracle.fp8.quantize, then scattered like the bits of
    any other format."""
    from .fp8 import quantize
    kq = quantize(key, dtype, k_scale)
    vq = quantize(value, dtype, v_scale)
    return reshape_and_cache(kq, vq, slot_mapping, key_cache, value_cache, block_size)

