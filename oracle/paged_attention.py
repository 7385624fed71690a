"""Oracle for paged decode attention (float64, plain numpy).

TEST INFRASTRUCTURE: see the package docstring.

What is computed.  During decoding every sequence keeps the key and value
vector of each token it has seen, per layer and per attention head
([TEQ] "Why the KV cache is an allocator problem").  The cache of a
sequence is cut into 16-token blocks; each sequence keeps a table whose
n-th entry names the pool block that holds its n-th run of 16 tokens, and
those blocks may lie anywhere in one shared pool ([TEQ] "The OS already
solved this in the 1960s"; [IV] "Architecture, step by step", steps 1-3;
[AITJ] "How logical blocks, physical blocks and the block table work").
Attention reads each token's key and value through that table ([IV] step
3).  Paging changes only where the bytes live, not the arithmetic
([AITJ] "What PagedAttention actually solves"), so the result is exactly
textbook scaled dot-product attention [VAS eq. 1] of the single new query
of each sequence over that sequence's cached tokens, in logical order.

Readings where the pages are silent (each is listed in the design notes):
* pool layout: key and value pools are [num_blocks, num_kv_heads,
  block_size, head_size]; token t of a sequence lives at physical block
  block_table[t // block_size], slot t % block_size;
* grouped-query heads: query head h reads kv head h // (Hq / Hkv);
* context_len counts every cached token including the one written this
  step; a context_len of 0 gives an all-zero output;
* softmax is the natural-base, max-subtracted one; the scale is the
  float32 value handed to the GPU, widened exactly;
* slots at or beyond context_len and blocks the table does not reach are
  never read (they may hold NaN garbage).

Parity: pinned.  Brute force on contiguous copies (pure-Python loops and
torch's float64 CPU attention), invariance under any permutation of
physical block placement, the grouped-query reduction to repeated
multi-head attention, the sharing invariance, the partition-merge
identity, and the special cases L = 1, q = 0 and a dominant logit.
"""

import numpy as np

from .formats import to_f64


def _check_table(block_table_row, context_len, num_blocks, block_size):
    nb = -(-context_len // block_size)
    if context_len < 0:
        raise ValueError("negative context length")
    if nb > len(block_table_row):
        raise ValueError("context length exceeds the block table")
    ids = np.asarray(block_table_row[:nb], dtype=np.int64)
    if nb and (ids.min() < 0 or ids.max() >= num_blocks):
        raise ValueError("block table entry outside the pool")


def gather_sequence_kv(cache, block_table_row, context_len, kv_head, dtype,
                       block_size=16):
    """Tokens 0..L-1 of one sequence and one kv head, logical order, [L, D] f64.

    Token t is read from physical block block_table_row[t // block_size]
    at slot t % block_size: the logical-to-physical translation of the
    block table ([AITJ] "How logical blocks, physical blocks and the block
    table work").
    """
    _check_table(block_table_row, context_len, cache.shape[0], block_size)
    t = np.arange(context_len)
    physical = np.asarray(block_table_row, dtype=np.int64)[t // block_size]
    slot = t % block_size
    return to_f64(cache[physical, kv_head, slot, :], dtype)


def attention_one_head(q, keys, values, scale):
    """softmax(scale * keys @ q) @ values for one query vector [VAS eq. 1].

    q: [D] f64; keys, values: [L, D] f64; scale: python float.
    Returns [D] f64; all zeros when L == 0 (no cached token).
    """
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    logits = scale * (keys @ q)
    w = np.exp(logits - logits.max())
    return (w @ values) / w.sum()


def decode_attention(query, key_cache, value_cache, block_tables, context_lens,
                     scale, num_kv_heads, dtype, block_size=16, seqs=None,
                     kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """Decode-step attention of every (sequence, query head), float64.

    query        [S, Hq, D]            storage format of `dtype`
    key_cache    [NB, Hkv, bs, D]      storage format of `kv_dtype`
    value_cache  [NB, Hkv, bs, D]      (default: `dtype`)
    block_tables [S, W] integer        physical block of each logical block
    context_lens [S] integer
    scale        float32 value (widened exactly)
    seqs         optional list of sequence indices to compute (others stay 0)
    k_scale, v_scale  float32 per-pool scales: a cached key element's value
                 is its decoded storage value times k_scale (values: v_scale);
                 1 for pools that hold the values themselves

    Returns [S, Hq, D] float64.
    """
    S, Hq, D = query.shape
    if Hq % num_kv_heads:
        raise ValueError("query heads must be a multiple of kv heads")
    group = Hq // num_kv_heads
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    scale64 = float(np.float32(scale))
    k_scale64 = float(np.float32(k_scale))
    v_scale64 = float(np.float32(v_scale))
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        q_s = to_f64(query[s], dtype)
        for g in range(num_kv_heads):
            keys = gather_sequence_kv(key_cache, block_tables[s], L, g, kv_dtype,
                                      block_size) * k_scale64
            values = gather_sequence_kv(value_cache, block_tables[s], L, g,
                                        kv_dtype, block_size) * v_scale64
            for h in range(g * group, (g + 1) * group):
                out[s, h] = attention_one_head(q_s[h], keys, values, scale64)
    return out


def decode_attention_partitioned(query, key_cache, value_cache, block_tables,
                                 context_lens, scale, num_kv_heads, dtype,
                                 partition_size, block_size=16, seqs=None,
                                 return_partials=False):
    """The split-context form: per-partition softmax state, then a merge.

    The logical tokens [0, L) of a sequence are cut into consecutive
    partitions of `partition_size` tokens.  For partition p with logits
    l_t (t in p):
        m_p = max_t l_t,  s_p = sum_t exp(l_t - m_p),
        o_p = sum_t exp(l_t - m_p) v_t / s_p.
    The merge takes M = max_p m_p and
        out = sum_p s_p exp(m_p - M) o_p / sum_p s_p exp(m_p - M),
    which equals the one-pass softmax exactly in real arithmetic (the
    exp(m_p - M) factors restore a common reference maximum).

    With return_partials the per-partition (m_p, s_p, o_p) are returned as
    a dict {(s, h): [(m, s, o), ...]} beside the merged output.
    """
    if partition_size <= 0:
        raise ValueError("partition size must be positive")
    S, Hq, D = query.shape
    group = Hq // num_kv_heads
    scale64 = float(np.float32(scale))
    out = np.zeros((S, Hq, D), dtype=np.float64)
    partials = {}
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        q_s = to_f64(query[s], dtype)
        for g in range(num_kv_heads):
            keys = gather_sequence_kv(key_cache, block_tables[s], L, g, dtype,
                                      block_size)
            values = gather_sequence_kv(value_cache, block_tables[s], L, g,
                                        dtype, block_size)
            for h in range(g * group, (g + 1) * group):
                parts = []
                for start in range(0, L, partition_size):
                    k_p = keys[start:start + partition_size]
                    v_p = values[start:start + partition_size]
                    logits = scale64 * (k_p @ q_s[h])
                    m_p = logits.max()
                    w = np.exp(logits - m_p)
                    s_p = w.sum()
                    parts.append((m_p, s_p, (w @ v_p) / s_p))
                partials[(s, h)] = parts
                if not parts:
                    continue  # L == 0: output stays zero
                M = max(m for m, _, _ in parts)
                num = sum(s_p * np.exp(m_p - M) * o_p for m_p, s_p, o_p in parts)
                den = sum(s_p * np.exp(m_p - M) for m_p, s_p, _ in parts)
                out[s, h] = num / den
    if return_partials:
        return out, partials
    return out
