"""Oracle for paged prefill attention (float64, plain numpy).

TEST INFRASTRUCTURE: see the package docstring.

What is computed.  When a request's prompt (or the next chunk of it) is
processed, the keys and values of all of its new tokens are written into
the blocks the runtime assigned ([AITJ] "A request lifecycle: allocation,
growth, sharing and release"), and every new token then attends to every
cached token at or before its own position: the masked self-attention of
a decoder, which excludes later positions [VAS section 3.2.3].  The keys
and values are read through the block table exactly as in decoding
([IV] "Architecture, step by step", step 3), so each output row is
textbook scaled dot-product attention [VAS eq. 1] over a prefix of the
sequence's cached tokens in logical order.

Readings where the pages are silent (each is listed in the design notes):
* the queries of all sequences are packed [T, Hq, D]; sequence s owns rows
  query_start_loc[s] .. query_start_loc[s+1]-1 (n_s rows);
* those rows are the last n_s tokens of the sequence: context_lens[s]
  (= L_s) counts the cached prefix and the new tokens, whose keys and
  values are already in the pool; row i sits at position L_s - n_s + i and
  attends to tokens 0 .. L_s - n_s + i (a chunk after a cached prefix, or
  the whole prompt when n_s = L_s);
* grouped-query heads, pool layout, scale and softmax as in decoding.

Parity: pinned.  Whole prompts (n = L) equal torch's float64 causal
attention on contiguous copies; chunks after a prefix equal pure-Python
loops with an explicit mask and, row by row, the decode oracle at that
row's length; outputs are bitwise invariant under permutation of the
physical block placement.
"""

import numpy as np

from .formats import to_f64
from .paged_attention import attention_one_head, gather_sequence_kv


def prefill_attention(query, key_cache, value_cache, block_tables, context_lens,
                      query_start_loc, scale, num_kv_heads, dtype, block_size=16, seqs=None):
    """Causal attention of every new token of every sequence, float64.

    query            [T, Hq, D]        storage format of `dtype`
    key_cache        [NB, Hkv, bs, D]
    value_cache      [NB, Hkv, bs, D]
    block_tables     [S, W] integer
    context_lens     [S] integer       L_s, cached prefix plus new tokens
    query_start_loc  [S + 1] integer   rows of each sequence in `query`
    scale            float32 value (widened exactly)
    seqs             optional list of sequences to compute (other rows stay 0)

    Returns [T, Hq, D] float64.
    """
    T, Hq, D = query.shape
    if Hq % num_kv_heads:
        raise ValueError("query heads must be a multiple of kv heads")
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    S = len(qsl) - 1
    if qsl[0] != 0 or qsl[-1] != T or (np.diff(qsl) < 0).any():
        raise ValueError("query_start_loc must rise from 0 to the number of rows")
    group = Hq // num_kv_heads
    scale64 = float(np.float32(scale))
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        n = int(qsl[s + 1] - qsl[s])
        if n > L:
            raise ValueError("more new tokens than the context holds")
        q_s = to_f64(query[qsl[s]:qsl[s + 1]], dtype)
        for g in range(num_kv_heads):
            keys = gather_sequence_kv(key_cache, block_tables[s], L, g, dtype, block_size)
            values = gather_sequence_kv(value_cache, block_tables[s], L, g, dtype, block_size)
            for i in range(n):
                visible = L - n + i + 1          # tokens 0 .. position of row i
                for h in range(g * group, (g + 1) * group):
                    out[qsl[s] + i, h] = attention_one_head(q_s[i, h], keys[:visible],
                                                            values[:visible], scale64)
    return out
