"""Oracle for KV-cache size accounting (exact integer arithmetic).

TEST INFRASTRUCTURE: see the package docstring.

* Bytes per token.  One token's cache is one key and one value vector per
  layer: 2 x hidden x layers x bytes-per-element; the OPT-13B worked
  example gives 2 x 5120 x 40 x 2 = 819,200 bytes, which the page rounds
  to "800 KB" ([TEQ] "Why the KV cache is an allocator problem").  With
  grouped heads the hidden size is replaced by kv_heads x head_size.
* Waste after paging.  A sequence can waste memory only in its last,
  partly filled block, so at most block_size - 1 empty slots ([TEQ] "The
  OS already solved this in the 1960s").

Parity: pinned (the page's worked example, its per-sequence figures for
2,000 tokens, and the waste bound over every length up to 4,096).
"""


def kv_bytes_per_token(hidden, layers, bytes_per_elem):
    """Bytes of key + value cache for one token over all layers."""
    return 2 * hidden * layers * bytes_per_elem


def kv_bytes_per_token_layer(num_kv_heads, head_size, bytes_per_elem):
    """Bytes of key + value cache for one token in one layer."""
    return 2 * num_kv_heads * head_size * bytes_per_elem


def sequence_cache_bytes(tokens, hidden, layers, bytes_per_elem):
    """Bytes of cache held by one sequence of `tokens` tokens (all layers)."""
    return tokens * kv_bytes_per_token(hidden, layers, bytes_per_elem)


def blocks_needed(context_len, block_size=16):
    """Physical blocks a sequence of context_len tokens occupies."""
    return -(-context_len // block_size)


def empty_slots(context_len, block_size=16):
    """Allocated but unused slots: only the last block can be partial."""
    return blocks_needed(context_len, block_size) * block_size - context_len


def waste_fraction(context_lens, block_size=16):
    """Fraction of allocated slots that hold no token, over a batch."""
    lens = [int(x) for x in context_lens]
    allocated = sum(blocks_needed(L, block_size) * block_size for L in lens)
    if allocated == 0:
        return 0.0
    return sum(empty_slots(L, block_size) for L in lens) / allocated
