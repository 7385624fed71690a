"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each pin takes `o`, a namespace exposing the oracle's public functions,
and raises (AssertionError or any other exception) when the oracle is
wrong.  The same pins run against the real oracle (test_oracle_pins.py)
and against copies with a planted mistake (test_oracle_mutations.py),
which must each fail at least one pin.

What pins what:
* brute force: sequences are first drawn as contiguous [L, Hkv, D] arrays
  and scattered into a NaN-poisoned pool by explicit loops; attention is
  then recomputed from the contiguous arrays with pure-Python loops and,
  separately, with torch's float64 CPU scaled_dot_product_attention;
* placement freedom: any permutation of physical blocks (with the tables
  relabelled) leaves the output bit-identical -- the blocks "do not need
  to sit next to one another" ([AITJ] "How logical blocks, physical
  blocks and the block table work");
* grouped-query heads reduce to multi-head attention over kv heads
  repeated per query head (consecutive grouping);
* sharing: a block referenced by several sequences gives the same output
  as private duplicates ([TEQ] "Paging's second gift: copy-on-write");
* the partition merge equals the one-pass softmax;
* special cases: L = 1 gives v_0 exactly, q = 0 the mean of the values, a
  dominant logit the value of its token, L = 0 zeros;
* the worked OPT-13B bytes-per-token example and the 15-slot waste bound
  ([TEQ] "Why the KV cache is an allocator problem", "The OS already solved
  this in the 1960s");
* reshape_and_cache / copy_blocks against element-by-element loops.
"""

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BS = 16


# --------------------------------------------------------------- encodings --
def encode(x, dtype):
    """float32/64 numpy values -> storage array of `dtype` (RNE)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32))
    if dtype == "f32":
        return t.numpy().copy()
    if dtype == "f16":
        return t.to(torch.float16).numpy().copy()
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def widen(arr, dtype):
    """Storage array -> float64 via torch (independent of the oracle)."""
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double()
    return torch.from_numpy(a).double()


def nan_bits(dtype):
    return encode(np.array([np.nan], np.float32), dtype)[0]


# ------------------------------------------------------------ case builder --
def scatter_case(seed, lens, Hq, Hkv, D, dtype, extra_blocks=3, width=None):
    """Contiguous sequences scattered into a NaN-poisoned pool by loops."""
    rng = np.random.default_rng(seed)
    S = len(lens)
    nblk = [-(-L // BS) for L in lens]
    nb = sum(nblk) + extra_blocks
    width = max(max(nblk), 1) if width is None else width
    perm = rng.permutation(nb)
    pool_k = np.empty((nb, Hkv, BS, D), dtype=encode(np.zeros(1), dtype).dtype)
    pool_k[...] = nan_bits(dtype)
    pool_v = pool_k.copy()
    tables = np.full((S, width), -1, dtype=np.int32)
    seqs_k, seqs_v = [], []
    nxt = 0
    for s, L in enumerate(lens):
        k = encode(rng.standard_normal((L, Hkv, D)), dtype)
        v = encode(rng.standard_normal((L, Hkv, D)), dtype)
        seqs_k.append(k)
        seqs_v.append(v)
        for n in range(nblk[s]):
            tables[s, n] = perm[nxt]
            nxt += 1
        for t in range(L):
            b = tables[s, t // BS]
            for g in range(Hkv):
                pool_k[b, g, t % BS, :] = k[t, g]
                pool_v[b, g, t % BS, :] = v[t, g]
    q = encode(rng.standard_normal((S, Hq, D)), dtype)
    return dict(query=q, key_cache=pool_k, value_cache=pool_v,
                block_tables=tables, context_lens=np.asarray(lens, np.int32),
                seqs_k=seqs_k, seqs_v=seqs_v, Hq=Hq, Hkv=Hkv, D=D,
                dtype=dtype)


def run_oracle(o, c, scale, **kw):
    return o.decode_attention(c["query"], c["key_cache"], c["value_cache"],
                              c["block_tables"], c["context_lens"], scale,
                              c["Hkv"], c["dtype"], **kw)


def brute_force(c, scale):
    """Pure-Python loops over the contiguous sequences."""
    S, Hq, Hkv, D = len(c["context_lens"]), c["Hq"], c["Hkv"], c["D"]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((S, Hq, D))
    q = widen(c["query"], c["dtype"]).numpy()
    for s in range(S):
        K = widen(c["seqs_k"][s], c["dtype"]).numpy()
        V = widen(c["seqs_v"][s], c["dtype"]).numpy()
        L = K.shape[0]
        for h in range(Hq):
            g = h // G
            if L == 0:
                continue
            logits = [sc * sum(q[s, h, d] * K[t, g, d] for d in range(D))
                      for t in range(L)]
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            den = sum(w)
            for d in range(D):
                out[s, h, d] = sum(w[t] * V[t, g, d] for t in range(L)) / den
    return out


def torch_sdpa(c, scale):
    S, Hq, Hkv, D = len(c["context_lens"]), c["Hq"], c["Hkv"], c["D"]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D))
    q = widen(c["query"], c["dtype"])
    for s in range(S):
        K = widen(c["seqs_k"][s], c["dtype"])  # [L, Hkv, D]
        V = widen(c["seqs_v"][s], c["dtype"])
        if K.shape[0] == 0:
            continue
        Kh = K.repeat_interleave(G, dim=1).permute(1, 0, 2)[None]  # [1,Hq,L,D]
        Vh = V.repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
        qh = q[s][None, :, None, :]                                 # [1,Hq,1,D]
        r = torch.nn.functional.scaled_dot_product_attention(
            qh, Kh, Vh, scale=float(np.float32(scale)))
        out[s] = r[0, :, 0, :].numpy()
    return out


SMALL_CASES = [
    # (seed, lens, Hq, Hkv, D, dtype)
    (1, [1, 16, 17, 40], 4, 4, 8, "f32"),
    (2, [33, 5], 4, 2, 8, "f16"),
    (3, [80, 1, 31], 4, 1, 8, "bf16"),
    (4, [23, 48], 8, 2, 64, "f32"),
    (5, [64], 2, 2, 64, "f16"),
]


# -------------------------------------------------------------------- pins --
def pin_brute_force(o):
    for seed, lens, Hq, Hkv, D, dt in SMALL_CASES:
        c = scatter_case(seed, lens, Hq, Hkv, D, dt)
        scale = np.float32(1.0 / math.sqrt(D))
        got = run_oracle(o, c, scale)
        ref = brute_force(c, scale)
        err = np.abs(got - ref).max()
        assert err <= 1e-12, (seed, err)


def pin_torch_sdpa(o):
    for seed, lens, Hq, Hkv, D, dt in SMALL_CASES:
        c = scatter_case(seed + 50, lens, Hq, Hkv, D, dt)
        scale = np.float32(0.3)
        got = run_oracle(o, c, scale)
        ref = torch_sdpa(c, scale)
        err = np.abs(got - ref).max()
        assert err <= 1e-12, (seed, err)


def pin_permutation_invariance(o):
    c = scatter_case(11, [50, 3, 16, 77], 4, 2, 16, "f16", extra_blocks=9)
    scale = np.float32(0.25)
    ref = run_oracle(o, c, scale)
    rng = np.random.default_rng(12)
    for _ in range(3):
        nb = c["key_cache"].shape[0]
        pi = rng.permutation(nb)           # block b moves to pi[b]
        kc = np.empty_like(c["key_cache"])
        vc = np.empty_like(c["value_cache"])
        kc[pi] = c["key_cache"]
        vc[pi] = c["value_cache"]
        bt = c["block_tables"].copy()
        live = bt >= 0
        bt[live] = pi[bt[live]]
        c2 = dict(c, key_cache=kc, value_cache=vc, block_tables=bt)
        got = run_oracle(o, c2, scale)
        assert np.array_equal(got, ref)


def pin_gqa_reduction(o):
    G = 4
    c = scatter_case(21, [37, 64, 5], 8, 2, 16, "bf16")
    scale = np.float32(0.2)
    gqa = run_oracle(o, c, scale)
    mha = dict(c, key_cache=np.repeat(c["key_cache"], G, axis=1),
               value_cache=np.repeat(c["value_cache"], G, axis=1), Hkv=8)
    ref = run_oracle(o, mha, scale)
    assert np.array_equal(gqa, ref)


def pin_sharing_invariance(o):
    # three sequences share the first two blocks of sequence 0
    c = scatter_case(31, [40, 0, 0], 4, 4, 8, "f16", extra_blocks=12)
    nb = c["key_cache"].shape[0]
    bt = c["block_tables"]
    width = 4
    tables = np.full((3, width), -1, np.int32)
    tables[0, :3] = bt[0, :3]
    free = [b for b in range(nb) if b not in set(bt[0, :3].tolist())]
    kc, vc = c["key_cache"].copy(), c["value_cache"].copy()
    rng = np.random.default_rng(32)
    lens = [40, 32 + 9, 32 + 14]
    for s in (1, 2):
        tables[s, :2] = tables[0, :2]               # shared prefix
        b = free.pop()
        tables[s, 2] = b
        n = lens[s] - 32
        vals = encode(rng.standard_normal((2, 4, n, 8)), "f16")
        kc[b, :, :n] = vals[0]
        vc[b, :, :n] = vals[1]
    shared = dict(c, key_cache=kc, value_cache=vc, block_tables=tables,
                  context_lens=np.asarray(lens, np.int32))
    scale = np.float32(0.35)
    ref = run_oracle(o, shared, scale)
    # privately duplicate the shared blocks for sequences 1 and 2
    kc2, vc2, t2 = kc.copy(), vc.copy(), tables.copy()
    for s in (1, 2):
        for n in range(2):
            d = free.pop()
            kc2[d] = kc[tables[s, n]]
            vc2[d] = vc[tables[s, n]]
            t2[s, n] = d
    dup = dict(shared, key_cache=kc2, value_cache=vc2, block_tables=t2)
    assert np.array_equal(run_oracle(o, dup, scale), ref)
    assert np.isfinite(ref).all()


def pin_partition_merge(o):
    c = scatter_case(41, [1, 100, 47, 64], 4, 2, 8, "f32")
    scale = np.float32(0.5)
    ref = run_oracle(o, c, scale)
    assert np.isfinite(ref).all()
    for ps in (16, 32, 48, 512):
        got = o.decode_attention_partitioned(
            c["query"], c["key_cache"], c["value_cache"], c["block_tables"],
            c["context_lens"], scale, c["Hkv"], c["dtype"], ps)
        err = np.abs(got - ref).max()
        assert err <= 1e-12, (ps, err)
    # partial triples are self-consistent: m_p is the max logit of its slice
    _, parts = o.decode_attention_partitioned(
        c["query"], c["key_cache"], c["value_cache"], c["block_tables"],
        c["context_lens"], scale, c["Hkv"], c["dtype"], 32,
        return_partials=True)
    assert len(parts[(1, 0)]) == 4 and len(parts[(0, 0)]) == 1
    K = widen(c["seqs_k"][1], "f32").numpy()[:, 0]
    q = widen(c["query"], "f32").numpy()[1, 0]
    logits = float(np.float32(scale)) * (K @ q)
    for p, (m, s, _) in enumerate(parts[(1, 0)]):
        sl = logits[32 * p:32 * p + 32]
        assert abs(m - sl.max()) <= 1e-12
        assert abs(s - np.exp(sl - sl.max()).sum()) <= 1e-9


def pin_special_cases(o):
    # L = 1: the single weight is exp(0) = 1, so out = v_0 exactly.
    c = scatter_case(51, [1, 1], 2, 2, 16, "bf16")
    got = run_oracle(o, c, np.float32(0.7))
    for s in range(2):
        v0 = widen(c["seqs_v"][s], "bf16").numpy()[0]
        assert np.array_equal(got[s], v0)
    # q = 0: all logits equal, out = mean of the values.
    c = scatter_case(52, [29, 64], 2, 1, 8, "f16")
    c["query"][...] = encode(np.zeros(1), "f16")[0]
    got = run_oracle(o, c, np.float32(0.7))
    for s in range(2):
        V = widen(c["seqs_v"][s], "f16").numpy()[:, 0]
        assert np.abs(got[s] - V.mean(axis=0)).max() <= 1e-12
    # scale = 0 gives the mean as well.
    c = scatter_case(53, [20], 2, 2, 8, "f32")
    got = run_oracle(o, c, np.float32(0.0))
    V = widen(c["seqs_v"][0], "f32").numpy()
    for h in range(2):
        assert np.abs(got[0, h] - V[:, h].mean(axis=0)).max() <= 1e-12
    # a dominant logit: every other weight underflows to 0 -> its value.
    c = scatter_case(54, [45], 1, 1, 8, "f32")
    K = widen(c["seqs_k"][0], "f32").numpy()[:, 0]
    q = widen(c["query"], "f32").numpy()[0, 0]
    dots = np.sort(K @ q)
    t_star = int(np.argmax(K @ q))
    big = np.float32(2000.0 / (dots[-1] - dots[-2]))   # runner-up e^-2000 = 0
    got = run_oracle(o, c, big)
    V = widen(c["seqs_v"][0], "f32").numpy()[:, 0]
    assert np.array_equal(got[0, 0], V[t_star])
    # L = 0: zeros.
    c = scatter_case(55, [0, 3], 2, 2, 8, "f16")
    got = run_oracle(o, c, np.float32(0.5))
    assert np.array_equal(got[0], np.zeros((2, 8)))
    assert np.isfinite(got[1]).all()


def pin_kv_bytes(o):
    with open(os.path.join(GOLDEN, "opt13b_kv_bytes.json")) as f:
        g = json.load(f)
    per_tok = o.kv_bytes_per_token(g["hidden"], g["layers"], g["bytes_per_value"])
    assert per_tok == g["kv_bytes_per_token"]
    assert per_tok == g["stated_kv_per_token_kb"] * 1024
    seq = o.sequence_cache_bytes(g["sequence_tokens"], g["hidden"], g["layers"],
                                 g["bytes_per_value"])
    assert abs(seq / 1e9 - g["stated_sequence_gb"]) < 0.05   # "roughly 1.6 GB"
    llama = o.sequence_cache_bytes(2048, 5120, 40, 2)
    assert llama / 1e9 <= g["llama13b_stated_upper_gb"]
    # one layer of the 40-head, 128-wide shape is 1/40 of the token's cache
    assert o.kv_bytes_per_token_layer(40, 128, 2) * g["layers"] == per_tok
    # grouped heads: 8 kv heads of 128 in bf16
    assert o.kv_bytes_per_token_layer(8, 128, 2) == 4096


def pin_waste_bound(o):
    with open(os.path.join(GOLDEN, "waste_bound.json")) as f:
        g = json.load(f)
    bs = g["block_size"]
    worst = max(o.empty_slots(L, bs) for L in range(1, 4097))
    assert worst == g["max_empty_slots_per_sequence"]
    assert all(o.empty_slots(L, bs) >= 0 for L in range(0, 4097))
    assert o.empty_slots(16, bs) == 0 and o.empty_slots(17, bs) == 15
    assert o.blocks_needed(0, bs) == 0 and o.blocks_needed(1, bs) == 1
    # the waste fraction of a batch is bounded by 15 / (16 * min blocks)
    rng = np.random.default_rng(61)
    lens = rng.integers(1, 2049, size=64)
    wf = o.waste_fraction(lens, bs)
    assert 0 <= wf < g["stated_waste_upper_fraction"]
    assert abs(wf - sum(o.empty_slots(int(L), bs) for L in lens) /
               sum(16 * o.blocks_needed(int(L), bs) for L in lens)) < 1e-15


def pin_reshape_and_cache(o):
    rng = np.random.default_rng(71)
    nb, Hkv, D, T = 6, 3, 8, 10
    for dt in ("f32", "f16", "bf16"):
        kc = encode(rng.standard_normal((nb, Hkv, BS, D)), dt)
        vc = encode(rng.standard_normal((nb, Hkv, BS, D)), dt)
        key = encode(rng.standard_normal((T, Hkv, D)), dt)
        val = encode(rng.standard_normal((T, Hkv, D)), dt)
        slots = rng.choice(nb * BS, size=T, replace=False).astype(np.int64)
        slots[3] = -1
        nk, nv = o.reshape_and_cache(key, val, slots, kc, vc)
        ek, ev = kc.copy(), vc.copy()
        for i in range(T):
            if slots[i] < 0:
                continue
            for g in range(Hkv):
                for d in range(D):
                    ek[slots[i] // BS, g, slots[i] % BS, d] = key[i, g, d]
                    ev[slots[i] // BS, g, slots[i] % BS, d] = val[i, g, d]
        assert nk.tobytes() == ek.tobytes() and nv.tobytes() == ev.tobytes()
        assert kc.tobytes() != nk.tobytes()          # inputs not modified
    # write-then-gather: tokens written through a table read back in order
    nb, Hkv, D = 5, 2, 4
    kc = encode(np.full((nb, Hkv, BS, D), np.nan), "f16")
    table = np.array([3, 0, 4], np.int32)
    L = 40
    key = encode(rng.standard_normal((L, Hkv, D)), "f16")
    slots = np.array([table[t // BS] * BS + t % BS for t in range(L)], np.int64)
    nk, nv = o.reshape_and_cache(key, key, slots, kc, kc)
    for g in range(Hkv):
        back = o.gather_sequence_kv(nk, table, L, g, "f16")
        assert np.array_equal(back, key[:, g].astype(np.float64))
    # rejections
    for bad in ([1, 1], [nb * BS]):
        try:
            o.reshape_and_cache(key[:len(bad)], key[:len(bad)],
                                np.array(bad, np.int64), kc, kc)
        except ValueError:
            continue
        raise AssertionError(f"slots {bad} accepted")


def pin_copy_blocks(o):
    rng = np.random.default_rng(81)
    nb, Hkv, D = 8, 2, 8
    for dt in ("f16", "bf16", "f32"):
        kc = encode(rng.standard_normal((nb, Hkv, BS, D)), dt)
        vc = encode(rng.standard_normal((nb, Hkv, BS, D)), dt)
        kc[1, 0, 3, 2] = nan_bits(dt)
        pairs = np.array([[1, 4], [1, 6], [2, 7]], np.int64)
        nk, nv = o.copy_blocks(kc, vc, pairs)
        ek, ev = kc.copy(), vc.copy()
        for s, d in pairs:
            for g in range(Hkv):
                for t in range(BS):
                    for e in range(D):
                        ek[d, g, t, e] = kc[s, g, t, e]
                        ev[d, g, t, e] = vc[s, g, t, e]
        assert nk.tobytes() == ek.tobytes() and nv.tobytes() == ev.tobytes()
    for bad in ([[1, 2], [3, 2]], [[1, 2], [2, 3]], [[0, nb]]):
        try:
            o.copy_blocks(kc, vc, np.array(bad, np.int64))
        except ValueError:
            continue
        raise AssertionError(f"pairs {bad} accepted")


def pin_formats(o):
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xC000, 0x0001, 0x7F80, 0xFF80],
                    dtype=np.uint16)
    want = np.array([0.0, -0.0, 1.0, -2.0, 2.0 ** -133, np.inf, -np.inf])
    got = o.to_f64(bits, "bf16")
    assert np.array_equal(got, want)
    assert np.signbit(got[1])
    assert np.isnan(o.to_f64(np.array([0x7FC0], np.uint16), "bf16")[0])
    h = np.array([1.5, -0.0, 65504.0, 2.0 ** -24], np.float16)
    assert np.array_equal(o.to_f64(h, "f16"), h.astype(np.float64))
    f = np.array([1e-45, 3.4e38, -7.25], np.float32)
    assert np.array_equal(o.to_f64(f, "f32"), f.astype(np.float64))


def _torch_e4m3(x32):
    """torch's float8_e4m3fn codes of float32 values (a library routine
    independent of the oracle; it rounds to nearest even and gives NaN
    beyond the largest finite value, so callers stay below 448)."""
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_codec(o):
    """OCP E4M3: every code decodes as torch's float8_e4m3fn does; hand
    values of the definition; encoding rounds as torch wherever torch stays
    finite (random values, every code's value, every midpoint between
    neighbouring codes: the ties); the round trip of every code; saturation
    at +-448 and NaN (the reading for values torch would turn into NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    d = o.e4m3_decode(codes)
    t = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(t)
    assert nan.sum() == 2 and np.array_equal(np.isnan(d), nan)
    assert np.array_equal(d[~nan], t[~nan])
    assert np.array_equal(np.signbit(d[~nan]), np.signbit(t[~nan]))
    for c, v in ((0x38, 1.0), (0x40, 2.0), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
                 (0x08, 2.0 ** -6), (0x0F, 1.875 * 2.0 ** -6), (0x80, -0.0), (0xB8, -1.0)):
        assert d[c] == v and np.signbit(d[c]) == np.signbit(v), hex(c)
    rng = np.random.default_rng(8)
    pos = d[(~nan) & (codes < 0x80)]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)      # exact in float32
    x = np.concatenate([rng.standard_normal(20000) * sd for sd in (0.003, 1.0, 60.0)] +
                       [mids, -mids, pos, -pos]).astype(np.float32)
    x = x[np.abs(x) < 448]
    assert np.array_equal(o.e4m3_encode(x), _torch_e4m3(x))
    assert np.array_equal(o.e4m3_encode(d[~nan].astype(np.float32)), codes[~nan])
    sat = o.e4m3_encode(np.float32([448.0, 460.0, 1e6, -1e30, np.inf, -np.inf]))
    assert sat.tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]
    assert o.e4m3_encode(np.float32([np.nan])).tolist() == [0x7F]


def pin_reshape_fp8(o):
    """New tokens land in their slots as the codes of value / scale (the
    quotient in float32, encoded by torch), untouched slots keep their
    codes, negative slots are skipped."""
    rng = np.random.default_rng(9)
    NB, Hkv, D = 6, 2, 8
    kc = rng.integers(0, 256, (NB, Hkv, BS, D), dtype=np.uint8)
    vc = rng.integers(0, 256, (NB, Hkv, BS, D), dtype=np.uint8)
    key = (rng.standard_normal((5, Hkv, D)) * 3).astype(np.float16)
    val = (rng.standard_normal((5, Hkv, D)) * 3).astype(np.float16)
    slots = np.array([17, -1, 0, 95, 40], np.int64)
    ks, vs = np.float32(0.0625), np.float32(0.03)
    nk, nv = o.reshape_and_cache_fp8(key, val, slots, kc, vc, ks, vs, "f16")
    ek, ev = kc.copy(), vc.copy()
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        b, off = divmod(int(slot), BS)
        ek[b, :, off, :] = _torch_e4m3(key[i].astype(np.float32) / ks)
        ev[b, :, off, :] = _torch_e4m3(val[i].astype(np.float32) / vs)
    assert nk.dtype == np.uint8 and np.array_equal(nk, ek) and np.array_equal(nv, ev)


def pin_decode_fp8(o):
    """Attention over e4m3 pools with per-pool scales equals attention over
    float32 pools holding decode(code) * scale, decoded by torch (scales are
    powers of two, so those products are exact)."""
    rng = np.random.default_rng(10)
    lens, Hq, Hkv, D = [1, 17, 40], 4, 2, 8
    NB = 12
    kc = rng.integers(0, 0x7E, (NB, Hkv, BS, D), dtype=np.uint8)
    vc = rng.integers(0, 0x7E, (NB, Hkv, BS, D), dtype=np.uint8)
    kc ^= (rng.integers(0, 2, kc.shape) * 0x80).astype(np.uint8)   # both signs
    vc ^= (rng.integers(0, 2, vc.shape) * 0x80).astype(np.uint8)
    tables = np.full((3, 4), -1, np.int64)
    perm = rng.permutation(NB)
    n = 0
    for s, L in enumerate(lens):
        nbk = -(-L // BS)
        tables[s, :nbk] = perm[n:n + nbk]
        n += nbk
    q = rng.standard_normal((3, Hq, D)).astype(np.float16)
    ks, vs = np.float32(0.125), np.float32(4.0)
    got = o.decode_attention(q, kc, vc, tables, np.array(lens), 0.5, Hkv, "f16",
                             kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    dec = lambda c: torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    want = o.decode_attention(q, dec(kc) * ks, dec(vc) * vs, tables, np.array(lens), 0.5, Hkv,
                              "f16", kv_dtype="f32")
    assert np.array_equal(got, want)
    assert np.isfinite(got).all() and np.abs(got).max() > 0


# ----------------------------------------------------------------- prefill --
def prefill_case(seed, lens, news, Hq, Hkv, D, dtype, extra_blocks=3):
    """scatter_case plus packed queries: sequence s has news[s] new rows,
    its last news[s] tokens."""
    c = scatter_case(seed, lens, Hq, Hkv, D, dtype, extra_blocks=extra_blocks)
    rng = np.random.default_rng(seed + 1000)
    qsl = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    c["query"] = encode(rng.standard_normal((int(qsl[-1]), Hq, D)), dtype)
    c["query_start_loc"] = qsl
    return c


def run_prefill(o, c, scale):
    return o.prefill_attention(c["query"], c["key_cache"], c["value_cache"],
                               c["block_tables"], c["context_lens"], c["query_start_loc"],
                               scale, c["Hkv"], c["dtype"])


def torch_causal(c, scale):
    """torch float64 attention on the contiguous copies with the mask written
    out: row i of a sequence with L tokens and n new rows sees t <= L - n + i
    (is_causal=True when n = L)."""
    Hq, Hkv = c["Hq"], c["Hkv"]
    G = Hq // Hkv
    q = widen(c["query"], c["dtype"])
    qsl = c["query_start_loc"]
    out = np.zeros(tuple(q.shape))
    for s in range(len(c["context_lens"])):
        a, b = int(qsl[s]), int(qsl[s + 1])
        n, L = b - a, int(c["context_lens"][s])
        if n == 0:
            continue
        K = widen(c["seqs_k"][s], c["dtype"]).repeat_interleave(G, dim=1).permute(1, 0, 2)
        V = widen(c["seqs_v"][s], c["dtype"]).repeat_interleave(G, dim=1).permute(1, 0, 2)
        qh = q[a:b].permute(1, 0, 2)                                  # [Hq, n, D]
        if n == L:
            r = torch.nn.functional.scaled_dot_product_attention(
                qh, K, V, is_causal=True, scale=float(np.float32(scale)))
        else:
            mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
            r = torch.nn.functional.scaled_dot_product_attention(
                qh, K, V, attn_mask=mask, scale=float(np.float32(scale)))
        out[a:b] = r.permute(1, 0, 2).numpy()
    return out


PREFILL_CASES = [
    # (seed, lens, new rows, Hq, Hkv, D, dtype)
    (21, [17, 40, 5], [17, 40, 5], 4, 2, 8, "f16"),     # whole prompts
    (22, [33, 70, 16], [9, 1, 16], 4, 4, 8, "bf16"),    # chunks after a prefix
    (23, [50, 3], [20, 0], 8, 2, 16, "f32"),
    (24, [64, 31], [32, 31], 2, 1, 64, "f16"),
]


def pin_prefill_torch(o):
    for seed, lens, news, Hq, Hkv, D, dt in PREFILL_CASES:
        c = prefill_case(seed, lens, news, Hq, Hkv, D, dt)
        # the usual scale, a negative one and zero (equal weights over the
        # visible tokens), each against torch's own float64 attention
        for scale in (np.float32(1.0 / math.sqrt(D)), np.float32(-0.3), np.float32(0.0)):
            got = run_prefill(o, c, scale)
            ref = torch_causal(c, scale)
            assert got.shape == ref.shape
            err = np.abs(got - ref).max()
            assert err <= 1e-12, (seed, float(scale), err)


def pin_prefill_loops(o):
    """Pure-Python loops with the visibility rule written out, tiny sizes."""
    c = prefill_case(25, [19, 6], [5, 6], 4, 2, 4, "f32")
    scale = np.float32(0.7)
    got = run_prefill(o, c, scale)
    q = widen(c["query"], "f32").numpy()
    qsl = c["query_start_loc"]
    for s, L in enumerate(c["context_lens"]):
        K = widen(c["seqs_k"][s], "f32").numpy()
        V = widen(c["seqs_v"][s], "f32").numpy()
        n = int(qsl[s + 1] - qsl[s])
        for i in range(n):
            for h in range(4):
                g = h // 2
                logits = [float(scale) * sum(q[qsl[s] + i, h, d] * K[t, g, d] for d in range(4))
                          for t in range(int(L)) if t <= int(L) - n + i]
                m = max(logits)
                w = [math.exp(x - m) for x in logits]
                for d in range(4):
                    want = sum(w[t] * V[t, g, d] for t in range(len(w))) / sum(w)
                    assert abs(got[qsl[s] + i, h, d] - want) <= 1e-12


def pin_prefill_rows_are_decodes(o):
    """Row i of a chunk equals a decode step of the same query at length
    L - n + i + 1 (same pool, same table): the two oracles agree exactly."""
    c = prefill_case(26, [45, 20], [13, 20], 4, 2, 8, "f16", extra_blocks=5)
    scale = np.float32(0.4)
    got = run_prefill(o, c, scale)
    qsl = c["query_start_loc"]
    for s, L in enumerate(c["context_lens"]):
        n = int(qsl[s + 1] - qsl[s])
        for i in range(n):
            lens = np.zeros(len(c["context_lens"]), np.int32)
            lens[s] = int(L) - n + i + 1
            q = np.zeros((len(lens),) + c["query"].shape[1:], c["query"].dtype)
            q[s] = c["query"][qsl[s] + i]
            d = o.decode_attention(q, c["key_cache"], c["value_cache"], c["block_tables"],
                                   lens, scale, c["Hkv"], c["dtype"], seqs=[s])
            assert np.array_equal(d[s], got[qsl[s] + i]), (s, i)


def pin_prefill_permutation_invariance(o):
    c = prefill_case(27, [50, 16, 77], [10, 16, 3], 4, 2, 16, "bf16", extra_blocks=9)
    scale = np.float32(0.25)
    ref = run_prefill(o, c, scale)
    pi = np.random.default_rng(28).permutation(c["key_cache"].shape[0])
    kc = np.empty_like(c["key_cache"])
    vc = np.empty_like(c["value_cache"])
    kc[pi] = c["key_cache"]
    vc[pi] = c["value_cache"]
    bt = c["block_tables"].copy()
    bt[bt >= 0] = pi[bt[bt >= 0]]
    got = run_prefill(o, dict(c, key_cache=kc, value_cache=vc, block_tables=bt), scale)
    assert np.array_equal(got, ref)


ALL_PINS = [
    pin_brute_force, pin_torch_sdpa, pin_permutation_invariance,
    pin_gqa_reduction, pin_sharing_invariance, pin_partition_merge,
    pin_special_cases, pin_kv_bytes, pin_waste_bound,
    pin_reshape_and_cache, pin_copy_blocks, pin_formats,
    pin_e4m3_codec, pin_reshape_fp8, pin_decode_fp8,
    pin_prefill_torch, pin_prefill_loops, pin_prefill_rows_are_decodes,
    pin_prefill_permutation_invariance,
]
