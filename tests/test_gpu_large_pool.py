"""Pools larger than 4 GiB per tensor (marked gpu).

Every kernel addresses a block as block id x block bytes; with 40 kv heads
of 128 float16 elements a block of one tensor is 160 KiB, so block ids above
26 214 lie beyond 2^32 bytes.  These tests place the sequences' blocks at the
top of a 30 000-block pool (4.6 GiB per tensor) and check, against the
oracle on host copies of just those blocks: decode (both piece policies),
the decode call that caches the new token, reshape_and_cache, copy_blocks
and prefill.  The decode output must also be bitwise the same as with the
same blocks moved to the bottom of the pool (placement invariance).
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_311_amd as pkv
from paged_kv_cache_311_amd import workloads as wl
from tests.gpu_helpers import BS, DEV, assert_close, bits, dev_i32, dev_i64, gather_blocks, say

pytestmark = pytest.mark.gpu

NB, HKV, HQ, D = 30000, 40, 40, 128
LENS = [37, 300, 1000, 17]
SCALE = np.float32(1.0 / np.sqrt(D))


@pytest.fixture(scope="module")
def big():
    """A 30 000-block float16 pool pair, the sequences' blocks at the top
    (one sequence also has a block near the bottom), random N(0,1) rows in
    those blocks only."""
    rng = np.random.default_rng(4242)
    need = [-(-L // BS) for L in LENS]
    ids = rng.choice(np.arange(NB - 3000, NB), size=sum(need), replace=False)
    ids[0] = 5
    W = max(need)
    bt = np.full((len(LENS), W), -1, np.int32)
    k = 0
    for s, n in enumerate(need):
        bt[s, :n] = ids[k:k + n]
        k += n
    kc = torch.empty((NB, HKV, BS, D), dtype=torch.float16, device=DEV)
    vc = torch.empty_like(kc)
    g = torch.Generator(device=DEV).manual_seed(7)
    used = torch.from_numpy(np.asarray(ids, np.int64)).to(DEV)
    kc[used] = torch.randn((len(ids), HKV, BS, D), generator=g, device=DEV).half()
    vc[used] = torch.randn((len(ids), HKV, BS, D), generator=g, device=DEV).half()
    q = torch.randn((len(LENS), HQ, D), generator=g, device=DEV).half()
    say(f"    pool {2 * kc.numel() * 2 / 2**30:.1f} GiB, highest block offset "
        f"{int(ids.max()) * HKV * BS * D * 2 / 2**30:.2f} GiB")
    yield dict(kc=kc, vc=vc, bt=bt, lens=np.asarray(LENS, np.int32), q=q, ids=ids)
    del kc, vc
    torch.cuda.empty_cache()


def sub_pool(kc, vc, bt, lens):
    """Host copies of the blocks the sequences read, and remapped tables."""
    ids = sorted({int(x) for s, L in enumerate(lens) for x in bt[s, :-(-int(L) // BS)]})
    remap = {b: i for i, b in enumerate(ids)}
    tables = np.full(bt.shape, -1, np.int32)
    for s, L in enumerate(lens):
        n = -(-int(L) // BS)
        tables[s, :n] = [remap[int(x)] for x in bt[s, :n]]
    return gather_blocks(kc, ids), gather_blocks(vc, ids), tables, remap


@pytest.mark.parametrize("ps", [0, 512])
def test_decode_beyond_4gib(gpu_lib, big, ps):
    b = big
    out = torch.empty_like(b["q"])
    pkv.paged_attention_decode(out, b["q"], b["kc"], b["vc"], dev_i32(b["bt"]),
                               dev_i32(b["lens"]), float(SCALE), HKV, partition_size=ps,
                               validate=True)
    torch.cuda.synchronize()
    kh, vh, tables, _ = sub_pool(b["kc"], b["vc"], b["bt"], b["lens"])
    ref = oracle.decode_attention(wl.to_host(b["q"]), kh, vh, tables, b["lens"], SCALE, HKV,
                                  "f16")
    assert_close(out, ref, "f16", f"decode, pool beyond 4 GiB, partition {ps}")
    # the same blocks at the bottom of a small pool: the same bits
    n = len(kh)
    kl = torch.from_numpy(kh).to(DEV)
    vl = torch.from_numpy(vh).to(DEV)
    out2 = torch.empty_like(out)
    pkv.paged_attention_decode(out2, b["q"], kl, vl, dev_i32(tables), dev_i32(b["lens"]),
                               float(SCALE), HKV, partition_size=ps)
    torch.cuda.synchronize()
    assert n < 200 and torch.equal(bits(out), bits(out2))


@pytest.mark.parametrize("group", [4, 16])
def test_grouped_decode_beyond_4gib(gpu_lib, big, group):
    """4 and 16 query heads per kv head: the matrix-core path (both products
    on MFMA, values through LDS) on the same pool beyond 4 GiB."""
    b = big
    g = torch.Generator(device=DEV).manual_seed(11 + group)
    q = torch.randn((len(LENS), HKV * group, D), generator=g, device=DEV).half()
    out = torch.empty_like(q)
    pkv.paged_attention_decode(out, q, b["kc"], b["vc"], dev_i32(b["bt"]), dev_i32(b["lens"]),
                               float(SCALE), HKV, partition_size=512, validate=True)
    torch.cuda.synchronize()
    kh, vh, tables, _ = sub_pool(b["kc"], b["vc"], b["bt"], b["lens"])
    ref = oracle.decode_attention(wl.to_host(q), kh, vh, tables, b["lens"], SCALE, HKV, "f16")
    assert_close(out, ref, "f16", f"decode, {group} heads per kv head, pool beyond 4 GiB")


def test_cache_ops_and_append_beyond_4gib(gpu_lib, big):
    """copy_blocks between high blocks, reshape_and_cache into high slots,
    then the decode call that caches each sequence's newest token there."""
    b = big
    bt = b["bt"].copy()
    lens = b["lens"]
    free = np.setdiff1d(np.arange(26500, NB - 3000), b["ids"])  # above 4 GiB, unused
    # copy-on-write of each sequence's last block into a fresh high block
    pairs = []
    for s, L in enumerate(lens):
        last = (int(L) - 1) // BS
        dst = int(free[s])
        pairs.append((int(bt[s, last]), dst))
        bt[s, last] = dst
    pairs = np.asarray(pairs, np.int64)
    # reshape_and_cache: two tokens per sequence before the newest one
    slots = []
    for s, L in enumerate(lens):
        for pos in (max(int(L) - 3, 0), max(int(L) - 2, 0)):
            slots.append(int(bt[s, pos // BS]) * BS + pos % BS)
    slots = np.asarray(slots, np.int64)
    g = torch.Generator(device=DEV).manual_seed(3)
    key = torch.randn((len(slots), HKV, D), generator=g, device=DEV).half()
    val = torch.randn((len(slots), HKV, D), generator=g, device=DEV).half()
    nk = torch.randn((len(lens), HKV, D), generator=g, device=DEV).half()
    nv = torch.randn((len(lens), HKV, D), generator=g, device=DEV).half()

    touched = sorted({int(x) for x in pairs.reshape(-1)} | {int(s) // BS for s in slots} |
                     {int(bt[s, (int(L) - 1) // BS]) for s, L in enumerate(lens)})
    remap = {x: i for i, x in enumerate(touched)}
    k0, v0 = gather_blocks(b["kc"], touched), gather_blocks(b["vc"], touched)

    pkv.copy_blocks(b["kc"], b["vc"], dev_i64(pairs), validate=True)
    pkv.reshape_and_cache(key, val, dev_i64(slots), b["kc"], b["vc"], validate=True)
    out = torch.empty_like(b["q"])
    pkv.paged_attention_decode_append(out, b["q"], b["kc"], b["vc"], dev_i32(bt), dev_i32(lens),
                                      nk, nv, float(SCALE), HKV, partition_size=512,
                                      validate=True)
    torch.cuda.synchronize()

    ek, ev = oracle.copy_blocks(k0, v0, np.asarray([(remap[int(a)], remap[int(c)])
                                                     for a, c in pairs], np.int64))
    sub = np.asarray([remap[int(x) // BS] * BS + int(x) % BS for x in slots], np.int64)
    ek, ev = oracle.reshape_and_cache(wl.to_host(key), wl.to_host(val), sub, ek, ev)
    new_slots = np.asarray([remap[int(bt[s, (int(L) - 1) // BS])] * BS + (int(L) - 1) % BS
                            for s, L in enumerate(lens)], np.int64)
    ek, ev = oracle.reshape_and_cache(wl.to_host(nk), wl.to_host(nv), new_slots, ek, ev)
    assert gather_blocks(b["kc"], touched).tobytes() == ek.tobytes()
    assert gather_blocks(b["vc"], touched).tobytes() == ev.tobytes()

    kh, vh, tables, _ = sub_pool(b["kc"], b["vc"], bt, lens)
    ref = oracle.decode_attention(wl.to_host(b["q"]), kh, vh, tables, lens, SCALE, HKV, "f16")
    assert_close(out, ref, "f16", "decode_append, pool beyond 4 GiB")


def test_prefill_beyond_4gib(gpu_lib, big):
    """The last 40 tokens of each sequence attended as a prefill chunk."""
    b = big
    lens = b["lens"]
    n = np.minimum(lens, 40)
    qsl = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    g = torch.Generator(device=DEV).manual_seed(9)
    q = torch.randn((int(qsl[-1]), HQ, D), generator=g, device=DEV).half()
    out = torch.empty_like(q)
    pkv.paged_attention_prefill(out, q, b["kc"], b["vc"], dev_i32(b["bt"]), dev_i32(lens),
                                dev_i32(qsl), float(SCALE), HKV, int(n.max()), validate=True)
    torch.cuda.synchronize()
    kh, vh, tables, _ = sub_pool(b["kc"], b["vc"], b["bt"], lens)
    ref = oracle.prefill_attention(wl.to_host(q), kh, vh, tables, lens, qsl, SCALE, HKV, "f16")
    assert_close(out, ref, "f16", "prefill, pool beyond 4 GiB")
