"""Decode on a virtually contiguous pool (pkv_vpool: HIP virtual-memory
ranges backed on demand; marked gpu).

Each sequence gets a run of consecutive virtual blocks, backed by physical
granules only where it has tokens ([TEQ] "The tradeoff: you just wrote a
virtual memory subsystem in userspace": the contiguous-but-virtual
alternative to block tables).  The kernels are the same, so the outputs
must equal the paged layout's bit for bit, and the appending call must
store the same bytes.  Before any launch every block a sequence reads is
checked to be mapped.
"""

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_311_amd as pkv
from paged_kv_cache_311_amd import workloads as wl
from tests.gpu_helpers import (BS, DEV, assert_close, bits, clone_pools, dev_i32,
                               oracle_decode_subset, run_decode, say)

pytestmark = pytest.mark.gpu


def into_virtual_pool(b):
    """The batch's blocks copied into a virtual pool, sequence s at virtual
    blocks s*W .. s*W + n_s - 1; returns (pool, virtual tables)."""
    w = b["workload"]
    bt, lens = b["block_tables"], b["context_lens"]
    S, W = bt.shape
    vp = pkv.VirtualPool(S * W, w.num_kv_heads, w.head_size, w.kv_dtype or w.dtype)
    vt = np.full_like(bt, -1)
    src, dst = [], []
    for s in range(S):
        n = -(-int(lens[s]) // BS)
        if n == 0:
            continue
        vp.map(s * W, n)
        assert vp.covers(s * W, n)
        vt[s, :n] = s * W + np.arange(n)
        src.extend(int(x) for x in bt[s, :n])
        dst.extend(int(x) for x in vt[s, :n])
    si = torch.tensor(src, dtype=torch.int64, device=DEV)
    di = torch.tensor(dst, dtype=torch.int64, device=DEV)
    for pool, src_pool in ((vp.key_cache, b["key_cache"]), (vp.value_cache, b["value_cache"])):
        pool[di] = src_pool[si].view(pool.dtype)   # bits (E4M3 pools hold uint8 codes)
    torch.cuda.synchronize()
    return vp, vt


@pytest.mark.parametrize("key,kw", [("opt13b", dict(num_seqs=8)),
                                    ("long_gqa", dict(num_seqs=1)),
                                    ("opt13b_fp8", dict(num_seqs=8))])
def test_decode_on_virtual_pool_matches_paged(gpu_lib, key, kw):
    w = dataclasses.replace(wl.WORKLOADS[key], **kw)
    b = wl.make_batch(w, w.default_seed + 5, DEV)
    kc0, vc0 = clone_pools(b)
    out = run_decode(b).clone()
    vp, vt = into_virtual_pool(b)
    try:
        out_v = run_decode(dict(b, key_cache=vp.key_cache, value_cache=vp.value_cache,
                                block_tables=vt))
        assert torch.equal(bits(out), bits(out_v))
        ref = oracle_decode_subset(b, kc0, vc0, list(range(w.num_seqs)))
        assert_close(out_v, ref, w.dtype, f"virtual pool {key}")
        used = sum(-(-int(L) // BS) for L in b["context_lens"]) * vp.block_bytes
        say(f"    {key}: {used / 2**20:.1f} MiB of blocks per tensor, "
            f"{vp.mapped_bytes / 2 / 2**20:.1f} MiB mapped, granule {vp.granularity >> 20} MiB")
    finally:
        vp.close()


def test_append_on_virtual_pool_matches_paged(gpu_lib):
    w = dataclasses.replace(wl.WORKLOADS["llama13b_conv"], num_seqs=12)
    b = wl.make_batch(w, 21, DEV)
    vp, vt = into_virtual_pool(b)
    try:
        outs = []
        for kc, vc, tables in ((b["key_cache"], b["value_cache"], b["block_tables"]),
                               (vp.key_cache, vp.value_cache, vt)):
            out = torch.empty_like(b["query"])
            pkv.paged_attention_decode_append(out, b["query"], kc, vc, dev_i32(tables),
                                              dev_i32(b["context_lens"]), b["key"], b["value"],
                                              float(w.scale), w.num_kv_heads, partition_size=512)
            torch.cuda.synchronize()
            outs.append(out)
        assert torch.equal(bits(outs[0]), bits(outs[1]))
        for s, L in enumerate(b["context_lens"]):
            n = (int(L) - 1) // BS
            pb, vb = int(b["block_tables"][s, n]), int(vt[s, n])
            assert torch.equal(bits(b["key_cache"][pb]), bits(vp.key_cache[vb]))
            assert torch.equal(bits(b["value_cache"][pb]), bits(vp.value_cache[vb]))
    finally:
        vp.close()


def test_virtual_pool_mapping(gpu_lib):
    """Granules are mapped on demand, once; coverage reflects them."""
    with pkv.VirtualPool(4096, 8, 128, "f16") as vp:  # 32 KiB blocks, 128 MiB per tensor
        g = vp.granularity
        per = g // vp.block_bytes
        assert g >= 2 << 20 and vp.mapped_bytes == 2 * g     # the first granule
        assert vp.covers(0, per) and not vp.covers(per, 1)
        vp.map(10 * per + 3, 2 * per)                        # spans three granules
        assert vp.mapped_bytes == 2 * 4 * g
        assert vp.covers(10 * per, 3 * per) and not vp.covers(13 * per, 1)
        vp.map(10 * per, per)                                # already mapped: no change
        assert vp.mapped_bytes == 2 * 4 * g
        with pytest.raises(pkv.PagedKVError):
            vp.map(4090, 10)                                 # past the end
        vp.key_cache[10 * per + 5].fill_(1.5)
        torch.cuda.synchronize()
        assert float(vp.key_cache[10 * per + 5].float().mean()) == 1.5
    assert vp.key_cache is None and vp.mapped_bytes == 0   # closed on exit
