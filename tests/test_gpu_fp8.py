"""Parity of the E4M3 pool path with the CPU oracle on an MI355X (marked gpu).

Pools hold OCP E4M3 codes with one float32 scale per pool.  The pages set
KV-cache quantization (cached values in a lower-precision representation)
beside paging as the remedy for too many bytes per token ("PagedAttention
KV cache memory management" [AITJ], "PagedAttention vs KV-cache
quantization vs prefix caching") and name no format; the 8-bit E4M3 format
is this project's choice, half the bytes of a 16-bit pool.  reshape_and_cache_fp8
and copy_blocks on such pools are compared bit for bit with the oracle;
paged_attention_decode_fp8 within the tolerances of the other parity tests
(5e-3 for float16/bfloat16 queries, plus half an output ulp for bfloat16),
against the oracle's float64 attention over the decoded, scaled codes.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_311_amd as pkv
from paged_kv_cache_311_amd import workloads as wl
from tests.gpu_helpers import (DEV, assert_close, bits, clone_pools, dev_i32, dev_i64,
                               full_step_and_check, oracle_decode_subset, run_decode,
                               sample_seqs, say)

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS
BS = wl.BLOCK_SIZE
# a scale that is not a power of two, so folding it into the logits rounds
ODD = dict(kv_dtype="e4m3", k_scale=0.0137, v_scale=0.0211)


def fp8_variant(key, **kw):
    return dataclasses.replace(W[key], kv_dtype="e4m3", k_scale=wl.FP8_K_SCALE,
                               v_scale=wl.FP8_V_SCALE, **kw)


# ------------------------------------------------------------- pool writes --
def special_values(scale):
    """Quotients x / scale on and around the E4M3 grid: ties between codes
    (even and odd mantissa), the saturation edge and beyond, subnormals and
    the underflow tie, zeros of both signs, infinities and NaN."""
    q = [1.0625, 1.1875, 0.5625 * 2 ** -6, 2 ** -10, 2 ** -11, 3 * 2 ** -10, 448.0, 464.0,
         480.0, 1e6, 0.0, -0.0, 240.0, 232.0, 1.0 + 2 ** -4 + 2 ** -12, 0.013671875]
    q = np.asarray(q + [-x for x in q], np.float64)
    vals = list(q * scale) + [np.inf, -np.inf, np.nan]
    return np.asarray(vals, np.float64)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_reshape_and_cache_fp8_bit_exact(gpu_lib, dtype, d):
    rng = np.random.default_rng(d + len(dtype))
    td = wl.torch_dtype(dtype)
    NB, Hkv, T = 12, 2, 70
    ks, vs = 1.0 / 64, 0.0211                     # one exact scale, one not
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    slots[5] = -1                                  # padding token: skipped
    gen = torch.Generator(device=DEV)
    gen.manual_seed(d)
    key = (torch.randn((T, Hkv, d), generator=gen, device=DEV) * 3).to(td)
    val = (torch.randn((T, Hkv, d), generator=gen, device=DEV) * 3).to(td)
    sk, sv = special_values(ks), special_values(vs)
    key.view(-1)[:len(sk)] = torch.from_numpy(sk).to(DEV).to(td)
    val.view(-1)[-len(sv):] = torch.from_numpy(sv).to(DEV).to(td)
    kc = torch.full((NB, Hkv, BS, d), wl.E4M3_NAN, dtype=torch.uint8, device=DEV)
    kc.view(-1)[::7] = 0x3C                        # bytes the call must leave alone
    vc = kc.clone()
    kc0, vc0 = wl.to_host(kc), wl.to_host(vc)
    pkv.reshape_and_cache_fp8(key, val, dev_i64(slots), kc, vc, ks, vs, validate=True)
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache_fp8(wl.to_host(key), wl.to_host(val), slots, kc0, vc0,
                                          ks, vs, dtype)
    assert wl.to_host(kc).tobytes() == ek.tobytes()
    assert wl.to_host(vc).tobytes() == ev.tobytes()
    codes = wl.to_host(kc)
    say(f"    {T - 1} tokens written bit-exact; codes 0x7E/0xFE (saturated) present: "
        f"{bool(((codes & 0x7F) == 0x7E).any())}")


def test_fp8_pool_accepts_float8_dtype(gpu_lib):
    """The binding takes pools as float8_e4m3fn tensors as well as uint8."""
    w = wl.custom([40, 3], 8, 2, 128, "bf16", **ODD)
    b = wl.make_batch(w, 12, DEV)
    ref_out = run_decode(b).clone()
    b8 = dict(b, key_cache=b["key_cache"].view(torch.float8_e4m3fn),
              value_cache=b["value_cache"].view(torch.float8_e4m3fn))
    out = run_decode(b8)
    assert torch.equal(bits(out), bits(ref_out))


# ------------------------------------------------------------------ decode --
@pytest.mark.parametrize("si", [0, 1])
@pytest.mark.parametrize("key,kw", [("opt13b", dict(num_seqs=8)),
                                    ("llama13b_conv", dict(num_seqs=24)),
                                    ("sampling_cow", dict(num_seqs=16, prompts=2)),
                                    ("long_gqa", dict(num_seqs=2))])
def test_fp8_reduced_workload_every_output(gpu_lib, key, kw, si):
    """Pool updates (copy_blocks of E4M3 blocks, reshape_and_cache_fp8) bit
    for bit, then every output of the decode."""
    w = fp8_variant(key, **kw)
    b = wl.make_batch(w, w.seeds()[si], DEV)
    full_step_and_check(b)


@pytest.mark.parametrize("key", ["opt13b_fp8", "long_gqa_fp8"])
def test_fp8_full_size_sampled(gpu_lib, key):
    """Full workload in the benchmark's launch configuration, oracle on a sample."""
    w = W[key]
    b = wl.make_batch(w, w.default_seed, DEV)
    full_step_and_check(b, seqs=sample_seqs(b["context_lens"]))


GROUPS = [(4, 4), (8, 2), (8, 1), (16, 2), (6, 2), (10, 2), (28, 4), (12, 1), (32, 2)]


@pytest.mark.parametrize("hq,hkv", GROUPS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_head_grouping_and_types(gpu_lib, dtype, d, hq, hkv):
    rng = np.random.default_rng(hq * 1000 + hkv * 10 + d + 1)
    lens = rng.integers(1, 300, size=4)
    w = wl.custom(lens, hq, hkv, d, dtype, max_len=320, partition_size=128, **ODD)
    b = wl.make_batch(w, int(rng.integers(1 << 30)), DEV)
    kc0, vc0 = clone_pools(b)
    out = run_decode(b)
    ref = oracle_decode_subset(b, kc0, vc0, list(range(4)))
    assert_close(out, ref, dtype, f"e4m3 {dtype} D={d} {hq}/{hkv}")


EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1023, 1024]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_edge_lengths(gpu_lib, dtype):
    w = wl.custom(EDGE_LENS, 8, 2, 128, dtype, max_len=1024, partition_size=512,
                  kv_dtype="e4m3", k_scale=0.0137, v_scale=2.0 ** -6)
    b = wl.make_batch(w, 98, DEV)
    kc0, vc0 = clone_pools(b)
    out = run_decode(b)
    ref = oracle_decode_subset(b, kc0, vc0, list(range(len(EDGE_LENS))))
    assert_close(out, ref, dtype, f"e4m3 edge lengths {dtype}")
    assert torch.count_nonzero(out[0]) == 0          # L = 0 gives zeros
    # L = 1: one weight of exactly 1, so the output is v_0 * v_scale rounded
    # once to the output format (a code times a power of two is exact)
    v0 = wl.to_host(b["value_cache"][int(b["block_tables"][1, 0]), :, 0, :])
    want = (oracle.e4m3_decode(v0).astype(np.float32) * np.float32(w.v_scale))
    want = torch.from_numpy(want).to(wl.torch_dtype(dtype))
    got = out[1].view(2, 4, 128)[:, 0].cpu()
    assert torch.equal(bits(got), bits(want))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (32, 2)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_sharp_softmax(gpu_lib, dtype, hq, hkv):
    """Queries scaled by 8 (exact): logits 8 times larger, so the running max
    jumps past the lazy rescale threshold of the matrix-core path often."""
    lens = [1, 17, 300, 1000, 2047]
    w = wl.custom(lens, hq, hkv, 128, dtype, max_len=2048, partition_size=512, **ODD)
    b = wl.make_batch(w, 9 + hq + hkv, DEV)
    b["query"].mul_(8)
    kc0, vc0 = clone_pools(b)
    out = run_decode(b)
    ref = oracle_decode_subset(b, kc0, vc0, list(range(len(lens))))
    assert_close(out, ref, dtype, f"e4m3 sharp softmax {dtype} {hq}/{hkv}")


@pytest.mark.parametrize("ps", [16, 48])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (16, 2), (32, 2)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_many_piece_merges(gpu_lib, dtype, hq, hkv, ps):
    """E4M3 pools on the matrix-core path with segments split up to 128 ways:
    the merges in a workgroup and in slices over the segment's ranges."""
    lens = [2048, 1500, 700, 33, 1]
    w = wl.custom(lens, hq, hkv, 128, dtype, max_len=2048, partition_size=ps, **ODD)
    b = wl.make_batch(w, 23 + hq + ps, DEV)
    kc0, vc0 = clone_pools(b)
    out = run_decode(b)
    ref = oracle_decode_subset(b, kc0, vc0, list(range(len(lens))))
    assert_close(out, ref, dtype, f"e4m3 many pieces {dtype} {hq}/{hkv} ps={ps}")


@pytest.mark.parametrize("ps", [0, 16, 128, 512, 4096])
def test_fp8_partition_sizes(gpu_lib, ps):
    w = fp8_variant("opt13b", num_seqs=6)
    b = wl.make_batch(w, 4243, DEV)
    kc0, vc0 = clone_pools(b)
    out = run_decode(b, partition_size=ps)
    ref = oracle_decode_subset(b, kc0, vc0, list(range(w.num_seqs)))
    assert_close(out, ref, w.dtype, f"e4m3 partition {ps}")


def test_fp8_many_short_sequences_and_empties(gpu_lib):
    rng = np.random.default_rng(18)
    lens = rng.integers(0, 40, size=300)
    lens[::7] = 0
    w = wl.custom(lens, 8, 8, 128, "f16", max_len=48, partition_size=0, **ODD)
    b = wl.make_batch(w, 5, DEV)
    kc0, vc0 = clone_pools(b)
    out = run_decode(b)
    ref = oracle_decode_subset(b, kc0, vc0, list(range(len(lens))))
    assert_close(out, ref, "f16", "e4m3 300 short sequences")


def test_fp8_matches_16bit_path_on_dequantized_pools(gpu_lib):
    """With unit scales, the E4M3 decode and the float16 decode over the same
    pools decoded to float16 (every E4M3 value is a float16) agree closely:
    the two kernels differ only in how the pool is read."""
    w = wl.custom([300, 17, 1024, 1], 8, 2, 128, "f16", max_len=1024, k_scale=1.0,
                  v_scale=1.0, kv_dtype="e4m3")
    b = wl.make_batch(w, 21, DEV)
    out8 = run_decode(b).clone()
    deq = lambda c: torch.from_numpy(oracle.e4m3_decode(wl.to_host(c))).to(torch.float16).to(DEV)
    w16 = dataclasses.replace(w, kv_dtype="", k_scale=1.0, v_scale=1.0)
    b16 = dict(b, workload=w16, key_cache=deq(b["key_cache"]), value_cache=deq(b["value_cache"]))
    out16 = run_decode(b16)
    # one float16 ulp of outputs below 8 at most: the two accumulate in
    # different orders before the single rounding of the output
    assert (out8.float() - out16.float()).abs().max().item() <= 4e-3


def test_fp8_scale_validation_raises(gpu_lib):
    w = wl.custom([4], 4, 4, 64, "f16", **ODD)
    b = wl.make_batch(w, 1, DEV)
    out = torch.empty_like(b["query"])
    for ks, vs in ((0.0, 1.0), (1.0, float("nan")), (-1.0, 1.0), (1.0, float("inf"))):
        with pytest.raises(pkv.PagedKVError):
            pkv.paged_attention_decode_fp8(out, b["query"], b["key_cache"], b["value_cache"],
                                           dev_i32(b["block_tables"]),
                                           dev_i32(b["context_lens"]), float(w.scale), ks, vs,
                                           w.num_kv_heads)


def test_fp8_workspace_reused_and_many_sequences(gpu_lib):
    """One workspace serves E4M3 and 16-bit calls of different shapes in
    turn; more than 2048 sequences run as several launches."""
    w1 = fp8_variant("opt13b", num_seqs=8)
    w2 = wl.custom(np.full(2100, 3), 4, 4, 64, "f16", max_len=16, partition_size=0, **ODD)
    ws = torch.zeros(max(pkv.workspace_bytes(8, 40, 40, 128, 128),
                         pkv.workspace_bytes(2100, 4, 4, 64, 1)), dtype=torch.uint8, device=DEV)
    for w, seed in ((w1, 1), (w2, 2), (w1, 3)):
        b = wl.make_batch(w, seed, DEV)
        kc0, vc0 = clone_pools(b)
        out = torch.empty_like(b["query"])
        pkv.paged_attention_decode_fp8(out, b["query"], b["key_cache"], b["value_cache"],
                                       dev_i32(b["block_tables"]), dev_i32(b["context_lens"]),
                                       float(w.scale), w.k_scale, w.v_scale, w.num_kv_heads,
                                       workspace=ws)
        torch.cuda.synchronize()
        seqs = list(range(w.num_seqs)) if w.num_seqs <= 64 else [0, 1, 2047, 2048, 2099]
        ref = oracle_decode_subset(b, kc0, vc0, seqs)
        assert_close(out[seqs], ref, w.dtype, f"e4m3 reuse {w.key} seed {seed}")
