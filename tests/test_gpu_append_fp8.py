"""Parity of paged_attention_decode_append_fp8 (the newest token encoded to
E4M3, cached and attended in one call) on an MI355X (marked gpu).

The fused call must leave the pools exactly as reshape_and_cache_fp8 of the
new rows would (every touched block compared bit for bit with the oracle's
encoding, every other block unchanged), produce the decode oracle's output
over the decoded, scaled codes within the 16-bit tolerances, and equal, bit
for bit, the separate calls reshape_and_cache_fp8 + paged_attention_decode_fp8.
"""

import dataclasses

import numpy as np
import pytest
import torch

from paged_kv_cache_311_amd import workloads as wl
from tests.gpu_helpers import DEV, bits, sample_seqs
from tests.test_gpu_append import append_and_check, append_inputs

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS


@pytest.mark.parametrize("key,kw", [("opt13b_fp8", dict(num_seqs=8)),
                                    ("long_gqa_fp8", dict(num_seqs=2))])
def test_append_fp8_reduced_every_output(gpu_lib, key, kw):
    w = dataclasses.replace(W[key], **kw)
    append_and_check(wl.make_batch(w, w.default_seed + 3, DEV), seed=3)


@pytest.mark.parametrize("key", ["opt13b_fp8", "long_gqa_fp8"])
def test_append_fp8_full_size_sampled(gpu_lib, key):
    """Full workload in the benchmark's launch configuration: the oracle on
    a sample of sequences, the separate calls on all of them."""
    w = W[key]
    b = wl.make_batch(w, w.default_seed, DEV)
    append_and_check(b, seqs=sample_seqs(b["context_lens"]))


# 1, 4 and 16 heads per kv head (the VALU and the matrix-core paths), both
# head sizes, both 16-bit query types, E4M3 pools
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (32, 2), (12, 1)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_append_fp8_groups_and_types(gpu_lib, dtype, d, hq, hkv):
    rng = np.random.default_rng(hq * 100 + hkv * 10 + d)
    lens = rng.integers(1, 300, size=4)
    w = wl.custom(lens, hq, hkv, d, dtype, max_len=320, partition_size=128, kv_dtype="e4m3",
                  k_scale=wl.FP8_K_SCALE, v_scale=wl.FP8_V_SCALE)
    append_and_check(wl.make_batch(w, int(rng.integers(1 << 30)), DEV), seed=hq + d)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_append_fp8_special_values(gpu_lib, dtype, monkeypatch):
    """New rows holding the encoder's hard cases: values exactly halfway
    between two codes (ties to the even code), values beyond the largest
    code and infinities (saturate to +-448), subnormal codes and signed
    zeros; L = 1 sequences see nothing but the new token."""
    lens = [1, 1, 17, 16, 33, 300]
    # power-of-two scales small enough that even saturated values attend to
    # outputs below 1, where the 16-bit output rounding stays inside the bound
    w = wl.custom(lens, 4, 2, 128, dtype, max_len=320, partition_size=0, kv_dtype="e4m3",
                  k_scale=2.0 ** -8, v_scale=2.0 ** -9)
    b = wl.make_batch(w, 77, DEV)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    # values that are exact in both 16-bit formats: code midpoints times the scale
    special = torch.tensor([1.0625, 1.1875, 0.0048828125, -0.0048828125, 0.0, -0.0, 480.0,
                            -1000.0, float("inf"), float("-inf"), 2.0 ** -10, 3.0 * 2.0 ** -10,
                            13.0, 15.0, -0.5, 300.0], dtype=torch.float32)
    real = append_inputs

    def with_special(bb, seed):
        nk, nv, live, slots = real(bb, seed)
        nk = nk.clone()
        nv = nv.clone()
        flat_k = nk.view(-1)
        flat_v = nv.view(-1)
        n = flat_k.numel()
        idx = torch.arange(n, device=DEV) % len(special)
        pick = torch.rand(n, generator=torch.Generator(device=DEV).manual_seed(seed),
                          device=DEV) < 0.25
        flat_k[pick] = (special.to(DEV)[idx] * w.k_scale).to(tdt)[pick]
        flat_v[pick] = (special.to(DEV)[idx] * w.v_scale).to(tdt)[pick]
        return nk, nv, live, slots

    import tests.test_gpu_append as ta
    monkeypatch.setattr(ta, "append_inputs", with_special)
    out = append_and_check(b, seed=5)
    assert torch.isfinite(out.float()).all()
