"""Benchmark of the paged decode path on one MI355X.

One step = one pass of the whole path over one seeded synthetic batch:
copy_blocks (workloads with copy-on-write pairs), reshape_and_cache of the
step's new tokens (one per sequence -- the token each sequence appends in
this decode step -- or the private tokens of the sampling workload), then
paged_attention_decode over every sequence.  Where every sequence appends
exactly its newest token into a 16/32-bit pool, the caching and the
attention are one call, paged_attention_decode_append (--no-fuse keeps
them apart).  Inputs are resident in HBM
before the timed region; K steps are timed between two synchronizations.

Each workload is measured in a child process of its own (the headline one,
with the CPU baseline and the translation legs, first), as a serving process
allocates its pools once at start-up; this process touches no GPU and only
spawns and collects.  --same-process measures them all in one process (then
later workloads run on pools allocated after earlier ones were freed, which
reads 1-4% slower), and so does a run with empty --also and --prefill lists,
as under a profiler.

Prints ONE JSON line.  `value` is whole-step KV throughput in GB/s: the
key/value bytes the attention must read (sum of context lengths x 2 x
kv_heads x head_size x element bytes) divided by the step time.
`roofline` covers the dominant kernel call, paged_attention_decode (or its
appending variant), timed with events on the launch stream: over the timed
region itself when a step is that call alone, else over a timed region of
the call alone repeated on the step's final pools; `cpu_baseline` times the float64 CPU
oracle on a bounded sample of the same batch (one thread, then one process
per core of the host share, at most 16);
`translation` times the same decode call on the same batch laid out with
every sequence's blocks physically consecutive (identity block tables) and
in a virtually contiguous pool (HIP virtual-memory ranges backed on
demand), against the random placement.  `prefill` times the prefill path (the
chunk's reshape_and_cache, then paged_attention_prefill) on its own
workloads, in TFLOP/s of causal attention against the MFMA peak.

    python bench.py [--steps K] [--warmup W] [--workload opt13b]
                    [--also long_gqa_p512,long_gqa,llama13b_conv,sampling_cow,beam,
                            sampling_cow_shuffled,beam_shuffled,opt13b_fp8,long_gqa_fp8,
                            gqa8_long,gqa16_long]
                    [--no-cpu-baseline]
                    [--no-translation]
"""

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, AMD's published figure
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix peak, AMD's published figure
METRIC = "paged decode attention KV GB/s (% of HBM peak) + decode tokens/s, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_cache_311_amd", "csrc", "paged_attention.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="opt13b")
    ap.add_argument("--also",
                    default="long_gqa_p512,long_gqa,llama13b_conv,sampling_cow,beam,"
                            "sampling_cow_shuffled,beam_shuffled,opt13b_fp8,long_gqa_fp8,"
                            "gqa8_long,gqa16_long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill", default="prefill_chunk,prefill_gqa",
                    help="prefill workloads to time ('' for none)")
    ap.add_argument("--no-translation", action="store_true",
                    help="skip the random vs contiguous placement comparison")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-fuse", action="store_true",
                    help="cache new tokens with reshape_and_cache instead of the decode call")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="cap on tokens per piece (default: the workload's, 0 = none)")
    ap.add_argument("--same-process", action="store_true",
                    help="measure every workload in this one process (later ones then run "
                         "on pools allocated after earlier ones were freed)")
    ap.add_argument("--child", default="",
                    help=argparse.SUPPRESS)  # internal: measure one workload, print its result
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (steps "
                         "times), to scale HBM byte counters; prints one JSON line")
    return ap.parse_args()


def copy_calibration(mib, steps):
    """A plain copy of known size: reads and writes exactly mib MiB per launch."""
    import torch
    n = mib << 20
    x = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        y.copy_(x)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                      "GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def kv_bytes(w, lens):
    return (int(np.asarray(lens, np.int64).sum()) * 2 * w.num_kv_heads * w.head_size
            * w.kv_elem_bytes)


def kv_unique_bytes(w, tables, lens):
    """K/V bytes of the distinct cached tokens: a physical block that several
    sequences map (a prompt shared by samples or beams) counts once, with
    the most tokens any of them uses in it."""
    used = {}
    for s, L in enumerate(np.asarray(lens, np.int64)):
        for n in range(-(-int(L) // 16)):
            b = int(tables[s, n])
            used[b] = max(used.get(b, 0), min(16, int(L) - 16 * n))
    return sum(used.values()) * 2 * w.num_kv_heads * w.head_size * w.kv_elem_bytes


def decode_algorithmic_bytes(w, lens):
    """Bytes the decode must move: K/V of every context token (in the pool's
    format: 1 byte per element for E4M3 pools), q in, out, the block-table
    entries it follows and the lengths."""
    eb = 4 if w.dtype == "f32" else 2
    lens = np.asarray(lens, np.int64)
    qo = 2 * w.num_seqs * w.num_heads * w.head_size * eb
    tables = 4 * int((-(-lens // 16)).sum()) + 4 * w.num_seqs
    return kv_bytes(w, lens) + qo + tables


class Step:
    """Device-resident batch and the calls of one step (no allocation inside)."""

    def __init__(self, w, seed, ps, fuse=True, shared=False):
        import torch
        import paged_kv_cache_311_amd as pkv
        from paged_kv_cache_311_amd import workloads as wl
        self.pkv, self.torch, self.w = pkv, torch, w
        dev = "cuda:0"
        b = wl.make_batch(w, seed, dev)
        self.b = b
        lens = b["context_lens"]
        self.lens = lens
        self.bt = torch.from_numpy(b["block_tables"]).to(dev)
        self.cl = torch.from_numpy(lens).to(dev)
        self.out = torch.empty_like(b["query"])
        self.ps = w.partition_size if ps is None else ps
        need = pkv.workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size,
                                   b["block_tables"].shape[1], self.ps)
        self.ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        if "slot_mapping" in b:
            slots = b["slot_mapping"]
            self.key, self.value = b["key"], b["value"]
        else:  # plain decode workload: append token L-1 of every sequence
            bt = b["block_tables"]
            pos = lens.astype(np.int64) - 1
            slots = bt[np.arange(len(lens)), pos // 16].astype(np.int64) * 16 + pos % 16
            g = torch.Generator(device=dev)
            g.manual_seed(seed + 1)
            shape = (w.num_seqs, w.num_kv_heads, w.head_size)
            self.key = torch.randn(shape, generator=g, device=dev).to(b["query"].dtype)
            self.value = torch.randn(shape, generator=g, device=dev).to(b["query"].dtype)
        self.slots = torch.from_numpy(np.asarray(slots, np.int64)).to(dev)
        # the runtime's reference counts above one, as the decode call's
        # cache-policy flags (workloads whose sequences share blocks)
        self.flags = (torch.from_numpy(b["block_shared"]).to(dev)
                      if "block_shared" in b else None)
        pairs = b.get("cow_pairs")
        self.pairs = (torch.from_numpy(pairs).to(dev)
                      if pairs is not None and len(pairs) else None)
        self.new_tokens = len(slots)
        # one new token per sequence, token s of sequence s, at position L-1:
        # the decode call caches it itself
        one_each = ("slot_mapping" not in b
                    or np.array_equal(b.get("token_seq", []), np.arange(w.num_seqs)))
        self.fused = bool(fuse and one_each and (lens >= 1).all())
        # the shared-prefix call: groups of sequences that begin with the same
        # blocks (samples, beams of one prompt), found from the tables; it
        # does not append, so the step caches its tokens first
        self.shared = shared
        if shared:
            self.fused = False
            order, gs, pb = pkv.shared_prefix_groups(b["block_tables"], lens)
            self.order = torch.from_numpy(order).to(dev)
            self.group_start = torch.from_numpy(gs).to(dev)
            self.prefix_blocks = torch.from_numpy(pb).to(dev)
            self.shared_groups = int((pb > 0).sum())
            self.sws = torch.zeros(max(pkv.shared_prefix_workspace_bytes(
                w.num_seqs, w.num_heads, w.head_size, b["block_tables"].shape[1]), 1),
                dtype=torch.uint8, device=dev)

    def updates(self):
        b, w = self.b, self.w
        if self.pairs is not None:
            self.pkv.copy_blocks(b["key_cache"], b["value_cache"], self.pairs)
        if self.fused:
            return
        if w.fp8:
            self.pkv.reshape_and_cache_fp8(self.key, self.value, self.slots, b["key_cache"],
                                           b["value_cache"], w.k_scale, w.v_scale)
        else:
            self.pkv.reshape_and_cache(self.key, self.value, self.slots, b["key_cache"],
                                       b["value_cache"])

    def decode_into(self, out, kc, vc, bt, flags=None):
        b, w = self.b, self.w
        if w.fp8:
            self.pkv.paged_attention_decode_fp8(out, b["query"], kc, vc, bt, self.cl,
                                                float(w.scale), w.k_scale, w.v_scale,
                                                w.num_kv_heads, partition_size=self.ps,
                                                workspace=self.ws, block_shared=flags)
        else:
            self.pkv.paged_attention_decode(out, b["query"], kc, vc, bt, self.cl,
                                            float(w.scale), w.num_kv_heads,
                                            partition_size=self.ps, workspace=self.ws,
                                            block_shared=flags)

    def decode(self):
        b, w = self.b, self.w
        if self.shared:
            self.pkv.paged_attention_decode_shared_prefix(
                self.out, b["query"], b["key_cache"], b["value_cache"], self.bt, self.cl,
                self.order, self.group_start, self.prefix_blocks, float(w.scale),
                w.num_kv_heads, workspace=self.sws)
        elif self.fused and w.fp8:
            self.pkv.paged_attention_decode_append_fp8(
                self.out, b["query"], b["key_cache"], b["value_cache"], self.bt, self.cl,
                self.key, self.value, float(w.scale), w.k_scale, w.v_scale, w.num_kv_heads,
                partition_size=self.ps, workspace=self.ws, block_shared=self.flags)
        elif self.fused:
            self.pkv.paged_attention_decode_append(
                self.out, b["query"], b["key_cache"], b["value_cache"], self.bt, self.cl,
                self.key, self.value, float(w.scale), w.num_kv_heads, partition_size=self.ps,
                workspace=self.ws, block_shared=self.flags)
        else:
            self.decode_into(self.out, b["key_cache"], b["value_cache"], self.bt, self.flags)

    def only_the_call(self):
        """True when a step issues nothing but the decode call."""
        return self.pairs is None and getattr(self, "fused", False)

    def run(self, steps, warmup):
        """Times `steps` steps between two events and two synchronizations
        (nothing else recorded in between: an event per call would add a
        few microseconds to every step), then the same steps again with an
        event pair around each call, for the call's own duration, and, when
        a step is more than the call, `steps` calls of the call alone
        between two events (its average duration without per-call events)."""
        torch = self.torch
        for _ in range(warmup):
            self.updates()
            self.decode()
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        t_start.record()
        for _ in range(steps):
            self.updates()
            self.decode()
        t_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = t_start.elapsed_time(t_end) / steps
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            self.updates()
            ev[i][0].record()
            self.decode()
            ev[i][1].record()
        torch.cuda.synchronize()
        dec = np.asarray([a.elapsed_time(c) for a, c in ev])
        self.call_only_ms = None
        if not self.only_the_call():
            # the state after the updates: repeating the call alone recomputes
            # the same outputs from the same pools
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            self.decode()
            torch.cuda.synchronize()
            c0.record()
            for _ in range(steps):
                self.decode()
            c1.record()
            torch.cuda.synchronize()
            self.call_only_ms = c0.elapsed_time(c1) / steps
        return step_ms, dec, wall


def prefill_flops(w, md):
    """Causal attention flops of a prefill step: per new token and query
    head, 2·D for each visible key in QK and 2·D in PV."""
    qsl = np.asarray(md["query_start_loc"], np.int64)
    lens = np.asarray(md["context_lens"], np.int64)
    visible = 0
    for s in range(len(lens)):
        n, L = int(qsl[s + 1] - qsl[s]), int(lens[s])
        visible += n * (L - n) + n * (n + 1) // 2
    return 4 * w.head_size * w.num_heads * visible


class PrefillStep:
    """A prefill batch resident on the GPU: the chunk's cache writes, then
    the attention (no allocation inside)."""

    def __init__(self, w, seed):
        import torch
        import paged_kv_cache_311_amd as pkv
        from paged_kv_cache_311_amd import workloads as wl
        self.pkv, self.torch, self.w = pkv, torch, w
        dev = "cuda:0"
        b = wl.make_batch(w, seed, dev)
        self.b = b
        self.bt = torch.from_numpy(b["block_tables"]).to(dev)
        self.cl = torch.from_numpy(b["context_lens"]).to(dev)
        self.qsl = torch.from_numpy(b["query_start_loc"]).to(dev)
        self.slots = torch.from_numpy(b["slot_mapping"]).to(dev)
        self.out = torch.empty_like(b["query"])

    def updates(self):
        b = self.b
        self.pkv.reshape_and_cache(b["key"], b["value"], self.slots, b["key_cache"],
                                   b["value_cache"])

    def decode(self):
        b, w = self.b, self.w
        self.pkv.paged_attention_prefill(self.out, b["query"], b["key_cache"], b["value_cache"],
                                         self.bt, self.cl, self.qsl, float(w.scale),
                                         w.num_kv_heads, w.max_query_len)

    run = Step.run

    def only_the_call(self):
        return False


def measure_prefill(w, seed, steps, warmup):
    st = PrefillStep(w, seed)
    step_ms, call_ms, wall = st.run(steps, warmup)
    fl = prefill_flops(w, st.b)
    call_avg = st.call_only_ms  # the prefill call alone, between two events
    qsl = st.b["query_start_loc"]
    return {
        "workload": w.key, "seed": seed, "seqs": w.num_seqs, "heads": w.num_heads,
        "kv_heads": w.num_kv_heads, "head_size": w.head_size, "dtype": w.dtype,
        "new_tokens": int(qsl[-1]), "context_tokens": int(st.b["context_lens"].sum()),
        "flops_per_step": fl, "ms_per_step": step_ms,
        "prefill_call_ms_avg": call_avg, "prefill_call_ms_events_avg": float(call_ms.mean()),
        "prefill_call_ms_min": float(call_ms.min()),
        "step_TFLOPs": fl / (step_ms * 1e-3) / 1e12,
        "prefill_TFLOPs": fl / (call_avg * 1e-3) / 1e12,
        "new_tokens_per_s": int(qsl[-1]) / (step_ms * 1e-3),
        "roofline": {"bound": "mfma", "achieved": round(fl / (call_avg * 1e-3) / 1e12, 2),
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fl / (call_avg * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)},
        "host_wall_s": wall,
    }


def measure(w, seed, steps, warmup, ps, fuse=True, shared=None):
    st = Step(w, seed, ps, fuse, shared=bool(shared))
    step_ms, dec_ms, wall = st.run(steps, warmup)
    kvb = kv_bytes(w, st.lens)
    algo = decode_algorithmic_bytes(w, st.lens)
    if st.fused:  # the call also writes each sequence's new key and value rows
        algo += 2 * w.num_seqs * w.num_kv_heads * w.head_size * w.kv_elem_bytes
    # the call's average duration: over the timed region itself when a step
    # is nothing but the call, else from a timed region of the call alone
    dec_avg = step_ms if st.only_the_call() else st.call_only_ms
    r = {
        "workload": w.key, "seed": seed, "seqs": w.num_seqs,
        "heads": w.num_heads, "kv_heads": w.num_kv_heads, "head_size": w.head_size,
        "dtype": w.dtype, "kv_dtype": w.kv_dtype or w.dtype, "partition_size": st.ps,
        "kv_tokens": int(st.lens.astype(np.int64).sum()), "kv_bytes_per_step": kvb,
        "new_tokens_per_step": st.new_tokens,
        "append": "fused into the decode call" if st.fused else "reshape_and_cache",
        "cow_pairs_per_step": 0 if st.pairs is None else int(st.pairs.shape[0]),
        "ms_per_step": step_ms, "kv_GBps": kvb / (step_ms * 1e-3) / 1e9,
        "decode_tokens_per_s": w.num_seqs / (step_ms * 1e-3),
        "decode_call_ms_avg": dec_avg,
        "decode_call_timing": ("timed region (a step is the call alone)" if st.only_the_call()
                               else "timed region of the call alone, repeated on the "
                                    "step's final pools"),
        "decode_call_ms_events_avg": float(dec_ms.mean()),
        "decode_call_ms_min": float(dec_ms.min()), "decode_call_ms_max": float(dec_ms.max()),
        "decode_algorithmic_bytes": algo,
        "decode_GBps": algo / (dec_avg * 1e-3) / 1e9,
        "host_wall_s": wall,
    }
    r["pct_of_hbm_peak"] = 100.0 * r["kv_GBps"] / HBM_PEAK_GBPS
    r["decode_pct_of_hbm_peak"] = 100.0 * r["decode_GBps"] / HBM_PEAK_GBPS
    uniq = kv_unique_bytes(w, st.b["block_tables"], st.lens)
    if uniq != kvb:  # blocks shared between sequences: logical and unique bytes
        r["kv_unique_bytes_per_step"] = uniq
        r["kv_shared_fraction"] = 1.0 - uniq / kvb
        r["kv_unique_GBps"] = uniq / (step_ms * 1e-3) / 1e9
        r["decode_unique_GBps"] = (algo - kvb + uniq) / (dec_avg * 1e-3) / 1e9
        if shared is None and not w.fp8:
            r["shared_prefix"] = measure_shared(w, seed, steps, warmup, ps, st)
    return r, st


def measure_shared(w, seed, steps, warmup, ps, plain):
    """The same steps with paged_attention_decode_shared_prefix (blocks a
    group of sequences shares read once for the group), beside the plain
    call's numbers; outputs compared with the plain call's on the same
    pools."""
    torch = plain.torch
    r, st = measure(w, seed, steps, warmup, ps, fuse=False, shared=True)
    # same pools as `plain` after its steps: recompute both on st's pools
    plain_out = torch.empty_like(st.out)
    st.decode_into(plain_out, st.b["key_cache"], st.b["value_cache"], st.bt, st.flags)
    st.decode()
    torch.cuda.synchronize()
    diff = (plain_out.float() - st.out.float()).abs().max().item()
    uniq = kv_unique_bytes(w, st.b["block_tables"], st.lens)
    out = {
        "call": "paged_attention_decode_shared_prefix",
        "groups_sharing": st.shared_groups,
        "ms_per_step": r["ms_per_step"],
        "decode_call_ms_avg": r["decode_call_ms_avg"],
        "decode_tokens_per_s": r["decode_tokens_per_s"],
        "decode_logical_GBps": r["decode_GBps"],
        "decode_unique_GBps": (r["decode_algorithmic_bytes"] - r["kv_bytes_per_step"] + uniq)
                              / (r["decode_call_ms_avg"] * 1e-3) / 1e9,
        "decode_unique_pct_of_hbm_peak": 100.0 * (r["decode_algorithmic_bytes"]
                                                  - r["kv_bytes_per_step"] + uniq)
                                         / (r["decode_call_ms_avg"] * 1e-3) / 1e9
                                         / HBM_PEAK_GBPS,
        "max_abs_diff_vs_plain_call": diff,
    }
    del st
    torch.cuda.empty_cache()
    return out


def contiguous_layout(st):
    """The same batch with every sequence's blocks made physically
    consecutive, in sequence order (identity block tables): the pool is
    permuted and the tables renumbered, so the attention result is the same.
    None if blocks are shared between sequences."""
    torch, b = st.torch, st.b
    bt, lens = b["block_tables"], st.lens
    order = []
    for s in range(len(lens)):
        order.extend(int(x) for x in bt[s, :-(-int(lens[s]) // 16)])
    if len(set(order)) != len(order):
        return None
    nb = b["key_cache"].shape[0]
    used = set(order)
    old_of_new = np.asarray(order + [x for x in range(nb) if x not in used], np.int64)
    new_of_old = np.empty(nb, np.int64)
    new_of_old[old_of_new] = np.arange(nb)
    tables = np.where(bt >= 0, new_of_old[np.maximum(bt, 0)], -1).astype(np.int32)
    idx = torch.from_numpy(old_of_new).to("cuda:0")
    return (b["key_cache"].index_select(0, idx), b["value_cache"].index_select(0, idx),
            torch.from_numpy(tables).to("cuda:0"))


def virtual_layout(st):
    """The same batch in a virtually contiguous pool (pkv_vpool): sequence s
    at virtual blocks s*W .. s*W + n_s - 1, physical memory mapped in
    granules behind them only.  Returns (pool, tables) or None if blocks are
    shared between sequences or the device refuses virtual-memory mapping."""
    torch, b, w, pkv = st.torch, st.b, st.w, st.pkv
    bt, lens = b["block_tables"], st.lens
    S, W = bt.shape
    need = [-(-int(L) // 16) for L in lens]
    src = [int(x) for s in range(S) for x in bt[s, :need[s]]]
    if len(set(src)) != len(src):
        return None
    try:
        vp = pkv.VirtualPool(S * W, w.num_kv_heads, w.head_size, w.kv_dtype or w.dtype)
    except pkv.PagedKVError:
        return None
    vt = np.full_like(bt, -1)
    for s in range(S):
        if need[s]:
            vp.map(s * W, need[s])
            vt[s, :need[s]] = s * W + np.arange(need[s])
    # every block a launch reads must be backed (an unmapped read faults)
    assert all(vp.covers(s * W, need[s]) for s in range(S) if need[s])
    dst = [int(x) for s in range(S) for x in vt[s, :need[s]]]
    si = torch.tensor(src, dtype=torch.int64, device="cuda:0")
    di = torch.tensor(dst, dtype=torch.int64, device="cuda:0")
    for pool, from_pool in ((vp.key_cache, b["key_cache"]), (vp.value_cache, b["value_cache"])):
        pool[di] = from_pool[si].view(pool.dtype)
    torch.cuda.synchronize()
    return vp, torch.from_numpy(vt).to("cuda:0")


def translation_overhead(st, steps):
    """Decode-call time with the batch's random block placement against the
    same batch laid out contiguously (same kernel, same values, identity
    tables) and in a virtually contiguous pool, the three timed in turn."""
    lay = contiguous_layout(st)
    if lay is None:
        return None
    torch, b, w = st.torch, st.b, st.w
    kc2, vc2, bt2 = lay
    out2 = torch.empty_like(st.out)
    vlay = virtual_layout(st)
    out3 = torch.empty_like(st.out)

    def call(kc, vc, bt, out):
        st.decode_into(out, kc, vc, bt)

    args = [(b["key_cache"], b["value_cache"], st.bt, st.out), (kc2, vc2, bt2, out2)]
    if vlay is not None:
        args.append((vlay[0].key_cache, vlay[0].value_cache, vlay[1], out3))
    for _ in range(3):
        for a in args:
            call(*a)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)] for _ in args]
    torch.cuda.synchronize()
    for i in range(steps):
        for j, a in enumerate(args):
            ev[j][i][0].record()
            call(*a)
            ev[j][i][1].record()
    torch.cuda.synchronize()
    us = [1000.0 * float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev[j]]))
          for j in range(len(args))]
    r = {"workload": w.key,
         "random_placement_call_us": round(us[0], 2),
         "contiguous_placement_call_us": round(us[1], 2),
         "translation_overhead_pct": round(100.0 * (us[0] / us[1] - 1.0), 2),
         "outputs_bitwise_equal": bool(torch.equal(st.out, out2)),
         "layout": "each sequence's blocks physically consecutive in sequence order "
                   "(identity block tables); same kernel, values and tables' content"}
    if vlay is not None:
        vp = vlay[0]
        r.update({
            "virtual_contiguous_call_us": round(us[2], 2),
            "translation_overhead_vs_virtual_pct": round(100.0 * (us[0] / us[2] - 1.0), 2),
            "virtual_outputs_bitwise_equal": bool(torch.equal(st.out, out3)),
            "virtual_layout": (f"each sequence's blocks virtually consecutive in a reserved "
                               f"range, backed by {vp.granularity >> 20}-MiB physical granules "
                               f"mapped on demand ({vp.mapped_bytes / 2**20:.0f} MiB mapped "
                               f"for both tensors)")})
        args.pop()
        vp.close()
    del kc2, vc2
    return r


def traffic_for_current_kernel(workload):
    """HBM bytes per decode call from committed PMC counters, if the kernel
    source is unchanged since they were taken (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(KERNEL_SOURCE, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    entry = t.get("workloads", {}).get(workload)
    if not entry or t.get("kernel_source_sha256") != h:
        return None
    return entry.get("hbm_bytes_per_call")


def _oracle_pass(q, kc, vc, tables, lens, w_args, seqs, budget_s):
    """The float64 oracle over `seqs` of the sample, one at a time and round
    and round, until `budget_s` seconds are spent: (decodes, tokens, s)."""
    import oracle
    scale, hkv, dtype, fp8 = w_args
    done, tokens, t_used = 0, 0, 0.0
    t0 = time.perf_counter()
    while t_used < budget_s and seqs:
        for s in seqs:
            oracle.decode_attention(q, kc, vc, tables, lens, scale, hkv, dtype, seqs=[s], **fp8)
            done += 1
            tokens += int(lens[s])
            t_used = time.perf_counter() - t0
            if t_used >= budget_s:
                break
    return done, tokens, t_used


def _oracle_worker(job):
    """One process of the all-cores leg: the sample memory-mapped from the
    files the parent wrote, sequences i, i + n, ... of it, one thread."""
    from threadpoolctl import threadpool_limits
    folder, i, n, w_args, budget_s = job
    a = {k: np.load(os.path.join(folder, k + ".npy"), mmap_mode="r")
         for k in ("q", "kc", "vc", "tables", "lens")}
    seqs = list(range(i, len(a["lens"]), n))
    with threadpool_limits(limits=1):
        return _oracle_pass(a["q"], a["kc"], a["vc"], a["tables"], np.asarray(a["lens"]),
                            w_args, seqs, budget_s)


def cpu_baseline(st, budget_s):
    """The float64 oracle on the host, on the first sequences of the batch:
    one thread, then one process per core of this process's CPU share (at
    most 16, the host share of one GPU), each on its own sequences."""
    import multiprocessing
    import shutil
    import tempfile
    from threadpoolctl import threadpool_limits
    from paged_kv_cache_311_amd import workloads as wl
    w, b = st.w, st.b
    bt, lens = b["block_tables"], b["context_lens"]
    n_max = min(w.num_seqs, 64)
    ids = sorted({int(x) for s in range(n_max) for x in bt[s, :-(-int(lens[s]) // 16)]})
    remap = {x: i for i, x in enumerate(ids)}
    idx = st.torch.tensor(ids, dtype=st.torch.int64, device=b["key_cache"].device)
    kc = wl.to_host(b["key_cache"].index_select(0, idx))
    vc = wl.to_host(b["value_cache"].index_select(0, idx))
    tables = np.full_like(bt[:n_max], -1)
    for s in range(n_max):
        n = -(-int(lens[s]) // 16)
        tables[s, :n] = [remap[int(x)] for x in bt[s, :n]]
    q = wl.to_host(b["query"])[:n_max]
    sample_lens = np.asarray(lens[:n_max])
    fp8 = (dict(kv_dtype="e4m3", k_scale=w.k_scale, v_scale=w.v_scale) if w.fp8 else {})
    w_args = (w.scale, w.num_kv_heads, w.dtype, fp8)
    per_token = 2 * w.num_kv_heads * w.head_size * w.kv_elem_bytes

    with threadpool_limits(limits=1):
        done1, tok1, t1 = _oracle_pass(q, kc, vc, tables, sample_lens, w_args,
                                       list(range(n_max)), budget_s)
    single = {"value": tok1 * per_token / t1 / 1e9, "unit": "GB/s", "cores": 1,
              "decode_tokens_per_s": done1 / t1, "seconds": t1,
              "sample": f"{done1} sequence-decodes ({tok1} KV tokens) in {t1:.1f} s"}

    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    shm = "/dev/shm" if os.path.isdir("/dev/shm") else None
    folder = tempfile.mkdtemp(prefix="pkv_oracle_", dir=shm)
    try:
        for k, v in (("q", q), ("kc", kc), ("vc", vc), ("tables", tables),
                     ("lens", sample_lens)):
            np.save(os.path.join(folder, k + ".npy"), v)
        del kc, vc
        jobs = [(folder, i, cores, w_args, budget_s) for i in range(cores)]
        # fresh interpreters (this process has initialised the GPU)
        with multiprocessing.get_context("spawn").Pool(cores) as pool:
            res = pool.map(_oracle_worker, jobs)
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    rate = sum(tok * per_token / t for _, tok, t in res if t > 0)
    decodes = sum(d / t for d, _, t in res if t > 0)
    done_all = sum(d for d, _, _ in res)
    tok_all = sum(tok for _, tok, _ in res)
    return {
        "value": rate / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": (f"float64 numpy oracle, {cores} processes of one thread each over the "
                   f"first {n_max} of {w.num_seqs} sequences of the {w.key} batch (process i "
                   f"takes sequences i, i + {cores}, ...): {done_all} sequence-decodes "
                   f"({tok_all} KV tokens) in about {budget_s:.0f} s each; rate = sum of the "
                   f"processes' rates"),
        "decode_tokens_per_s": decodes, "seconds": max(t for _, _, t in res),
        "single_thread": single, "cpu_model": _cpu_model(),
        "cpus_visible": len(os.sched_getaffinity(0)),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_child(a, job):
    """Measure in a child process of its own and return its JSON result.

    Called only from a parent that has not initialised the GPU (it spawns,
    the children measure)."""
    cmd = [sys.executable, os.path.abspath(__file__), "--child", job, "--workload", a.workload,
           "--steps", str(a.steps), "--warmup", str(a.warmup),
           "--cpu-seconds", str(a.cpu_seconds)]
    if a.partition_size is not None:
        cmd += ["--partition-size", str(a.partition_size)]
    for flag in ("no_fuse", "no_cpu_baseline", "no_translation"):
        if getattr(a, flag):
            cmd.append("--" + flag.replace("_", "-"))
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=900)
    if r.returncode != 0:
        print(f"bench.py: measuring {job} failed (status {r.returncode})", file=sys.stderr)
        sys.exit(1)
    return json.loads([l for l in r.stdout.splitlines() if l.startswith("{")][-1])


def child(a):
    """One measurement in this process: the headline workload with the CPU
    baseline and the translation legs ("main"), or one other workload."""
    import torch
    import paged_kv_cache_311_amd as pkv
    from paged_kv_cache_311_amd import workloads as wl
    pkv.load_library()
    if a.child == "main":
        w = wl.WORKLOADS[a.workload]
        print(f"# measuring {w.key}", file=sys.stderr, flush=True)
        r, st = measure(w, w.default_seed, a.steps, a.warmup, a.partition_size, not a.no_fuse)
        cpu = None if a.no_cpu_baseline else cpu_baseline(st, a.cpu_seconds)
        trans = None if a.no_translation else translation_overhead(st, a.steps)
        out = {"main": r, "cpu": cpu, "trans": trans}
    else:
        w = wl.WORKLOADS[a.child]
        print(f"# measuring {w.key}", file=sys.stderr, flush=True)
        if w.step == "prefill":
            out = measure_prefill(w, w.default_seed, a.steps, a.warmup)
        else:
            out, st = measure(w, w.default_seed, a.steps, a.warmup, a.partition_size,
                              not a.no_fuse)
    torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(this path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    import torch
    if a.child:
        child(a)
        return
    if a.copy_calibration_mib:
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(2)
        copy_calibration(a.copy_calibration_mib, a.steps)
        return
    from paged_kv_cache_311_amd import workloads as wl
    w = wl.WORKLOADS[a.workload]
    also = [k for k in a.also.split(",") if k and k != w.key]
    pre = [k for k in a.prefill.split(",") if k]
    if also or pre:
        if not a.same_process:
            # One process per workload, as a serving process allocates its
            # pools once at start-up: measured in one process after others
            # were freed, later workloads run 1-4% slower (long_gqa 336 ->
            # 350 us per call).  This process touches no GPU (counting
            # devices does not initialise it) and only spawns.
            if torch.cuda.device_count() < 1:
                print("bench.py needs a GPU", file=sys.stderr)
                sys.exit(2)
            m = run_child(a, "main")
            main_r, cpu, trans = m["main"], m["cpu"], m["trans"]
            others = {k: run_child(a, k) for k in also}
            prefill = {k: run_child(a, k) for k in pre}
            emit(a, w, main_r, cpu, trans, others, prefill)
            return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import paged_kv_cache_311_amd as pkv
    pkv.load_library()

    print(f"# measuring {w.key}", file=sys.stderr, flush=True)
    main_r, st = measure(w, w.default_seed, a.steps, a.warmup, a.partition_size,
                         not a.no_fuse)
    cpu = None if a.no_cpu_baseline else cpu_baseline(st, a.cpu_seconds)
    trans = None if a.no_translation else translation_overhead(st, a.steps)
    del st
    torch.cuda.empty_cache()

    others = {}
    for key in also:
        print(f"# measuring {key}", file=sys.stderr, flush=True)
        ow = wl.WORKLOADS[key]
        r, st = measure(ow, ow.default_seed, a.steps, a.warmup, a.partition_size,
                        not a.no_fuse)
        others[key] = r
        del st
        torch.cuda.empty_cache()

    prefill = {}
    for key in pre:
        print(f"# measuring {key}", file=sys.stderr, flush=True)
        pw = wl.WORKLOADS[key]
        prefill[key] = measure_prefill(pw, pw.default_seed, a.steps, a.warmup)
        torch.cuda.empty_cache()
    emit(a, w, main_r, cpu, trans, others, prefill)


def emit(a, w, main_r, cpu, trans, others, prefill):
    """Print the one JSON line."""
    dec_ms = main_r["decode_call_ms_avg"]
    achieved = main_r["decode_GBps"]
    line = {
        "metric": METRIC,
        "value": round(main_r["kv_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(main_r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) K/V, random block placement, NaN-filled free slots)",
        "config": {
            "workload": (f"{w.key}: {w.num_seqs} seqs, {w.num_heads} heads / "
                         f"{w.num_kv_heads} kv heads x {w.head_size}, {w.dtype}, "
                         f"16-token blocks, lengths {w.lengths}, pool {w.pool}"),
            "seqs": w.num_seqs, "kv_tokens": main_r["kv_tokens"],
            "kv_bytes_per_step": main_r["kv_bytes_per_step"],
            "partition_size": main_r["partition_size"], "seed": main_r["seed"],
        },
        "pct_of_hbm_peak": round(main_r["pct_of_hbm_peak"], 2),
        "decode_tokens_per_s": round(main_r["decode_tokens_per_s"], 1),
        "roofline": {
            "kernel": ((("paged_attention_decode_append_fp8" if w.fp8 else
                         "paged_attention_decode_append") if main_r["append"].startswith("fused")
                        else ("paged_attention_decode_fp8" if w.fp8 else
                              "paged_attention_decode")) +
                       " call (decode kernel + merge kernel)"),
            "timing": main_r["decode_call_timing"],
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_for_current_kernel(w.key),
            "algorithmic_bytes_per_call": main_r["decode_algorithmic_bytes"],
            "avg_call_ms": round(dec_ms, 5),
        },
        "cpu_baseline": cpu,
        "translation": trans,
        "workloads": {w.key: main_r, **others},
        "prefill": prefill,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
