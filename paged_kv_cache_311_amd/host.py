"""Binding of the host block manager and decode-loop simulator
(libpkvhost.so, include/pkv_block_manager.h): argument marshalling only.

    bm = BlockManager(num_blocks, block_size=16)
    bm.add_sequence(seq_id, prompt_tokens)
    bm.fork(parent, child)
    slots, pairs = bm.append_slots([seq ids])     # one new token each
    order, starts, shared = bm.prefix_groups([seq ids])  # shared-prefix decode
    tables, lens = bm.block_tables([seq ids], width)
    bm.free_sequence(seq_id)

    paged, slab = simulate(num_requests=..., lengths="uniform", ...)

Errors raise: PoolExhausted when the pool has too few free blocks (the
manager is unchanged), ValueError for anything else the library rejects.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB_PATH = os.path.join(HERE, "libpkvhost.so")

OK, INVALID, NO_BLOCKS = 0, -1, -5
ABI_VERSION = 3

_lib = None


class PoolExhausted(RuntimeError):
    """The pool has too few free blocks; nothing was changed."""


class _SimConfig(ctypes.Structure):
    _fields_ = [("num_requests", ctypes.c_int64), ("lengths", ctypes.c_int32),
                ("min_len", ctypes.c_int32), ("max_len", ctypes.c_int32),
                ("median", ctypes.c_double), ("sigma", ctypes.c_double),
                ("prompt_fraction", ctypes.c_double), ("pool_tokens", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class _SimResult(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("tokens_generated", ctypes.c_int64),
                ("utilization", ctypes.c_double), ("mean_batch", ctypes.c_double),
                ("max_batch", ctypes.c_int32), ("preemptions", ctypes.c_int64),
                ("recomputed_tokens", ctypes.c_int64), ("max_tail_waste", ctypes.c_int32)]


def load_host_library(path=HOST_LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "pkv_bm_abi_version": ([], ctypes.c_int),
        "pkv_bm_create": ([I32, I32], P),
        "pkv_bm_destroy": ([P], None),
        "pkv_bm_num_blocks": ([P], I32),
        "pkv_bm_block_size": ([P], I32),
        "pkv_bm_num_free": ([P], I32),
        "pkv_bm_num_sequences": ([P], I32),
        "pkv_bm_refcount": ([P, I32], I32),
        "pkv_bm_shared_flags": ([P, P, I32], I32),
        "pkv_bm_prefix_groups": ([P, P, I32, P, P, P, P], ctypes.c_int),
        "pkv_bm_add_sequence": ([P, I64, I64], ctypes.c_int),
        "pkv_bm_fork": ([P, I64, I64], ctypes.c_int),
        "pkv_bm_append_slot": ([P, I64, P, P, P], ctypes.c_int),
        "pkv_bm_append_slots": ([P, P, I32, P, P, P, P], ctypes.c_int),
        "pkv_bm_free_sequence": ([P, I64], ctypes.c_int),
        "pkv_bm_seq_len": ([P, I64], I64),
        "pkv_bm_block_table": ([P, I64, P, I32], I32),
        "pkv_bm_block_tables": ([P, P, I32, P, I32, P], ctypes.c_int),
        "pkv_sim_decode": ([ctypes.POINTER(_SimConfig), ctypes.POINTER(_SimResult),
                            ctypes.POINTER(_SimResult)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, res
    if lib.pkv_bm_abi_version() != ABI_VERSION:
        raise RuntimeError("libpkvhost.so was built from another header version")
    _lib = lib
    return lib


def _check(rc):
    if rc == NO_BLOCKS:
        raise PoolExhausted("not enough free blocks")
    if rc != OK:
        raise ValueError(f"block manager rejected the call (status {rc})")


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


class BlockManager:
    """A pool of fixed-size KV blocks with per-sequence block tables,
    reference-counted sharing and copy-on-write (see pkv_block_manager.h)."""

    def __init__(self, num_blocks, block_size=16):
        self._lib = load_host_library()
        self._h = self._lib.pkv_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError("invalid pool size")

    def close(self):
        if self._h:
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    num_blocks = property(lambda self: self._lib.pkv_bm_num_blocks(self._h))
    block_size = property(lambda self: self._lib.pkv_bm_block_size(self._h))
    num_free = property(lambda self: self._lib.pkv_bm_num_free(self._h))
    num_sequences = property(lambda self: self._lib.pkv_bm_num_sequences(self._h))

    def refcount(self, block):
        return self._lib.pkv_bm_refcount(self._h, int(block))

    def shared_flags(self):
        """uint8 [num_blocks]: 1 where a block has more than one reference
        (the decode calls' block_shared flags)."""
        out = np.zeros(self.num_blocks, dtype=np.uint8)
        n = self._lib.pkv_bm_shared_flags(self._h, out.ctypes.data_as(ctypes.c_void_p),
                                          len(out))
        _check(n if n < 0 else 0)
        return out

    def prefix_groups(self, seq_ids):
        """(order int32 [n], group_start int32 [G + 1], prefix_blocks int32
        [G]) for a batch of these sequences: the group description of
        paged_attention_decode_shared_prefix, from the tables and reference
        counts (sequences sharing a full first block grouped, with their
        common full leading blocks)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = len(ids)
        order = np.empty(n, np.int32)
        starts = np.empty(n + 1, np.int32)
        shared = np.empty(max(n, 1), np.int32)
        g = ctypes.c_int32()
        _check(self._lib.pkv_bm_prefix_groups(self._h, _ptr(ids), n, _ptr(order),
                                               _ptr(starts), _ptr(shared), ctypes.byref(g)))
        return order, starts[:g.value + 1].copy(), shared[:g.value].copy()

    def add_sequence(self, seq_id, num_tokens):
        _check(self._lib.pkv_bm_add_sequence(self._h, int(seq_id), int(num_tokens)))

    def fork(self, parent, child):
        _check(self._lib.pkv_bm_fork(self._h, int(parent), int(child)))

    def append_slot(self, seq_id):
        """Slot of the sequence's next token and the copy-on-write pair
        (src, dst), or None."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pkv_bm_append_slot(self._h, int(seq_id), ctypes.byref(slot),
                                            ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def append_slots(self, seq_ids):
        """One new token for each sequence, in order: slots int64 [n] and
        copy-on-write pairs int64 [k, 2] (the inputs of reshape_and_cache
        and copy_blocks)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = len(ids)
        slots = np.empty(n, np.int64)
        pairs = np.empty((max(n, 1), 2), np.int64)
        npairs, done = ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pkv_bm_append_slots(self._h, _ptr(ids), n, _ptr(slots), _ptr(pairs),
                                             ctypes.byref(npairs), ctypes.byref(done)))
        return slots, pairs[:npairs.value].copy()

    def free_sequence(self, seq_id):
        _check(self._lib.pkv_bm_free_sequence(self._h, int(seq_id)))

    def seq_len(self, seq_id):
        n = self._lib.pkv_bm_seq_len(self._h, int(seq_id))
        if n < 0:
            raise ValueError(f"unknown sequence {seq_id}")
        return n

    def block_table(self, seq_id, width=None):
        if width is None:
            width = -(-self.seq_len(seq_id) // self.block_size)
        out = np.empty(width, np.int32)
        n = self._lib.pkv_bm_block_table(self._h, int(seq_id), _ptr(out), int(width))
        if n < 0:
            raise ValueError(f"unknown sequence {seq_id} or table wider than {width}")
        return out

    def block_tables(self, seq_ids, width):
        """int32 block tables [n, width] (-1 past each sequence's last block)
        and int32 context lengths [n] -- the decode kernel's inputs."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((len(ids), width), np.int32)
        lens = np.empty(len(ids), np.int32)
        _check(self._lib.pkv_bm_block_tables(self._h, _ptr(ids), len(ids), _ptr(tables),
                                             int(width), _ptr(lens)))
        return tables, lens


def simulate(num_requests, lengths="uniform", min_len=2, max_len=2048, median=600.0,
             sigma=0.8, prompt_fraction=0.5, pool_tokens=None, block_size=16, seed=0):
    """Run the decode-loop simulator (pkv_sim_decode) and return the paged
    and slab results as dicts."""
    lib = load_host_library()
    if pool_tokens is None:
        pool_tokens = 64 * max_len
    cfg = _SimConfig(num_requests, {"uniform": 0, "lognormal": 1}[lengths], min_len, max_len,
                     median, sigma, prompt_fraction, pool_tokens, block_size, seed)
    paged, slab = _SimResult(), _SimResult()
    _check(lib.pkv_sim_decode(ctypes.byref(cfg), ctypes.byref(paged), ctypes.byref(slab)))
    as_dict = lambda r: {f: getattr(r, f) for f, _ in r._fields_}
    return as_dict(paged), as_dict(slab)
