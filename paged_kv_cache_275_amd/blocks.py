"""ctypes binding of the host block manager in libpa.so (pa_bm_*, include/pa.h).

Argument marshalling only: the manager itself is C++ inside libpa.so.  It hands
out the pool's block ids to sequences and produces the block tables, context
lengths, slot mappings and copy-on-write pairs that the kernels take.
"""
from __future__ import annotations

import ctypes
from typing import List, Sequence, Tuple

import numpy as np

from paged_kv_cache_275_amd import ops


def _lib():
    lib = ops.load_library()
    if not getattr(lib, "_pa_bm_declared", False):
        p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.pa_bm_create.argtypes = [i64, i32]
        lib.pa_bm_create.restype = p
        lib.pa_bm_destroy.argtypes = [p]
        lib.pa_bm_destroy.restype = None
        lib.pa_bm_num_free.argtypes = [p]
        lib.pa_bm_num_free.restype = i64
        lib.pa_bm_refcount.argtypes = [p, i32]
        lib.pa_bm_refcount.restype = i32
        lib.pa_bm_add_sequence.argtypes = [p, i64, i64]
        lib.pa_bm_add_sequence.restype = ctypes.c_int
        lib.pa_bm_fork.argtypes = [p, i64, i64]
        lib.pa_bm_fork.restype = ctypes.c_int
        lib.pa_bm_free.argtypes = [p, i64]
        lib.pa_bm_free.restype = ctypes.c_int
        lib.pa_bm_num_tokens.argtypes = [p, i64]
        lib.pa_bm_num_tokens.restype = i64
        lib.pa_bm_append_batch.argtypes = [p, p, i32, p, p, i32, p]
        lib.pa_bm_append_batch.restype = ctypes.c_int
        lib.pa_bm_batch_tables.argtypes = [p, p, i32, p, i32, p]
        lib.pa_bm_batch_tables.restype = ctypes.c_int
        lib.pa_copy_blocks.argtypes = [p, p, p, i32, i32, i32, i32, i64, ctypes.c_int, p]
        lib.pa_copy_blocks.restype = ctypes.c_int
        lib._pa_bm_declared = True
    return lib


class BlockManager:
    """Owner of one pa_block_manager (see include/pa.h for the policy)."""

    def __init__(self, num_blocks: int, block_size: int = ops.BLOCK_SIZE):
        self._lib = _lib()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError("pa_bm_create refused the pool size or block size")
        self.num_blocks = int(num_blocks)

    def close(self) -> None:
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _check(self, fn, rc):
        if rc != ops.PA_OK:
            raise ops.PAError(fn, rc, self._lib.pa_status_string(rc).decode())

    @property
    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_refcount(self._h, int(block)))

    def add_sequence(self, seq_id: int, num_tokens: int) -> None:
        self._check("pa_bm_add_sequence", self._lib.pa_bm_add_sequence(self._h, int(seq_id), int(num_tokens)))

    def fork(self, parent_id: int, child_id: int) -> None:
        self._check("pa_bm_fork", self._lib.pa_bm_fork(self._h, int(parent_id), int(child_id)))

    def free(self, seq_id: int) -> None:
        self._check("pa_bm_free", self._lib.pa_bm_free(self._h, int(seq_id)))

    def num_tokens(self, seq_id: int) -> int:
        return int(self._lib.pa_bm_num_tokens(self._h, int(seq_id)))

    def append_batch(self, seq_ids: Sequence[int]) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """One new token per sequence: (slot_mapping int32 [n], copy pairs)."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = len(ids)
        slots = np.empty(n, np.int32)
        copies = np.empty(2 * max(n, 1), np.int32)
        nc = ctypes.c_int32(0)
        rc = self._lib.pa_bm_append_batch(self._h, ids.ctypes.data, n, slots.ctypes.data, copies.ctypes.data,
                                          n, ctypes.byref(nc))
        self._check("pa_bm_append_batch", rc)
        pairs = [(int(copies[2 * k]), int(copies[2 * k + 1])) for k in range(nc.value)]
        return slots, pairs

    def batch_tables(self, seq_ids: Sequence[int], max_blocks_per_seq: int) -> Tuple[np.ndarray, np.ndarray]:
        """(block_tables int32 [n, max_blocks_per_seq] padded with -1, context_lens int32 [n])."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = len(ids)
        bt = np.empty((n, max_blocks_per_seq), np.int32)
        cl = np.empty(n, np.int32)
        rc = self._lib.pa_bm_batch_tables(self._h, ids.ctypes.data, n, bt.ctypes.data, int(max_blocks_per_seq),
                                          cl.ctypes.data)
        self._check("pa_bm_batch_tables", rc)
        return bt, cl


def copy_blocks(k_cache, v_cache, pairs, stream=None) -> None:
    """pa_copy_blocks: block pairs[p, 1] of both caches becomes a copy of block
    pairs[p, 0]; pairs is a GPU int32 tensor [n, 2]."""
    import torch
    lib = _lib()
    ops._need(k_cache, "k_cache", dim=4)
    ops._need(v_cache, "v_cache", k_cache.dtype, 4)
    ops._need(pairs, "pairs", torch.int32, 2)
    if v_cache.shape != k_cache.shape or pairs.shape[1] != 2:
        raise ValueError("caches must match and pairs must be [n, 2]")
    nb, bs, hkv, d = k_cache.shape
    rc = lib.pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), pairs.data_ptr(), pairs.shape[0], hkv, d, bs,
                            nb, ops._dtype_code(k_cache), ops._stream_handle(k_cache, stream))
    ops._check(lib, "pa_copy_blocks", rc)
