"""fp64 CPU oracle for paged KV-cache attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product package
``paged_kv_cache_275_amd`` never imports it, and the two share no code.

The arithmetic lives in ``pa_oracle.c`` (plain fp64 loops, one token at a
time through the block table); this module only marshals numpy arrays into
it.  Element arrays are numpy ``float32`` for fp32 data, ``uint16`` (the raw
bit patterns) for bfloat16 data and ``float64`` for values exact only in fp64
(a dequantized fp8 cache; ``oracle.fp8``).

Every function here is pinned by ``tests/test_oracle.py`` against quantities
the oracle does not compute itself: dense attention over contiguously laid-out
K/V in numpy, PyTorch's scaled-dot-product attention in fp64, numpy fancy-index
assignment for the cache write, hand-worked cases under ``tests/golden/`` and
invariants (block permutation, weights summing to one, single-token context,
constant V, zero query).  No oracle function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DT_F32 = 0
DT_BF16 = 1
DT_F64 = 2

_lib: Optional[ctypes.CDLL] = None


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (-O2, no fast-math) into a shared object."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = _LIB_PATH) -> ctypes.CDLL:
    """Load a compiled oracle (building it only if no library is present)."""
    global _lib
    if path == _LIB_PATH and _lib is not None:
        return _lib
    if not os.path.exists(path):
        if path != _LIB_PATH:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    p, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_reshape_and_cache.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i32]
    lib.oracle_decode.argtypes = [p, p, p, p, p, i64, p, i64, i64, i64, i64, i64, i64, i64,
                                  f64, i32]
    lib.oracle_prefill.argtypes = [p, p, p, p, p, i64, p, p, i64, i64, i64, i64, i64, i64,
                                   i64, f64, i32]
    lib.oracle_decode_row_weights.argtypes = [p, p, p, p, p, p, i64, p, i64, i64, i64, i64,
                                              i64, i64, i64, f64, i32]
    for fn in (lib.oracle_reshape_and_cache, lib.oracle_decode, lib.oracle_prefill,
               lib.oracle_decode_row_weights):
        fn.restype = ctypes.c_int
    if path == _LIB_PATH:
        _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float64:
        return DT_F64
    raise TypeError(f"oracle element arrays are float32, uint16(bf16 bits) or float64, got {a.dtype}")


def _c(a: np.ndarray, dtype=None) -> np.ndarray:
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what}: oracle rejected the input (code {rc})")


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, lib=None) -> None:
    """In place: cache[slot // B, slot % B] = key[i] (and value) for slot >= 0."""
    lib = lib or load()
    for a in (key, value, k_cache, v_cache):
        assert a.flags.c_contiguous
    nb, bs, hkv, d = k_cache.shape
    sm = _c(slot_mapping, np.int32)
    rc = lib.oracle_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(sm), key.shape[0], hkv, d, bs, nb,
                                      _dtype_code(k_cache))
    _check(rc, "reshape_and_cache")


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float,
           seq_range=None, lib=None) -> np.ndarray:
    """fp64 decode attention, [S, Hq, D].  seq_range=(a, b) limits the rows computed."""
    lib = lib or load()
    s, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    bt = _c(block_tables, np.int32)
    cl = _c(context_lens, np.int32)
    out = np.zeros((s, hq, d), dtype=np.float64)
    a, b = seq_range if seq_range is not None else (0, s)
    rc = lib.oracle_decode(_ptr(out), _ptr(_c(q)), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                           bt.shape[1], _ptr(cl), a, b, hq, hkv, d, bs, nb, float(scale),
                           _dtype_code(k_cache))
    _check(rc, "decode")
    return out


def decode_rows_into(out: np.ndarray, q, k_cache, v_cache, block_tables, context_lens,
                     scale: float, a: int, b: int, lib=None) -> None:
    """Like decode() but writes sequences [a, b) into a caller-owned fp64 array."""
    lib = lib or load()
    s, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    rc = lib.oracle_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                           _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                           a, b, hq, hkv, d, bs, nb, float(scale), _dtype_code(k_cache))
    _check(rc, "decode")


def prefill(q, k_cache, v_cache, block_tables, query_start_loc, context_lens, scale: float,
            seq_range=None, lib=None) -> np.ndarray:
    """fp64 causal chunked-prefill attention, [total_rows, Hq, D]."""
    lib = lib or load()
    rows, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    bt = _c(block_tables, np.int32)
    qsl = _c(query_start_loc, np.int32)
    cl = _c(context_lens, np.int32)
    out = np.zeros((rows, hq, d), dtype=np.float64)
    a, b = seq_range if seq_range is not None else (0, cl.shape[0])
    rc = lib.oracle_prefill(_ptr(out), _ptr(_c(q)), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                            bt.shape[1], _ptr(qsl), _ptr(cl), a, b, hq, hkv, d, bs, nb,
                            float(scale), _dtype_code(k_cache))
    _check(rc, "prefill")
    return out


def decode_row_weights(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                       s: int, h: int, lib=None):
    """(weights[N_s], out_row[D]) of one decode row, both fp64."""
    lib = lib or load()
    _, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    bt = _c(block_tables, np.int32)
    cl = _c(context_lens, np.int32)
    w = np.zeros(max(int(cl[s]), 1), dtype=np.float64)
    o = np.zeros(d, dtype=np.float64)
    rc = lib.oracle_decode_row_weights(_ptr(w), _ptr(o), _ptr(_c(q)), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(bt), bt.shape[1], _ptr(cl), s, h,
                                       hq, hkv, d, bs, nb, float(scale), _dtype_code(k_cache))
    _check(rc, "decode_row_weights")
    return w[: int(cl[s])], o

