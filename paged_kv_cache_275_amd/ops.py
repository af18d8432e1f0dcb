"""Thin ctypes binding over libpa.so (C ABI in include/pa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libpa.so.  Tensors are torch CUDA/HIP tensors on the current
device; their data pointers and the current stream are handed to the library
as they are.  The library must have been built (``python -m
paged_kv_cache_275_amd.build``); if it is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "pa.h")

PA_F32 = 0
PA_BF16 = 1
PA_FP8_E4M3 = 2
PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_ELAUNCH, PA_ENOMEM = 0, -1, -2, -3, -4, -5
BLOCK_SIZE = 16

_lib: Optional[ctypes.CDLL] = None


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpa.so and declare its signatures; raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_275_amd.build`")
    lib = ctypes.CDLL(path)
    p, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    lib.pa_reshape_and_cache.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i64, ctypes.c_int, p]
    lib.pa_reshape_and_cache.restype = ctypes.c_int
    lib.pa_reshape_and_cache_fp8.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i64, ctypes.c_int, f32, f32, p]
    lib.pa_reshape_and_cache_fp8.restype = ctypes.c_int
    lib.pa_decode_fp8.argtypes = [p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i64, f32, f32, f32,
                                  ctypes.c_int, p, sz, p]
    lib.pa_decode_fp8.restype = ctypes.c_int
    lib.pa_decode_fp8_timed.argtypes = [p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i64, f32, f32, f32,
                                        ctypes.c_int, p, sz, p, p, p]
    lib.pa_decode_fp8_timed.restype = ctypes.c_int
    lib.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.pa_decode_workspace_size.restype = sz
    lib.pa_decode.argtypes = [p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i64, f32,
                              ctypes.c_int, p, sz, p]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_timed.argtypes = [p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i64, f32,
                                    ctypes.c_int, p, sz, p, p, p]
    lib.pa_decode_timed.restype = ctypes.c_int
    lib.pa_decode_append.argtypes = [p, p, p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i64, f32,
                                     ctypes.c_int, p, sz, p]
    lib.pa_decode_append.restype = ctypes.c_int
    lib.pa_decode_append_timed.argtypes = [p, p, p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i64, f32,
                                           ctypes.c_int, p, sz, p, p, p]
    lib.pa_decode_append_timed.restype = ctypes.c_int
    lib.pa_decode_append_noalloc.argtypes = [p, p, p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i64, f32,
                                             ctypes.c_int, p]
    lib.pa_decode_append_noalloc.restype = ctypes.c_int
    lib.pa_decode_append_graph.argtypes = [ctypes.POINTER(p), p, p, p, p, p, p, p, i32, p, i32, i32, i32, i32,
                                           i32, i64, f32, ctypes.c_int, p, sz]
    lib.pa_decode_append_graph.restype = ctypes.c_int
    lib.pa_decode_append_fp8.argtypes = [p, p, p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i64, f32, f32, f32,
                                         ctypes.c_int, p, sz, p]
    lib.pa_decode_append_fp8.restype = ctypes.c_int
    lib.pa_decode_append_fp8_graph.argtypes = [ctypes.POINTER(p), p, p, p, p, p, p, p, i32, p, i32, i32, i32,
                                               i32, i32, i64, f32, f32, f32, ctypes.c_int, p, sz]
    lib.pa_decode_append_fp8_graph.restype = ctypes.c_int
    lib.pa_graph_launch.argtypes = [p, p]
    lib.pa_graph_launch.restype = ctypes.c_int
    lib.pa_graph_destroy.argtypes = [p]
    lib.pa_graph_destroy.restype = ctypes.c_int
    lib.pa_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.pa_prefill_workspace_size.restype = sz
    lib.pa_prefill_chunk.argtypes = [p, p, p, p, p, i32, p, i32, p, i32, i32, i32, i32, i32, i64,
                                     f32, ctypes.c_int, p, sz, p]
    lib.pa_prefill_chunk.restype = ctypes.c_int
    lib.pa_prefill_chunk_fp8.argtypes = [p, p, p, p, p, i32, p, i32, p, i32, i32, i32, i32, i32, i64,
                                         f32, f32, f32, ctypes.c_int, p, sz, p]
    lib.pa_prefill_chunk_fp8.restype = ctypes.c_int
    lib.pa_stream_read_probe.argtypes = [p, sz, p, p]
    lib.pa_stream_read_probe.restype = ctypes.c_int
    lib.pa_decode_set_launch.argtypes = [i32, i32, i32]
    lib.pa_decode_set_launch.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def header_functions(header: str = HEADER) -> list:
    """Names of the functions include/pa.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def _check(lib, fn: str, rc: int) -> None:
    if rc != PA_OK:
        raise PAError(fn, rc, lib.pa_status_string(rc).decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):  # the bytes of an fp8 cache
        return PA_FP8_E4M3
    raise TypeError(f"unsupported element type {t.dtype}; use float32, bfloat16 or fp8 (uint8) bytes")


def _need(t, name: str, dtype=None, dim: Optional[int] = None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")


def _stream_handle(t, stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return s.cuda_stream


def _reshape_and_cache_args(key, value, k_cache, v_cache, slot_mapping, stream) -> tuple:
    import torch
    _need(key, "key", dim=3)
    _need(value, "value", key.dtype, 3)
    _need(k_cache, "k_cache", key.dtype, 4)
    _need(v_cache, "v_cache", key.dtype, 4)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    nb, bs, hkv, d = k_cache.shape
    if tuple(key.shape[1:]) != (hkv, d) or value.shape != key.shape or v_cache.shape != k_cache.shape:
        raise ValueError("key/value [T, Hkv, D] must match caches [NB, 16, Hkv, D]")
    if slot_mapping.shape[0] != key.shape[0]:
        raise ValueError("slot_mapping must have one entry per token")
    return (key.data_ptr(), value.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            slot_mapping.data_ptr(), key.shape[0], hkv, d, bs, nb, _dtype_code(key),
            _stream_handle(key, stream))


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """k_cache[slot // 16, slot % 16] = key[i] (and value), for slot_mapping[i] >= 0."""
    lib = load_library()
    args = _reshape_and_cache_args(key, value, k_cache, v_cache, slot_mapping, stream)
    _check(lib, "pa_reshape_and_cache", lib.pa_reshape_and_cache(*args))


def bind_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """Check the arguments once; return f() that enqueues the same append again.

    For loops that repeat one call on fixed buffers (benchmarks): the returned
    function only crosses the C ABI.  The tensors must stay alive.
    """
    lib = load_library()
    args = _reshape_and_cache_args(key, value, k_cache, v_cache, slot_mapping, stream)
    fn = lib.pa_reshape_and_cache

    def call():
        _check(lib, "pa_reshape_and_cache", fn(*args))
    return call


def _need_fp8_cache(t, name: str):
    import torch
    _need(t, name, dim=4)
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"{name} must hold fp8 E4M3 bytes (torch.uint8 or torch.float8_e4m3fn), got {t.dtype}")


def _reshape_and_cache_fp8_args(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale, stream) -> tuple:
    import torch
    _need(key, "key", dim=3)
    _need(value, "value", key.dtype, 3)
    _need_fp8_cache(k_cache, "k_cache")
    _need_fp8_cache(v_cache, "v_cache")
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    nb, bs, hkv, d = k_cache.shape
    if tuple(key.shape[1:]) != (hkv, d) or value.shape != key.shape or v_cache.shape != k_cache.shape:
        raise ValueError("key/value [T, Hkv, D] must match caches [NB, 16, Hkv, D]")
    if slot_mapping.shape[0] != key.shape[0]:
        raise ValueError("slot_mapping must have one entry per token")
    return (key.data_ptr(), value.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            slot_mapping.data_ptr(), key.shape[0], hkv, d, bs, nb, _dtype_code(key), float(k_scale),
            float(v_scale), _stream_handle(key, stream))


def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale: float, v_scale: float,
                          stream=None) -> None:
    """KV append into fp8 caches (pa_reshape_and_cache_fp8): key/value fp32 or
    bf16 [T, Hkv, D]; caches uint8 [NB, 16, Hkv, D] holding E4M3 bytes, whose
    values are k_scale (v_scale) times the stored number."""
    lib = load_library()
    args = _reshape_and_cache_fp8_args(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale, stream)
    _check(lib, "pa_reshape_and_cache_fp8", lib.pa_reshape_and_cache_fp8(*args))


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          block_size=BLOCK_SIZE) -> int:
    return int(load_library().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                       head_dim, max_blocks_per_seq, block_size))


def decode_workspace(q, k_cache, block_tables, stream=None):
    """Allocate a workspace (torch, uint8) big enough for decode() with these shapes.

    With a stream other than the current one, the allocation is marked as in
    use by that stream (record_stream): the caching allocator then keeps the
    memory until the work enqueued there has finished, even when the caller
    drops the tensor right after enqueueing."""
    import torch
    n = decode_workspace_size(q.shape[0], q.shape[1], k_cache.shape[2], q.shape[2],
                              block_tables.shape[1], k_cache.shape[1])
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    if stream is not None:
        ws.record_stream(stream)
    return ws


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, workspace, stream) -> tuple:
    import torch
    _need(q, "q", dim=3)
    _need(out, "out", q.dtype, 3)
    _need(k_cache, "k_cache", q.dtype, 4)
    _need(v_cache, "v_cache", q.dtype, 4)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    s, hq, d = q.shape
    nb, bs, hkv, dk = k_cache.shape
    if out.shape != q.shape or dk != d or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q/out and the caches")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("block_tables and context_lens need one row per sequence")
    if workspace is None:
        workspace = decode_workspace(q, k_cache, block_tables, stream)
    args = (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(), s,
            hq, hkv, d, bs, nb, float(scale), _dtype_code(q), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_handle(q, stream))
    return args, workspace


def _event_handles(kernel_events):
    ev0, ev1 = kernel_events
    if not ev0.cuda_event or not ev1.cuda_event:
        raise ValueError("kernel_events must be created (recorded once) before use")
    return ev0.cuda_event, ev1.cuda_event


def decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, workspace=None,
           stream=None, kernel_events=None) -> None:
    """Paged-attention decode into out [S, Hq, D].

    kernel_events: optional (start, stop) pair of torch.cuda.Event, already
    created (recorded once); they receive the start and stop times of the
    library's streaming kernel (pa_decode_timed).
    """
    lib = load_library()
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, workspace, stream)
    if kernel_events is None:
        _check(lib, "pa_decode", lib.pa_decode(*args))
    else:
        _check(lib, "pa_decode_timed", lib.pa_decode_timed(*args, *_event_handles(kernel_events)))


def bind_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, workspace=None,
                stream=None):
    """Check the arguments once; return f(kernel_events=None) that enqueues the
    same decode again (see bind_reshape_and_cache)."""
    lib = load_library()
    args, ws = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, workspace, stream)
    plain, timed = lib.pa_decode, lib.pa_decode_timed

    def call(kernel_events=None, _keep=ws):
        if kernel_events is None:
            _check(lib, "pa_decode", plain(*args))
        else:
            _check(lib, "pa_decode_timed", timed(*args, *kernel_events))
    return call


def _decode_fp8_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale, workspace,
                     stream) -> tuple:
    import torch
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", q.dtype, 3)
    _need_fp8_cache(k_cache, "k_cache")
    _need_fp8_cache(v_cache, "v_cache")
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    s, hq, d = q.shape
    nb, bs, hkv, dk = k_cache.shape
    if out.shape != q.shape or dk != d or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q/out and the caches")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("block_tables and context_lens need one row per sequence")
    if workspace is None:
        workspace = decode_workspace(q, k_cache, block_tables, stream)
    args = (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(), s,
            hq, hkv, d, bs, nb, float(scale), float(k_scale), float(v_scale), PA_BF16, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_handle(q, stream))
    return args, workspace


def decode_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, k_scale: float,
               v_scale: float, workspace=None, stream=None, kernel_events=None) -> None:
    """Paged-attention decode over fp8 caches (pa_decode_fp8): q/out bf16
    [S, Hq, D], caches uint8 E4M3 bytes; kernel_events as in decode()."""
    lib = load_library()
    args, _ = _decode_fp8_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
                               workspace, stream)
    if kernel_events is None:
        _check(lib, "pa_decode_fp8", lib.pa_decode_fp8(*args))
    else:
        _check(lib, "pa_decode_fp8_timed", lib.pa_decode_fp8_timed(*args, *_event_handles(kernel_events)))


def bind_decode_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, k_scale: float,
                    v_scale: float, workspace=None, stream=None):
    """Check the arguments once; return f(kernel_events=None) that enqueues the
    same fp8 decode again (see bind_reshape_and_cache)."""
    lib = load_library()
    args, ws = _decode_fp8_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
                                workspace, stream)
    plain, timed = lib.pa_decode_fp8, lib.pa_decode_fp8_timed

    def call(kernel_events=None, _keep=ws):
        if kernel_events is None:
            _check(lib, "pa_decode_fp8", plain(*args))
        else:
            _check(lib, "pa_decode_fp8_timed", timed(*args, *kernel_events))
    return call


def _decode_append_args(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale, workspace,
                        stream) -> tuple:
    args, ws = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, workspace, stream)
    _need(key, "key", q.dtype, 3)
    _need(value, "value", q.dtype, 3)
    if tuple(key.shape) != (q.shape[0], k_cache.shape[2], q.shape[2]) or value.shape != key.shape:
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim]")
    return args[:2] + (key.data_ptr(), value.data_ptr()) + args[2:], ws


def decode_append(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale: float,
                  workspace=None, stream=None, kernel_events=None) -> None:
    """Decode step with the KV append fused in (pa_decode_append): key/value
    [S, Hkv, D] are each sequence's new token at position context_lens[s] - 1."""
    lib = load_library()
    args, _ = _decode_append_args(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale,
                                  workspace, stream)
    if kernel_events is None:
        _check(lib, "pa_decode_append", lib.pa_decode_append(*args))
    else:
        _check(lib, "pa_decode_append_timed",
               lib.pa_decode_append_timed(*args, *_event_handles(kernel_events)))


def bind_decode_append(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale: float,
                       workspace=None, stream=None):
    """Check the arguments once; return f(kernel_events=None) that enqueues the
    same fused decode step again (see bind_reshape_and_cache)."""
    lib = load_library()
    args, ws = _decode_append_args(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale,
                                   workspace, stream)
    plain, timed = lib.pa_decode_append, lib.pa_decode_append_timed

    def call(kernel_events=None, _keep=ws):
        if kernel_events is None:
            _check(lib, "pa_decode_append", plain(*args))
        else:
            _check(lib, "pa_decode_append_timed", timed(*args, *kernel_events))
    return call


def decode_append_noalloc(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale: float,
                          stream=None) -> None:
    """pa_decode_append_noalloc: the fused decode step with the library's fixed
    per-device scratch instead of a workspace (nothing is allocated)."""
    lib = load_library()
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, _NO_WORKSPACE, stream)
    _need(key, "key", q.dtype, 3)
    _need(value, "value", q.dtype, 3)
    if tuple(key.shape) != (q.shape[0], k_cache.shape[2], q.shape[2]) or value.shape != key.shape:
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim]")
    args = args[:2] + (key.data_ptr(), value.data_ptr()) + args[2:15] + (args[17],)
    _check(lib, "pa_decode_append_noalloc", lib.pa_decode_append_noalloc(*args))


def _decode_append_fp8_args(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                            v_scale, workspace, stream) -> tuple:
    import torch
    args, ws = _decode_fp8_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
                                workspace, stream)
    _need(key, "key", torch.bfloat16, 3)
    _need(value, "value", torch.bfloat16, 3)
    if tuple(key.shape) != (q.shape[0], k_cache.shape[2], q.shape[2]) or value.shape != key.shape:
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim]")
    return args[:2] + (key.data_ptr(), value.data_ptr()) + args[2:], ws


def decode_append_fp8(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale: float,
                      k_scale: float, v_scale: float, workspace=None, stream=None) -> None:
    """Decode step over fp8 caches (pa_decode_append_fp8): key/value bf16
    [S, Hkv, D], each sequence's new token, quantized into the caches at
    position context_lens[s] - 1, then attention over all tokens."""
    lib = load_library()
    args, _ = _decode_append_fp8_args(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale,
                                      k_scale, v_scale, workspace, stream)
    _check(lib, "pa_decode_append_fp8", lib.pa_decode_append_fp8(*args))


def bind_decode_append_fp8(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale: float,
                           k_scale: float, v_scale: float, workspace=None, stream=None):
    """Check the arguments once; return f() that enqueues the same fp8 decode
    step again (see bind_reshape_and_cache)."""
    lib = load_library()
    args, ws = _decode_append_fp8_args(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale,
                                       k_scale, v_scale, workspace, stream)
    fn = lib.pa_decode_append_fp8

    def call(_keep=ws):
        _check(lib, "pa_decode_append_fp8", fn(*args))
    return call


class _NoWorkspace:
    """Stands in for a workspace tensor where none is passed (no allocation)."""

    def data_ptr(self):
        return 0

    def numel(self):
        return 0

    def element_size(self):
        return 1


_NO_WORKSPACE = _NoWorkspace()


class DecodeStepGraph:
    """pa_decode_append recorded once as a HIP graph (pa_decode_append_graph),
    or pa_decode_append_fp8 (pa_decode_append_fp8_graph) when kv_scales =
    (k_scale, v_scale) is given for fp8 caches; launch() replays it on the
    current (or given) stream.  The tensors are kept alive by this object;
    refill their contents between launches."""

    def __init__(self, out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale: float,
                 workspace=None, kv_scales=None):
        lib = load_library()
        self._lib = lib
        self._h = ctypes.c_void_p()
        if kv_scales is None:
            args, ws = _decode_append_args(out, q, key, value, k_cache, v_cache, block_tables, context_lens,
                                           scale, workspace, None)
            _check(lib, "pa_decode_append_graph", lib.pa_decode_append_graph(ctypes.byref(self._h), *args[:-1]))
        else:
            args, ws = _decode_append_fp8_args(out, q, key, value, k_cache, v_cache, block_tables, context_lens,
                                               scale, kv_scales[0], kv_scales[1], workspace, None)
            _check(lib, "pa_decode_append_fp8_graph",
                   lib.pa_decode_append_fp8_graph(ctypes.byref(self._h), *args[:-1]))
        self._keep = (out, q, key, value, k_cache, v_cache, block_tables, context_lens, ws)
        self._device = q.device

    def launch(self, stream=None) -> None:
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self._device)
        _check(self._lib, "pa_graph_launch", self._lib.pa_graph_launch(self._h, s.cuda_stream))

    def close(self) -> None:
        if self._h:
            self._lib.pa_graph_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        self.close()


def prefill_workspace_size(num_seqs, total_query_rows, num_q_heads, head_dim, max_blocks_per_seq,
                           block_size=BLOCK_SIZE) -> int:
    return int(load_library().pa_prefill_workspace_size(num_seqs, total_query_rows, num_q_heads,
                                                        head_dim, max_blocks_per_seq, block_size))


def _prefill_args(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens, scale, workspace,
                  stream, fp8=False) -> tuple:
    import torch
    _need(q, "q", torch.bfloat16 if fp8 else None, dim=3)
    _need(out, "out", q.dtype, 3)
    if fp8:
        _need_fp8_cache(k_cache, "k_cache")
        _need_fp8_cache(v_cache, "v_cache")
    else:
        _need(k_cache, "k_cache", q.dtype, 4)
        _need(v_cache, "v_cache", q.dtype, 4)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    _need(context_lens, "context_lens", torch.int32, 1)
    rows, hq, d = q.shape
    nb, bs, hkv, dk = k_cache.shape
    sp = context_lens.shape[0]
    if out.shape != q.shape or dk != d or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q/out and the caches")
    if block_tables.shape[0] != sp or query_start_loc.shape[0] != sp + 1:
        raise ValueError("block_tables [S, MB] and query_start_loc [S+1] must match context_lens [S]")
    need = prefill_workspace_size(sp, rows, hq, d, block_tables.shape[1], bs)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if stream is not None:
            workspace.record_stream(stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), block_tables.shape[1], query_start_loc.data_ptr(), rows,
            context_lens.data_ptr(), sp, hq, hkv, d, bs, nb, float(scale), _dtype_code(q), ws_ptr,
            ws_bytes, _stream_handle(q, stream))
    return args, workspace


def prefill_chunk(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                  scale: float, workspace=None, stream=None) -> None:
    """Causal chunked prefill into out [rows, Hq, D] (see pa_prefill_chunk)."""
    lib = load_library()
    args, _ = _prefill_args(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens, scale,
                            workspace, stream)
    _check(lib, "pa_prefill_chunk", lib.pa_prefill_chunk(*args))


def prefill_chunk_fp8(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens, scale: float,
                      k_scale: float, v_scale: float, workspace=None, stream=None) -> None:
    """Causal chunked prefill over fp8 caches (pa_prefill_chunk_fp8): q/out bf16
    [rows, Hq, D], caches uint8 E4M3 bytes with per-tensor scales."""
    lib = load_library()
    args, _ = _prefill_args(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens, scale,
                            workspace, stream, fp8=True)
    args = args[:16] + (float(k_scale), float(v_scale)) + args[16:]
    _check(lib, "pa_prefill_chunk_fp8", lib.pa_prefill_chunk_fp8(*args))


def bind_prefill_chunk(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                       scale: float, workspace=None, stream=None):
    """Check the arguments once; return f() that enqueues the same prefill again
    (see bind_reshape_and_cache)."""
    lib = load_library()
    args, ws = _prefill_args(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens, scale,
                             workspace, stream)
    fn = lib.pa_prefill_chunk

    def call(_keep=ws):
        _check(lib, "pa_prefill_chunk", fn(*args))
    return call


def set_decode_launch(waves: int = 0, stages: int = 0, switch_ticks: int = -1) -> None:
    """pa_decode_set_launch: launch shape of later decode calls in this process
    (0 / 0 / -1 restore the defaults)."""
    lib = load_library()
    _check(lib, "pa_decode_set_launch", lib.pa_decode_set_launch(int(waves), int(stages), int(switch_ticks)))


class decode_launch:
    """Context manager: decode calls inside use this launch shape; the defaults
    are restored on exit."""

    def __init__(self, waves: int = 0, stages: int = 0, switch_ticks: int = -1):
        self.shape = (waves, stages, switch_ticks)

    def __enter__(self):
        set_decode_launch(*self.shape)
        return self

    def __exit__(self, *exc):
        set_decode_launch()
        return False


def stream_read_probe(src, xor_out, stream=None) -> None:
    """pa_stream_read_probe: one streaming read of the contiguous device tensor
    src (a multiple of 16 bytes), XOR-folding its 32-bit words into xor_out (a
    one-element int32 device tensor the caller sets; zero gives the XOR of src)."""
    import torch
    if not src.is_contiguous() or xor_out.dtype != torch.int32 or xor_out.numel() < 1:
        raise ValueError("src must be contiguous and xor_out a one-element int32 tensor")
    lib = load_library()
    _check(lib, "pa_stream_read_probe",
           lib.pa_stream_read_probe(src.data_ptr(), src.numel() * src.element_size(), xor_out.data_ptr(),
                                    _stream_handle(src, stream)))
