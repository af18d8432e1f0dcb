"""C-ABI checks that need no GPU: the library loads, exports every function
include/pa.h declares, and rejects bad arguments on the host before any HIP
call (fake non-null pointers are never dereferenced on these paths)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

from paged_kv_cache_275_amd import ops

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        from paged_kv_cache_275_amd import build
        build.build()
    return ops.load_library()


def test_exports_every_declared_symbol(lib):
    names = ops.header_functions()
    assert {"pa_reshape_and_cache", "pa_decode", "pa_prefill_chunk", "pa_decode_workspace_size",
            "pa_prefill_workspace_size", "pa_status_string", "pa_decode_timed",
            "pa_decode_append", "pa_decode_append_timed", "pa_decode_append_graph", "pa_graph_launch",
            "pa_graph_destroy", "pa_copy_blocks", "pa_bm_create", "pa_bm_append_batch",
            "pa_reshape_and_cache_fp8", "pa_decode_fp8", "pa_decode_fp8_timed", "pa_prefill_chunk_fp8"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libpa.so does not export {n}"
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.pa_status_string(code).startswith(b"PA_")
    assert lib.pa_status_string(123) == b"unknown pa_status"


def _decode_append(lib, timed=False, **kw):
    a = dict(out=FAKE, q=FAKE, key=FAKE, value=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, mb=4, cl=FAKE, s=2, hq=8,
             hkv=2, d=128, bs=16, nb=64, scale=0.1, dtype=ops.PA_BF16, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    args = (a["out"], a["q"], a["key"], a["value"], a["kc"], a["vc"], a["bt"], a["mb"], a["cl"], a["s"],
            a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["scale"], a["dtype"], a["ws"], a["ws_bytes"],
            a["stream"])
    if timed:
        return lib.pa_decode_append_timed(*args, FAKE, FAKE)
    return lib.pa_decode_append(*args)


def _decode(lib, timed=False, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, mb=4, cl=FAKE, s=2, hq=8, hkv=2, d=128,
             bs=16, nb=64, scale=0.1, dtype=ops.PA_BF16, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    args = (a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["mb"], a["cl"], a["s"],
            a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["scale"], a["dtype"],
            a["ws"], a["ws_bytes"], a["stream"])
    if timed:
        # fake event handles: argument checks come first, so they are never used
        return lib.pa_decode_timed(*args, FAKE, FAKE)
    return lib.pa_decode(*args)


@pytest.mark.parametrize("kw,code", [
    (dict(hq=6, hkv=4), ops.PA_EINVAL),               # heads not a multiple
    (dict(hkv=0), ops.PA_EINVAL),
    (dict(d=96), ops.PA_EUNSUPPORTED),
    (dict(bs=32), ops.PA_EUNSUPPORTED),
    (dict(dtype=7), ops.PA_EUNSUPPORTED),
    (dict(hq=130, hkv=2), ops.PA_EUNSUPPORTED),        # 65 query heads per kv head
    (dict(s=-1), ops.PA_EINVAL),
    (dict(nb=0), ops.PA_EINVAL),
    (dict(nb=(1 << 31) // 16 + 1), ops.PA_EINVAL),     # slots overflow int32
    (dict(mb=0), ops.PA_EINVAL),
    (dict(scale=float("nan")), ops.PA_EINVAL),
    (dict(q=None), ops.PA_EINVAL),
    (dict(bt=None), ops.PA_EINVAL),
    (dict(ws=None), ops.PA_EWORKSPACE),
    (dict(ws_bytes=16), ops.PA_EWORKSPACE),
    (dict(s=8193), ops.PA_EUNSUPPORTED),
])
def test_decode_rejects(lib, kw, code):
    assert _decode(lib, **kw) == code
    assert _decode(lib, timed=True, **kw) == code
    assert _decode_append(lib, **kw) == code
    assert _decode_append(lib, timed=True, **kw) == code


def test_graph_entry_points_reject_without_launching(lib):
    h = ctypes.c_void_p()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 8, 2, 128, 16, 64, 0.1, ops.PA_BF16, FAKE,
            1 << 30]
    assert lib.pa_decode_append_graph(None, *args) == ops.PA_EINVAL
    bad = list(args); bad[9] = 0                                 # num_seqs 0
    assert lib.pa_decode_append_graph(ctypes.byref(h), *bad) == ops.PA_EINVAL
    bad = list(args); bad[12] = 96                               # head_dim 96
    assert lib.pa_decode_append_graph(ctypes.byref(h), *bad) == ops.PA_EUNSUPPORTED
    bad = list(args); bad[2] = None                              # key
    assert lib.pa_decode_append_graph(ctypes.byref(h), *bad) == ops.PA_EINVAL
    assert not h.value
    assert lib.pa_graph_launch(None, None) == ops.PA_EINVAL
    assert lib.pa_graph_destroy(None) == ops.PA_OK


@pytest.mark.parametrize("kw", [dict(key=None), dict(value=None)])
def test_decode_append_needs_new_tokens(lib, kw):
    assert _decode_append(lib, **kw) == ops.PA_EINVAL
    assert _decode_append(lib, timed=True, **kw) == ops.PA_EINVAL


def test_decode_empty_batch_is_noop(lib):
    assert _decode(lib, s=0, q=None, out=None) == ops.PA_OK


def test_decode_workspace_size(lib):
    small = lib.pa_decode_workspace_size(128, 32, 8, 128, 4, 16)
    assert small > 0                                   # prefix sums + partial records
    # monotone in the shape arguments that size it; independent of the table width
    assert lib.pa_decode_workspace_size(256, 32, 8, 128, 4, 16) >= small
    assert lib.pa_decode_workspace_size(128, 64, 8, 128, 4, 16) >= small
    assert lib.pa_decode_workspace_size(128, 32, 8, 128, 4096, 16) == small
    assert lib.pa_decode_workspace_size(128, 30, 8, 128, 4, 16) == 0   # invalid heads


def test_reshape_and_cache_rejects(lib):
    f = lib.pa_reshape_and_cache
    ok = dict(k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, sm=FAKE, t=4, hkv=8, d=128, bs=16, nb=32,
              dt=ops.PA_BF16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["k"], a["v"], a["kc"], a["vc"], a["sm"], a["t"], a["hkv"], a["d"], a["bs"],
                 a["nb"], a["dt"], None)

    assert call(t=-1) == ops.PA_EINVAL
    assert call(hkv=0) == ops.PA_EINVAL
    assert call(d=80) == ops.PA_EUNSUPPORTED
    assert call(bs=8) == ops.PA_EUNSUPPORTED
    assert call(dt=3) == ops.PA_EUNSUPPORTED
    assert call(sm=None) == ops.PA_EINVAL
    assert call(t=0, k=None, v=None) == ops.PA_OK      # nothing to append


def test_prefill_rejects(lib):
    f = lib.pa_prefill_chunk

    def call(**kw):
        a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, mb=8, qsl=FAKE, rows=64, cl=FAKE,
                 s=2, hq=32, hkv=8, d=128, bs=16, nb=64, scale=0.1, dt=ops.PA_BF16)
        a.update(kw)
        return f(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["mb"], a["qsl"], a["rows"],
                 a["cl"], a["s"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["scale"], a["dt"],
                 None, 0, None)

    assert call(hq=30) == ops.PA_EINVAL
    assert call(rows=-1) == ops.PA_EINVAL
    assert call(d=256) == ops.PA_EUNSUPPORTED
    assert call(qsl=None) == ops.PA_EINVAL
    assert call(rows=0, q=None) == ops.PA_OK


# ---------------------------------------------------------------- fp8 caches
def _decode_fp8(lib, timed=False, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, mb=4, cl=FAKE, s=2, hq=8, hkv=2, d=128,
             bs=16, nb=64, scale=0.1, ks=0.02, vs=0.03, dtype=ops.PA_BF16, ws=FAKE, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    args = (a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["mb"], a["cl"], a["s"], a["hq"], a["hkv"], a["d"],
            a["bs"], a["nb"], a["scale"], a["ks"], a["vs"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])
    if timed:
        return lib.pa_decode_fp8_timed(*args, FAKE, FAKE)
    return lib.pa_decode_fp8(*args)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=ops.PA_F32), ops.PA_EUNSUPPORTED),     # fp8 caches go with bf16 q/out
    (dict(dtype=ops.PA_FP8_E4M3), ops.PA_EUNSUPPORTED),
    (dict(s=0, ks=0.0), ops.PA_EINVAL),                # scale checks come before the empty-batch exit
    (dict(s=0, vs=-1.0), ops.PA_EINVAL),
    (dict(s=0, ks=float("inf")), ops.PA_EINVAL),
    (dict(s=0, vs=float("nan")), ops.PA_EINVAL),
    (dict(s=0, ks=1e-39), ops.PA_EINVAL),               # reciprocal would overflow
    (dict(d=96), ops.PA_EUNSUPPORTED),
    (dict(hq=6, hkv=4), ops.PA_EINVAL),
    (dict(q=None), ops.PA_EINVAL),
    (dict(ws_bytes=16), ops.PA_EWORKSPACE),
    (dict(s=8193), ops.PA_EUNSUPPORTED),
    (dict(s=0, q=None, out=None), ops.PA_OK),
])
def test_decode_fp8_rejects(lib, kw, code):
    assert _decode_fp8(lib, **kw) == code
    assert _decode_fp8(lib, timed=True, **kw) == code


def test_reshape_and_cache_fp8_rejects(lib):
    f = lib.pa_reshape_and_cache_fp8

    def call(**kw):
        a = dict(k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, sm=FAKE, t=4, hkv=8, d=128, bs=16, nb=32, dt=ops.PA_BF16,
                 ks=0.5, vs=0.25)
        a.update(kw)
        return f(a["k"], a["v"], a["kc"], a["vc"], a["sm"], a["t"], a["hkv"], a["d"], a["bs"], a["nb"], a["dt"],
                 a["ks"], a["vs"], None)

    assert call(t=-1) == ops.PA_EINVAL
    assert call(d=80) == ops.PA_EUNSUPPORTED
    assert call(dt=ops.PA_FP8_E4M3) == ops.PA_EUNSUPPORTED   # sources are fp32 or bf16
    assert call(t=0, ks=0.0) == ops.PA_EINVAL
    assert call(t=0, vs=float("nan")) == ops.PA_EINVAL
    assert call(sm=None) == ops.PA_EINVAL
    assert call(t=0, k=None, v=None) == ops.PA_OK


def test_bit_copies_accept_fp8_storage(lib):
    # pa_reshape_and_cache and pa_copy_blocks treat PA_FP8_E4M3 as a 1-byte
    # element type: with nothing to copy they succeed, with an unknown type not
    from paged_kv_cache_275_amd import blocks
    lib = blocks._lib()   # declares pa_copy_blocks' signature
    assert lib.pa_reshape_and_cache(None, None, FAKE, FAKE, None, 0, 8, 128, 16, 32, ops.PA_FP8_E4M3, None) == 0
    assert lib.pa_copy_blocks(FAKE, FAKE, None, 0, 8, 64, 16, 32, ops.PA_FP8_E4M3, None) == 0
    assert lib.pa_copy_blocks(FAKE, FAKE, None, 0, 8, 64, 16, 32, 9, None) == ops.PA_EUNSUPPORTED


def test_prefill_fp8_rejects(lib):
    f = lib.pa_prefill_chunk_fp8

    def call(**kw):
        a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, mb=8, qsl=FAKE, rows=64, cl=FAKE,
                 s=2, hq=32, hkv=8, d=128, bs=16, nb=64, scale=0.1, ks=0.02, vs=0.03, dt=ops.PA_BF16)
        a.update(kw)
        return f(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["mb"], a["qsl"], a["rows"], a["cl"], a["s"],
                 a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["scale"], a["ks"], a["vs"], a["dt"], None, 0, None)

    assert call(hq=30) == ops.PA_EINVAL
    assert call(d=256) == ops.PA_EUNSUPPORTED
    assert call(dt=ops.PA_F32) == ops.PA_EUNSUPPORTED
    assert call(rows=0, ks=0.0) == ops.PA_EINVAL           # scale checks before the empty exit
    assert call(rows=0, vs=float("inf")) == ops.PA_EINVAL
    assert call(qsl=None) == ops.PA_EINVAL
    assert call(rows=0, q=None) == ops.PA_OK


def test_stream_read_probe_argument_checks(lib):
    """Rejected on the host before any HIP call: null pointers, a size that is
    not a multiple of 16, a misaligned source; zero bytes is a no-op."""
    assert lib.pa_stream_read_probe(None, 64, FAKE, None) == ops.PA_EINVAL
    assert lib.pa_stream_read_probe(FAKE, 64, None, None) == ops.PA_EINVAL
    assert lib.pa_stream_read_probe(FAKE, 24, FAKE, None) == ops.PA_EINVAL
    assert lib.pa_stream_read_probe(ctypes.c_void_p(0x1008), 64, FAKE, None) == ops.PA_EINVAL
    assert lib.pa_stream_read_probe(None, 0, None, None) == ops.PA_OK


def _decode_append_fp8(lib, graph=False, **kw):
    a = dict(out=FAKE, q=FAKE, key=FAKE, value=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, mb=4, cl=FAKE, s=2, hq=8, hkv=2,
             d=128, bs=16, nb=64, scale=0.1, ks=0.02, vs=0.03, dtype=ops.PA_BF16, ws=FAKE, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    args = (a["out"], a["q"], a["key"], a["value"], a["kc"], a["vc"], a["bt"], a["mb"], a["cl"], a["s"], a["hq"],
            a["hkv"], a["d"], a["bs"], a["nb"], a["scale"], a["ks"], a["vs"], a["dtype"], a["ws"], a["ws_bytes"])
    if graph:
        h = ctypes.c_void_p()
        rc = lib.pa_decode_append_fp8_graph(ctypes.byref(h), *args)
        assert not h.value, "a rejected call must not return a graph"
        return rc
    return lib.pa_decode_append_fp8(*args, a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(key=None), ops.PA_EINVAL),                   # the step needs the new rows
    (dict(value=None), ops.PA_EINVAL),
    (dict(dtype=ops.PA_F32), ops.PA_EUNSUPPORTED),     # fp8 caches go with bf16 q/out/rows
    (dict(s=0, ks=0.0), ops.PA_EINVAL),
    (dict(s=0, vs=float("nan")), ops.PA_EINVAL),
    (dict(d=96), ops.PA_EUNSUPPORTED),
    (dict(hq=6, hkv=4), ops.PA_EINVAL),
    (dict(ws_bytes=16), ops.PA_EWORKSPACE),
    (dict(s=8193), ops.PA_EUNSUPPORTED),
])
def test_decode_append_fp8_rejects(lib, kw, code):
    """Rejected before anything is enqueued (FAKE pointers are never touched)."""
    assert _decode_append_fp8(lib, **kw) == code
    assert _decode_append_fp8(lib, graph=True, **kw) == code


def test_decode_append_fp8_graph_needs_sequences(lib):
    assert _decode_append_fp8(lib, graph=True, s=0) == ops.PA_EINVAL
    assert lib.pa_decode_append_fp8_graph(None, *([FAKE] * 7), 4, FAKE, 2, 8, 2, 128, 16, 64, 0.1, 0.02,
                                          0.03, ops.PA_BF16, FAKE, 1 << 30) == ops.PA_EINVAL
    assert _decode_append_fp8(lib, s=0, q=None, out=None) == ops.PA_OK   # empty batch: nothing to do
