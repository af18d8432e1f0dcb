"""Test-side helpers: bf16 widening and dense (non-paged) attention in numpy.

None of this is used by the product path or by the oracle; it is the second,
independent formulation the oracle is pinned against: the pages' first,
contiguous KV layout (page "从零实现一个 mini vLLM--开篇", section
"8. 本系列的代码目标", step one), evaluated with whole-matrix numpy operations.
"""
from __future__ import annotations

import numpy as np


def widen(a: np.ndarray) -> np.ndarray:
    """Exact fp64 value of a float32 array or of bf16 bit patterns (uint16)."""
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise TypeError(a.dtype)


def gather_dense(cache: np.ndarray, table_row: np.ndarray, n: int) -> np.ndarray:
    """Contiguous [n, Hkv, D] copy of a sequence's first n tokens (numpy fancy indexing)."""
    nb, bs, hkv, d = cache.shape
    t = np.arange(n)
    return cache.reshape(nb * bs, hkv, d)[table_row[t // bs].astype(np.int64) * bs + t % bs]


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    allowed: np.ndarray | None = None) -> np.ndarray:
    """softmax(scale * q K^T) V with GQA by head repetition.

    q [R, Hq, D]; k, v [n, Hkv, D]; allowed [R, n] boolean mask (None = all).
    Returns [R, Hq, D] in fp64.
    """
    q = widen(q) if q.dtype != np.float64 else q
    k = widen(k) if k.dtype != np.float64 else k
    v = widen(v) if v.dtype != np.float64 else v
    hq, hkv = q.shape[1], k.shape[1]
    kr = np.repeat(k, hq // hkv, axis=1)          # [n, Hq, D]
    vr = np.repeat(v, hq // hkv, axis=1)
    s = np.einsum("rhd,nhd->rhn", q, kr) * scale    # [R, Hq, n]
    if allowed is not None:
        s = np.where(allowed[:, None, :], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    w = np.exp(s)
    w = w / w.sum(axis=-1, keepdims=True)
    return np.einsum("rhn,nhd->rhd", w, vr)


def dense_decode(wl_q, k_cache, v_cache, tables, ctx, scale, seqs=None) -> np.ndarray:
    s_all, hq, d = wl_q.shape
    out = np.zeros((s_all, hq, d))
    for s in (range(s_all) if seqs is None else seqs):
        n = int(ctx[s])
        if n == 0:
            continue
        k = gather_dense(k_cache, tables[s], n)
        v = gather_dense(v_cache, tables[s], n)
        out[s] = dense_attention(wl_q[s:s + 1], k, v, scale)[0]
    return out


def dense_prefill(q, k_cache, v_cache, tables, qsl, ctx, scale) -> np.ndarray:
    rows, hq, d = q.shape
    out = np.zeros((rows, hq, d))
    for s in range(len(ctx)):
        r0, r1, n = int(qsl[s]), int(qsl[s + 1]), int(ctx[s])
        c = r1 - r0
        k = gather_dense(k_cache, tables[s], n)
        v = gather_dense(v_cache, tables[s], n)
        pos = n - c + np.arange(c)
        allowed = np.arange(n)[None, :] <= pos[:, None]
        out[r0:r1] = dense_attention(q[r0:r1], k, v, scale, allowed)
    return out


def bf16_bits_from_float(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- tolerances
F32_ATOL = 1e-5          # fp32 attention: max-abs
BF16_ATOL = 2e-2         # bf16 attention: max-abs ...
BF16_ROW_RTOL = 1e-2     # ... and per (row, head): max|gpu - ref| / max|ref|


def attention_errors(got: np.ndarray, ref: np.ndarray):
    """(max-abs error, worst per-(row, head) relative error) of [R, H, D] arrays."""
    diff = np.abs(got - ref)
    scale = np.abs(ref).max(axis=-1)
    row = diff.max(axis=-1) / np.where(scale > 0, scale, 1.0)
    return float(diff.max()) if diff.size else 0.0, float(row.max()) if row.size else 0.0


def assert_attention_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, rel = attention_errors(got, ref)
    if dtype == "f32":
        assert mx <= F32_ATOL, f"{what}: fp32 max-abs error {mx:.3e} > {F32_ATOL}"
    else:
        assert mx <= BF16_ATOL, f"{what}: bf16 max-abs error {mx:.3e} > {BF16_ATOL}"
        assert rel <= BF16_ROW_RTOL, f"{what}: bf16 row-relative error {rel:.3e} > {BF16_ROW_RTOL}"
    return mx, rel
