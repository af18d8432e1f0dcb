"""Seeded synthetic workloads for paged-KV decode, KV append and chunked prefill.

This module only draws inputs: context lengths, block tables, slot mappings,
query/key/value values and the KV pool's initial contents.  It holds none of
the attention arithmetic.  Both the HIP path (through the tests and the bench)
and the CPU oracle consume what it returns.

Recipe (the same for every workload):
  * structure from ``numpy.random.default_rng(seed)``, drawn in this order:
    context lengths, then one random permutation of the physical pool;
  * values from a seeded ``torch.Generator`` (CPU), drawn in this order:
    decode queries, new keys, new values, prefill queries, then the cached
    history, all fp32 N(0, 1) rounded to the workload's dtype (round to
    nearest even);
  * every sequence takes consecutive entries of the permutation as its block
    table (so logically adjacent blocks are physically scattered); unused
    table entries are -1 unless the workload says otherwise;
  * every slot that holds no history token -- unreferenced blocks, the stale
    tail of each sequence's last block, and the slots the new tokens are about
    to be written to -- holds NaN, so a read of a slot that should not be read
    poisons the result;
  * decode appends one new token per sequence at logical position N_s - 1
    (N_s counts the token being decoded); a prefill chunk of c tokens appends
    positions N_s - c .. N_s - 1;
  * pool size, where the workload fixes none: the smallest power of two that is
    at least twice the number of blocks the sequences need.

Block size is 16 tokens, the example size of the mini-vllm write-up
(page "轻量级的vLLM", section 核心机制一：分页 KV Cache).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

BLOCK_SIZE = 16
BF16_NAN_BITS = 0x7FC0


@dataclass
class PrefillPart:
    """Chunked-prefill sequences: one chunk of query rows per sequence."""
    context_lens: np.ndarray      # [Sp] int32, prefix + chunk
    block_tables: np.ndarray      # [Sp, MB] int32
    query_start_loc: np.ndarray   # [Sp + 1] int32
    q: np.ndarray                 # [rows, Hq, D] float32 or uint16 (bf16 bits)


@dataclass
class Workload:
    name: str
    dtype: str                    # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    num_blocks: int
    max_blocks_per_seq: int
    # decode sequences
    context_lens: np.ndarray      # [S] int32
    block_tables: np.ndarray      # [S, MB] int32
    q: np.ndarray                 # [S, Hq, D]
    # tokens appended this step (prefill chunk tokens first, then decode tokens)
    slot_mapping: np.ndarray      # [T] int32
    k_new: np.ndarray             # [T, Hkv, D]
    v_new: np.ndarray             # [T, Hkv, D]
    # KV pool before the append
    k_cache: np.ndarray           # [NB, 16, Hkv, D]
    v_cache: np.ndarray
    prefill: Optional[PrefillPart] = None
    meta: Dict = field(default_factory=dict)

    @property
    def block_size(self) -> int:
        return BLOCK_SIZE

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def decode_kv_bytes(self) -> int:
        """Bytes of K and V that decode must read once: sum N_s * Hkv * D * 2 * e."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * \
            self.head_dim * 2 * self.elem_bytes


# ----------------------------------------------------------------------------------
# Named workloads.  Sizes follow the model shapes they are named after:
# Qwen3-0.6B (16 query / 8 kv heads, head_dim 128) and Llama-3-8B (32 / 8, 128).
# ----------------------------------------------------------------------------------
CONFIG_NAMES = ("tiny_fp32", "qwen3_0p6b", "llama3_8b", "long_skewed", "mixed_prefill")


def _pow2_pool(blocks_needed: int) -> int:
    n = 1
    while n < 2 * blocks_needed:
        n *= 2
    return n


def _draw_context_lens(name: str, rng: np.random.Generator, num_seqs: int) -> np.ndarray:
    if name == "tiny_fp32":
        return rng.integers(1, 64, size=num_seqs, endpoint=True)
    if name == "qwen3_0p6b":
        return rng.integers(128, 2048, size=num_seqs, endpoint=True)
    if name == "llama3_8b":
        u = rng.uniform(math.log(64), math.log(4097), size=num_seqs)
        return np.clip(np.floor(np.exp(u)), 64, 4096).astype(np.int64)
    if name == "long_skewed":
        # truncated Pareto(x_m = 1024, alpha = 1.2) on [1024, 65536] by inverse CDF,
        # sequence 0 pinned at 65536
        xm, cap, alpha = 1024.0, 65536.0, 1.2
        u = rng.uniform(0.0, 1.0, size=num_seqs)
        x = xm / np.power(1.0 - u * (1.0 - (xm / cap) ** alpha), 1.0 / alpha)
        n = np.clip(np.floor(x), 1024, 65536).astype(np.int64)
        n[0] = 65536
        return n
    if name == "mixed_prefill":
        return rng.integers(256, 4096, size=num_seqs, endpoint=True)
    raise KeyError(name)


_SHAPES = {
    # name: (default seqs, Hq, Hkv, D, dtype, max context for the block-table width)
    "tiny_fp32": (4, 4, 2, 64, "f32", 64),
    "qwen3_0p6b": (32, 16, 8, 128, "bf16", 2048),
    "llama3_8b": (128, 32, 8, 128, "bf16", 4096),
    "long_skewed": (16, 16, 8, 128, "bf16", 65536),
    "mixed_prefill": (124, 32, 8, 128, "bf16", 4096),
}

# mixed_prefill: number of chunked-prefill sequences, chunk length, prefix range
_PREFILL_SEQS, _CHUNK, _PREFIX_LO, _PREFIX_HI = 4, 512, 1024, 3072


class _Values:
    """fp32 N(0,1) draws from one seeded torch generator, rounded to the dtype."""

    def __init__(self, seed: int, dtype: str):
        import torch
        self.torch = torch
        self.gen = torch.Generator().manual_seed(seed)
        self.dtype = dtype

    def draw(self, *shape) -> np.ndarray:
        torch = self.torch
        x = torch.randn(*shape, generator=self.gen, dtype=torch.float32)
        if self.dtype == "f32":
            return x.numpy()
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _nan_pool(nb: int, hkv: int, d: int, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.full((nb, BLOCK_SIZE, hkv, d), np.nan, dtype=np.float32)
    return np.full((nb, BLOCK_SIZE, hkv, d), BF16_NAN_BITS, dtype=np.uint16)


def token_slots(block_table_row: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Physical slot (block * 16 + offset) of logical positions of one sequence.

    This is how a cache manager turns a block table into the slot mapping it
    hands to the KV append; it is input bookkeeping, not attention arithmetic.
    """
    positions = np.asarray(positions, dtype=np.int64)
    return block_table_row[positions // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + \
        positions % BLOCK_SIZE


def make_workload(name: str, seed: int = 0, num_seqs: Optional[int] = None,
                  with_values: bool = True) -> Workload:
    """Build one named workload.

    ``num_seqs`` overrides the number of decode sequences (same length
    distribution), which gives small parity cases with the full-size shape.
    ``with_values=False`` skips the value draws (structure only).
    """
    if name not in _SHAPES:
        raise KeyError(f"unknown workload {name!r}; known: {CONFIG_NAMES}")
    s_default, hq, hkv, d, dtype, max_ctx = _SHAPES[name]
    s = int(num_seqs if num_seqs is not None else s_default)
    rng = np.random.default_rng(seed)

    # 1. context lengths (decode sequences, then prefill prefixes)
    ctx = _draw_context_lens(name, rng, s).astype(np.int64)
    pre_ctx = None
    if name == "mixed_prefill":
        prefix = rng.integers(_PREFIX_LO, _PREFIX_HI, size=_PREFILL_SEQS, endpoint=True)
        pre_ctx = prefix.astype(np.int64) + _CHUNK
        max_ctx = max(max_ctx, _PREFIX_HI + _CHUNK)
    mb = -(-max_ctx // BLOCK_SIZE)

    # 2. pool and block tables
    all_ctx = ctx if pre_ctx is None else np.concatenate([pre_ctx, ctx])
    need = -(-all_ctx // BLOCK_SIZE)
    if name == "tiny_fp32":
        nb = 32
        mb = nb // s_default if s == s_default else mb
    elif name == "qwen3_0p6b" and s == s_default:
        nb = 8192
    else:
        nb = _pow2_pool(int(need.sum()))
    perm = rng.permutation(nb).astype(np.int64)
    tables = np.full((all_ctx.shape[0], mb), -1, dtype=np.int32)
    if name == "tiny_fp32" and s == s_default:
        # the whole pool, permuted, is the block table
        tables[:] = perm.reshape(s, mb)
    else:
        off = 0
        for i, k in enumerate(need):
            tables[i, :k] = perm[off:off + k]
            off += k
    pre_tables = None
    if pre_ctx is not None:
        pre_tables, tables = tables[:_PREFILL_SEQS].copy(), tables[_PREFILL_SEQS:].copy()

    scale = 0.125 if name == "tiny_fp32" else 1.0 / math.sqrt(d)

    # slot mapping: prefill chunk tokens first, then one new token per decode sequence
    slots = []
    qsl = None
    if pre_ctx is not None:
        qsl = np.zeros(_PREFILL_SEQS + 1, dtype=np.int32)
        for i in range(_PREFILL_SEQS):
            n = int(pre_ctx[i])
            slots.append(token_slots(pre_tables[i], np.arange(n - _CHUNK, n)))
            qsl[i + 1] = qsl[i] + _CHUNK
    for i in range(s):
        n = int(ctx[i])
        slots.append(token_slots(tables[i], np.array([n - 1])))
    slot_mapping = np.concatenate(slots).astype(np.int32)
    t_new = slot_mapping.shape[0]

    wl_kwargs = dict(
        name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, scale=scale,
        num_blocks=nb, max_blocks_per_seq=mb, context_lens=ctx.astype(np.int32),
        block_tables=tables, slot_mapping=slot_mapping,
        meta=dict(seed=seed, pool_blocks=nb, tokens_appended=t_new),
    )
    if not with_values:
        return Workload(q=None, k_new=None, v_new=None, k_cache=None, v_cache=None,
                        prefill=None if pre_ctx is None else PrefillPart(
                            pre_ctx.astype(np.int32), pre_tables, qsl, None),
                        **wl_kwargs)

    # 3. values: q, k_new, v_new, prefill q, then the pool's history tokens
    vals = _Values(seed, dtype)
    q = vals.draw(s, hq, d)
    k_new = vals.draw(t_new, hkv, d)
    v_new = vals.draw(t_new, hkv, d)
    pre = None
    if pre_ctx is not None:
        pre = PrefillPart(pre_ctx.astype(np.int32), pre_tables, qsl,
                          vals.draw(int(qsl[-1]), hq, d))

    k_cache = _nan_pool(nb, hkv, d, dtype)
    v_cache = _nan_pool(nb, hkv, d, dtype)
    kflat = k_cache.reshape(nb * BLOCK_SIZE, hkv, d)
    vflat = v_cache.reshape(nb * BLOCK_SIZE, hkv, d)
    hist = []
    if pre_ctx is not None:
        for i in range(_PREFILL_SEQS):
            hist.append(token_slots(pre_tables[i], np.arange(int(pre_ctx[i]) - _CHUNK)))
    for i in range(s):
        hist.append(token_slots(tables[i], np.arange(int(ctx[i]) - 1)))
    hist_slots = np.concatenate(hist) if hist else np.zeros(0, np.int64)
    chunk = 1 << 15
    for a in range(0, hist_slots.shape[0], chunk):
        sl = hist_slots[a:a + chunk]
        kflat[sl] = vals.draw(sl.shape[0], hkv, d)
        vflat[sl] = vals.draw(sl.shape[0], hkv, d)

    return Workload(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                    prefill=pre, **wl_kwargs)
