"""FP8 E4M3 KV cache, fp64 oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the product package never does.

The pages name quantized inference as a later topic (page "从零实现一个 mini
vLLM--开篇", section "5. 这个系列会怎么展开", stage six, and section "6. 我们不会
一开始就做什么") but fix no format.  The reading used here: each cache tensor
holds OCP FP8 E4M3 values ("E4M3FN": 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, subnormals, no infinities, NaN = S.1111.111) with one scale per
tensor, so stored byte e stands for scale * e4m3(e).

* ``e4m3_value`` -- the format's definition, written out for one byte.
* ``quantize`` -- an element x is stored as the E4M3 value nearest to
  clamp(x * inv, -448, 448), ties to the even code, with inv = 1 / scale and
  the product both IEEE single precision.  Written as a search over the 127
  finite magnitudes, not as bit manipulation.
* ``decode_fp8`` -- paged decode attention over the dequantized caches: the
  stored bytes become fp64 values scale * e4m3(e) (exact: a 4-bit significand
  times a 24-bit one) and go through the fp64 decode oracle unchanged.
* ``prefill_fp8`` -- causal chunked prefill over the dequantized caches, the
  same way, through the fp64 prefill oracle.

Pins (tests/test_oracle_fp8.py): the value table against PyTorch's
float8_e4m3fn type and hand-decoded codes, the quantizer against PyTorch's
cast on clamped inputs, hand-worked ties, the half-spacing error bound and
monotonicity, and decode_fp8 and prefill_fp8 against dense attention on the
dequantized rows.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

FP8_MAX = 448.0
NAN_CODES = (0x7F, 0xFF)


def e4m3_value(code: int) -> float:
    """The number an E4M3FN byte stands for (NaN for S.1111.111)."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:  # subnormal: 0.man * 2^(1 - bias)
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


# value of every byte, fp64
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# the 127 finite non-negative magnitudes in code order (codes 0x00 .. 0x7E),
# which is also increasing order
_MAGS = E4M3_TABLE[:0x7F].copy()


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """scale * e4m3(code) for every byte, fp64 (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)] * float(scale)


def _nearest_code(y: np.ndarray) -> np.ndarray:
    """E4M3 byte nearest to each fp64 value y (|y| <= 448 or NaN), ties to the
    even code; the sign bit follows y's sign, zero included."""
    y = np.asarray(y, dtype=np.float64)
    nan = np.isnan(y)
    mag = np.where(nan, 0.0, np.abs(y))
    assert np.all(mag <= FP8_MAX)
    hi = np.searchsorted(_MAGS, mag, side="left")  # first magnitude >= |y|
    hi = np.minimum(hi, len(_MAGS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _MAGS[lo]
    d_hi = _MAGS[hi] - mag
    exact = d_hi == 0
    pick_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = code | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), code).astype(np.uint8)


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """Bytes of an fp8 cache for the fp32 elements x: nearest E4M3 to
    clamp(fp32(x * fp32(1 / scale)), +-448), ties to even.  NaN gives a NaN
    code (compare NaN inputs by NaN-ness, not by byte)."""
    x32 = np.asarray(x, dtype=np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (x32 * inv).astype(np.float32)
    y64 = y.astype(np.float64)
    y64 = np.where(y64 > FP8_MAX, FP8_MAX, np.where(y64 < -FP8_MAX, -FP8_MAX, y64))
    return _nearest_code(y64)


def quantize_bf16(bits: np.ndarray, scale: float) -> np.ndarray:
    """``quantize`` of bfloat16 inputs given as bit patterns (uint16): the
    quantizer applied once to each of the 65536 bf16 values, then looked up."""
    every = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    table = quantize(every, scale)
    return table[np.asarray(bits, dtype=np.uint16)]


def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale: float,
                          v_scale: float) -> None:
    """In place on uint8 caches [nb, bs, hkv, d]: the row of token i goes to
    slot slot_mapping[i] (skipped when negative), quantized as ``quantize``."""
    nb, bs, hkv, d = k_cache.shape
    kq = quantize(key, k_scale).reshape(-1, hkv, d)
    vq = quantize(value, v_scale).reshape(-1, hkv, d)
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        b, o = divmod(int(slot), bs)
        k_cache[b, o] = kq[i]
        v_cache[b, o] = vq[i]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to fp64, exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_fp8(q_bits, k_codes, v_codes, block_tables, context_lens, scale: float,
               k_scale: float, v_scale: float, seq_range=None) -> np.ndarray:
    """fp64 decode attention over fp8 caches: q as bf16 bits [S, Hq, D], caches
    uint8 [nb, 16, Hkv, D]; returns [S, Hq, D] fp64."""
    q64 = np.ascontiguousarray(bf16_bits_to_f64(q_bits))
    kd = np.ascontiguousarray(dequantize(k_codes, k_scale))
    vd = np.ascontiguousarray(dequantize(v_codes, v_scale))
    return oracle.decode(q64, kd, vd, block_tables, context_lens, scale, seq_range=seq_range)


def prefill_fp8(q_bits, k_codes, v_codes, block_tables, query_start_loc, context_lens, scale: float,
                k_scale: float, v_scale: float, seq_range=None) -> np.ndarray:
    """fp64 causal chunked prefill over fp8 caches: q as bf16 bits [rows, Hq, D],
    caches uint8 [nb, 16, Hkv, D]; returns [rows, Hq, D] fp64."""
    q64 = np.ascontiguousarray(bf16_bits_to_f64(q_bits))
    kd = np.ascontiguousarray(dequantize(k_codes, k_scale))
    vd = np.ascontiguousarray(dequantize(v_codes, v_scale))
    return oracle.prefill(q64, kd, vd, block_tables, query_start_loc, context_lens, scale, seq_range=seq_range)
