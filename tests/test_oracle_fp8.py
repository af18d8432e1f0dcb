"""Pins of the fp8 KV-cache oracle (oracle/fp8.py) against what fixes it from
outside: the OCP E4M3 ("E4M3FN") definition decoded by hand, PyTorch's own
float8_e4m3fn type (an independent implementation of the format and of its
round-to-nearest-even cast), hand-worked ties, the half-spacing error bound,
and dense attention over the dequantized rows."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.fp8 as F
from tests._helpers import dense_decode, dense_prefill, gather_dense

torch = pytest.importorskip("torch")


def _torch_e4m3_values() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_value_table_matches_torch_float8_e4m3fn():
    tv = _torch_e4m3_values()
    nan = np.isnan(F.E4M3_TABLE)
    assert np.array_equal(nan, np.isnan(tv))
    assert np.array_equal(F.E4M3_TABLE[~nan], tv[~nan])
    # signed zeros too
    assert np.signbit(F.E4M3_TABLE[0x80]) and not np.signbit(F.E4M3_TABLE[0x00])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0),
    (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
])
def test_hand_decoded_codes(code, value):
    # sign | exponent (bias 7) | mantissa, subnormal when the exponent is 0
    assert F.e4m3_value(code) == value


def test_only_two_nan_codes_and_no_infinity():
    nan_codes = [c for c in range(256) if math.isnan(F.E4M3_TABLE[c])]
    assert nan_codes == list(F.NAN_CODES)
    assert np.all(np.isfinite(F.E4M3_TABLE[~np.isnan(F.E4M3_TABLE)]))
    assert np.nanmax(F.E4M3_TABLE) == F.FP8_MAX


def test_quantize_matches_torch_cast_on_clamped_inputs():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-14, 7, 200_000))).astype(np.float32)
    specials = np.array([0.0, -0.0, 448, -448, 464, -464, 447.9, 1e-9, -1e-9, 2.0 ** -10, 3 * 2.0 ** -10],
                        dtype=np.float32)
    x = np.concatenate([x, specials])
    got = F.quantize(x, 1.0)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),          # halfway between 1 (0x38) and 1.125 (0x39): even code
    (1.1875, 0x3A),          # halfway between 1.125 and 1.25 (0x3A): even code
    (2.0 ** -10, 0x00),      # half the smallest subnormal: to zero
    (3 * 2.0 ** -10, 0x02),  # halfway between 2^-9 and 2^-8: even code
    (-0.0, 0x80), (0.0, 0x00),
    (500.0, 0x7E), (-1.0e6, 0xFE),  # clamped to +-448
    (240.0, 0x77),           # 240 = 1.875 * 2^7, exactly representable
])
def test_hand_worked_roundings(x, code):
    assert int(F.quantize(np.array([x], np.float32), 1.0)[0]) == code


def test_quantize_uses_fp32_reciprocal_and_product():
    # scale 3: fp32(1/3) = 0.3333333432674408, and for the fp32 input
    # x = 0.0556640587747097 the fp32 product x * fp32(1/3) is exactly
    # 0.0185546875, the midpoint of 0x09 (1.125 * 2^-6) and 0x0A (1.25 * 2^-6):
    # the tie goes to the even code 0x0A.  The exact quotient x / 3 =
    # 0.0185546862... lies below the midpoint and would give 0x09.
    x = np.array([0.0556640587747097], np.float32)
    assert float(x[0] * (np.float32(1) / np.float32(3))) == 0.0185546875
    assert int(F.quantize(x, 3.0)[0]) == 0x0A


def test_quantize_bf16_is_quantize_of_the_widened_values():
    rng = np.random.default_rng(8)
    bits = rng.integers(0, 65536, size=50_000).astype(np.uint16)
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    got, ref = F.quantize_bf16(bits, 0.03), F.quantize(x, 0.03)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isin(got[nan], F.NAN_CODES))


def test_nan_input_gives_nan_code():
    c = F.quantize(np.array([np.nan, -np.nan], np.float32), 1.0)
    assert all(int(v) in F.NAN_CODES for v in c)


def test_error_bound_and_monotonicity():
    rng = np.random.default_rng(5)
    x = np.sort(rng.uniform(-448, 448, 100_000).astype(np.float32))
    v = F.E4M3_TABLE[F.quantize(x, 1.0)]
    # half the spacing of the binade holding |x|: 2^(e - 3) / 2 with e = floor(log2|x|),
    # and 2^-10 in the subnormal range
    ax = np.abs(x.astype(np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -6)))
    half = 2.0 ** (e - 4)
    assert np.all(np.abs(v - x) <= half)
    assert np.all(np.diff(v) >= 0)


def test_reshape_and_cache_fp8_against_fancy_indexing():
    rng = np.random.default_rng(3)
    nb, hkv, d, t = 6, 2, 64, 20
    kc = np.full((nb, 16, hkv, d), 0x7F, np.uint8)
    vc = kc.copy()
    slots = rng.permutation(nb * 16)[:t].astype(np.int32)
    slots[4] = -1
    k = rng.standard_normal((t, hkv, d)).astype(np.float32)
    v = rng.standard_normal((t, hkv, d)).astype(np.float32)
    F.reshape_and_cache_fp8(k, v, kc, vc, slots, 0.05, 0.02)
    ek = np.full_like(kc, 0x7F).reshape(-1, hkv, d)
    ev = ek.copy()
    keep = slots >= 0
    ek[slots[keep]] = torch.from_numpy(np.clip(k[keep] * (np.float32(1) / np.float32(0.05)), -448, 448)) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ev[slots[keep]] = torch.from_numpy(np.clip(v[keep] * (np.float32(1) / np.float32(0.02)), -448, 448)) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(kc.reshape(-1, hkv, d), ek)
    assert np.array_equal(vc.reshape(-1, hkv, d), ev)


def _fp8_case(rng, hq, hkv, d, lens, k_scale, v_scale):
    s = len(lens)
    need = [-(-n // 16) for n in lens]
    nb = sum(need) + 3
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((s, max(need)), -1, np.int32)
    off = 0
    for i, k in enumerate(need):
        bt[i, :k] = perm[off:off + k]
        off += k
    kc = rng.integers(0, 256, size=(nb, 16, hkv, d), dtype=np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x00  # no NaN codes in used slots
    vc = rng.integers(0, 256, size=(nb, 16, hkv, d), dtype=np.uint8)
    vc[(vc & 0x7F) == 0x7F] = 0x01
    q = (rng.standard_normal((s, hq, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return q, kc, vc, bt, np.asarray(lens, np.int32)


def test_decode_fp8_against_dense_attention_on_dequantized_rows():
    rng = np.random.default_rng(9)
    ks, vs, scale = 0.003, 0.007, 0.11
    q, kc, vc, bt, lens = _fp8_case(rng, 8, 2, 64, [1, 17, 40], ks, vs)
    got = F.decode_fp8(q, kc, vc, bt, lens, scale, ks, vs)
    kd = F.E4M3_TABLE[kc] * ks
    vd = F.E4M3_TABLE[vc] * vs
    ref = dense_decode(q, kd, vd, bt, lens, scale)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    # k_scale and v_scale are not interchangeable
    wrong = dense_decode(q, F.E4M3_TABLE[kc] * vs, F.E4M3_TABLE[vc] * ks, bt, lens, scale)
    assert not np.allclose(got, wrong, rtol=1e-3, atol=1e-6)


def test_decode_fp8_single_token_is_v_scaled_row():
    rng = np.random.default_rng(4)
    q, kc, vc, bt, lens = _fp8_case(rng, 4, 4, 64, [1], 0.5, 0.25)
    got = F.decode_fp8(q, kc, vc, bt, lens, 0.3, 0.5, 0.25)
    row = gather_dense(vc, bt[0], 1)[0]  # [Hkv, D] codes
    assert np.array_equal(got[0], F.E4M3_TABLE[row] * 0.25)


def test_prefill_fp8_against_dense_causal_attention():
    rng = np.random.default_rng(12)
    ks, vs, scale = 0.004, 0.006, 0.1
    chunks, prefixes = [5, 19], [0, 30]
    lens = [c + p for c, p in zip(chunks, prefixes)]
    q_all, kc, vc, bt, cl = _fp8_case(rng, 8, 2, 64, lens, ks, vs)
    qsl = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = (rng.standard_normal((int(qsl[-1]), 8, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    got = F.prefill_fp8(q, kc, vc, bt, qsl, cl, scale, ks, vs)
    ref = dense_prefill(q, F.E4M3_TABLE[kc] * ks, F.E4M3_TABLE[vc] * vs, bt, qsl, cl, scale)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    wrong = dense_prefill(q, F.E4M3_TABLE[kc] * vs, F.E4M3_TABLE[vc] * ks, bt, qsl, cl, scale)
    assert not np.allclose(got, wrong, rtol=1e-3, atol=1e-6)
