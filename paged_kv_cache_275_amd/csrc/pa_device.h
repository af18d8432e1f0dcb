// pa_device.h -- device-side helpers shared by the libpa kernels (gfx950 only).
//
// Wave64 lane exchanges use DPP row patterns and the gfx950 permlane swaps;
// bf16 arithmetic uses v_dot2_f32_bf16 (two bf16 products accumulated into an
// fp32) and v_cvt_pk_bf16_f32 (round to nearest even).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockTokens = 16;  // tokens per KV block
constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// DPP controls (row = 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within each 8 lanes
constexpr int kDppRowRor8 = 0x128;     // lane i <- lane (i+8) mod 16 within a row
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor2 = 0x122;
constexpr int kDppRowRor1 = 0x121;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 lanes that share lane bits 3..5 (an aligned group of 8).
__device__ __forceinline__ float sum_lanes8(float x) {
    x += dpp_f32<kDppQuadXor1>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppHalfMirror>(x);
    return x;
}

// Reduce across lane bits 3..5 (the eight groups of 8 lanes): xor 8 within a
// row by DPP, xor 16 and xor 32 by the gfx950 permlane swaps.
__device__ __forceinline__ float max_groups8(float x) {
    x = fmaxf(x, dpp_f32<kDppRowRor8>(x));
    {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return x;
}

__device__ __forceinline__ float sum_groups8(float x) {
    x += dpp_f32<kDppRowRor8>(x);
    {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return x;
}

__device__ __forceinline__ float readlane_f32(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Inclusive prefix sum over the 64 lanes of a wave: row_shr 1, 2, 4, 8 within
// each 16-lane row, then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then the first two rows' total into rows 2 and 3
// (row_bcast:31).  Lanes without a source read 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_src_i32(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWMASK, 0xF, true);
}
__device__ __forceinline__ int wave_scan_incl(int x) {
    x += dpp_src_i32<0x111, 0xF>(x);
    x += dpp_src_i32<0x112, 0xF>(x);
    x += dpp_src_i32<0x114, 0xF>(x);
    x += dpp_src_i32<0x118, 0xF>(x);
    x += dpp_src_i32<0x142, 0xA>(x);
    x += dpp_src_i32<0x143, 0xC>(x);
    return x;
}

// D[16x16] += A[16x32] * B[32x16] in bf16 with fp32 accumulation.  Lane l holds
// A row l%16 and B column l%16, k-slots 8*(l/16) .. +8 (8 bf16 in 16 bytes);
// it receives D column l%16, rows 4*(l/16) .. +3.
__device__ __forceinline__ f32x4_t mfma16x16x32_bf16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D[16x16] += A[16x16] * B[16x16] in bf16 with fp32 accumulation.  Lane l holds
// A row l%16 and B column l%16, k-slots 4*(l/16) .. +4 (4 bf16 in two dwords,
// slot 0 in the low half of the first); it receives D column l%16, rows
// 4*(l/16) .. +3.
__device__ __forceinline__ f32x4_t mfma16x16x16_bf16(uint2 a, uint2 b, f32x4_t c) {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                     0, 0, 0);
}

// Sum and max over the four 16-lane rows (lanes l, l^16, l^32, l^48) by the
// gfx950 permlane swaps; every lane gets the result.
__device__ __forceinline__ float sum_rows4(float x) {
    {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return x;
}
__device__ __forceinline__ float max_rows4(float x) {
    {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return x;
}

// Max and sum over all 64 lanes (every lane gets the result): DPP rotations
// within each 16-lane row, then the permlane swaps across rows.
__device__ __forceinline__ float wave_max64(float x) {
    x = fmaxf(x, dpp_f32<kDppRowRor8>(x));
    x = fmaxf(x, dpp_f32<kDppRowRor4>(x));
    x = fmaxf(x, dpp_f32<kDppRowRor2>(x));
    x = fmaxf(x, dpp_f32<kDppRowRor1>(x));
    return max_rows4(x);
}
__device__ __forceinline__ float wave_sum64(float x) {
    x += dpp_f32<kDppRowRor8>(x);
    x += dpp_f32<kDppRowRor4>(x);
    x += dpp_f32<kDppRowRor2>(x);
    x += dpp_f32<kDppRowRor1>(x);
    return sum_rows4(x);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two fp32 values to a packed bf16 pair (lo in bits 0..15), nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load with the non-temporal hint (global_load ... nt): for data read
// exactly once, such as the KV stream of decode.  Measured on llama3_8b decode:
// about 2 us of 93 faster than plain loads.
__device__ __forceinline__ uint4 ldg_nt(const void* p) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// KW consecutive dwords (KW = 1, 2 or 4, aligned to their size), non-temporal.
template <int KW>
__device__ __forceinline__ void ldg_nt_words(uint32_t (&dst)[KW], const void* p) {
    if constexpr (KW == 4) {
        const uint4 v = ldg_nt(p);
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    } else if constexpr (KW == 2) {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        dst[0] = v.x; dst[1] = v.y;
    } else {
        static_assert(KW == 1, "1, 2 or 4 dwords");
        dst[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
}

// ---- FP8 E4M3 (OCP "E4M3FN": bias 7, largest finite 448, no infinities).
// gfx950's conversions use this format and round to nearest even; a value
// beyond +-448 would become NaN, so quantization clamps first.
constexpr float kFp8Max = 448.0f;

// Two fp8 values (bytes 0 and 1 of w, or bytes 2 and 3 when HI) as a bf16
// pair, first value in the low half.  Exact: every e4m3 value is a bf16.  The
// gfx950 conversion takes an f32 scale of which it uses only the exponent;
// 1.0 leaves the values as they are.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Eight fp8 values (two dwords, value 0 in the low byte) as eight bf16, in
// order, in a uint4 (an MFMA operand).
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    return make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
                      fp8x2_to_bf16x2<true>(w1));
}

// Clamp to the finite range, NaN kept (comparisons with NaN are false).
__device__ __forceinline__ float fp8_clamp(float x) { return x > kFp8Max ? kFp8Max : (x < -kFp8Max ? -kFp8Max : x); }

// Four floats to four e4m3 bytes (value 0 in the low byte), nearest even.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(a), fp8_clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(c), fp8_clamp(d), w, true);
    return (uint32_t)w;
}

}  // namespace pa
