// pa_decode.hip -- paged-attention decode for gfx950.
//
// What is computed: for every sequence s and query head h, exact softmax
// attention of q[s,h] over the n = context_lens[s] cached tokens of s, each
// token found through the block table (block_tables[s, t/16], offset t%16).
// Pages: "从零实现一个 mini vLLM--开篇", sections 2 (decode attends to every
// earlier token) and 5 (block table, PagedAttention); "vllm-v0 版本介绍",
// section 为什么需要推理框架？ (physically scattered blocks).
//
// How (MI355X design):
//  * A UNIT is one 16-token block of one (sequence, head group): the K and V
//    rows of one kv head in that block.  The persistent grid (sized to the
//    chip) is cut into wave GROUPS of n_kvg waves; wave kvg of a group owns head
//    group kvg.  The blocks of all sequences, concatenated, are split into one
//    contiguous range per group (stream-K style), and every wave of the group
//    streams that range for its head group.  So the waves of a group read the
//    kv heads of a block at about the same time -- whole 2 KB token rows, one
//    DRAM page each -- instead of one 256-byte head slice per page opening, and
//    every wave streams the same number of bytes whatever the length mix.
//    The split is measured in ticks: a block costs unit_ticks and each
//    sequence in a range adds switch_ticks for closing its segment, so waves
//    with many short sequences get fewer blocks.  Consecutive units of a wave
//    are consecutive blocks of one (sequence, head group) SEGMENT.
//    With 2 KB bf16 rows (8 kv heads, head_dim 128) the head groups form two
//    BANDS (kv heads 0-3 and 4-7), each with groups of 4 waves and its own
//    split; the second half of a token row streams slower, so the second band
//    gets a few more groups (DecodeArgs, decode_bands in pa_api.hip).
//  * Each wave owns ALL query heads (up to GP) that share the kv head, so every
//    K/V byte is read from HBM exactly once and reused from registers by the
//    whole GQA group.
//  * Lane layout for one block, bf16 queries: lane = 16*q + r.  For the
//    scores lane r loads 16 bytes of token r's key row per MFMA step; for
//    P*V lane (q, r) loads D/16 contiguous dims (r*D/16 ..) of tokens 4q ..
//    4q+3, so each load instruction reads four whole 128-byte (fp8) or
//    256-byte (bf16) head rows.  fp32 path: lane = 8*tg + dl, token group tg
//    (0..7) owns tokens tg and tg+8, and chunk c of lane dl holds dims
//    c*8*E + dl*E .. +E (E = elements per 16 bytes).
//  * K/V are loaded with the non-temporal hint (read once, never reused).
//  * A ring of STAGES blocks is in flight per wave: the loads of unit x+STAGES
//    are issued as soon as unit x has been consumed (unconditionally, so that
//    the hardware load counter only has to drain to the stage being
//    consumed).  Block ids (and the valid token count of each block) are
//    staged per wave in LDS up front, so no load waits on a block-table read.
//    The query rows of a segment are loaded once, during the segment's first
//    unit for the wave's first segment and during the previous segment's last
//    unit otherwise, into registers (MFMA B operands); loading them with
//    every unit instead measured 4.7 us slower on llama3_8b (50% more load
//    instructions, all L2 hits).
//  * bf16 queries: scores and P*V on the matrix cores.  The scores come out
//    transposed (S^T = K Q^T, 16x16x32 steps: the block's 16 tokens by 16 score
//    columns, head g of the group in column g*16/GP), so each lane ends with
//    one column's scores for four tokens: after the softmax these are the A
//    operand of O = P V (16x16x16 steps, one per dim of the lane's D/16), with
//    no exchange between lanes.  The output row of head g then lies whole in
//    the lanes of one 16-lane row.  fp32: FMA dot products summed over the 8
//    lanes of a token group by DPP, and P*V by FMA.
//  * Online softmax in the log2 domain with a running max per head that is
//    only raised when a block holds a score more than kRescaleSlack above it
//    (ballot -> uniform branch): the same softmax, with rare accumulator
//    rescales and exp2 <= 2^kRescaleSlack.  Probabilities enter P*V rounded
//    to bf16, and the normaliser sums the same rounded values.
//  * A segment that one wave covers entirely is normalised and written to out.
//    A segment split across waves leaves (max, sum, unnormalised acc) records
//    in the workspace (slot 0: the wave's first segment, slot 1: its last) and
//    the wave holding its first unit notes it; decode_fixup_kernel then merges
//    the records of each noted segment (log-sum-exp).  Merging in a second
//    kernel costs a launch and the gap before it.  Merging in place (records
//    stored at agent scope, an arrival counter per segment, the last part to
//    arrive merging) measured slower on llama3_8b (88.9-92 us against 81.4 us
//    here, with the merge kernel on top: 85-86.6 us per step): 41% of the
//    wave groups hold a part strictly inside one long segment, which ends
//    with the wave's stream, so the store, the arrival and the record loads
//    are round trips after the last unit of the call either way.
//  * Finished segments wait in LDS and are written after the wave's last load:
//    a store in mid-stream would hold up the completion count of the loads
//    issued after it.
//  * Tokens >= n in a sequence's last block are masked (score -inf, V zeroed),
//    so stale slots -- even NaN -- never reach the result.  Sequences with no
//    tokens get zero rows.
//  * Fused append (pa_decode_append): the unit holding a sequence's new token
//    reads that token's K/V rows from the inputs; the merge kernel copies them
//    into the cache afterwards.
//  * FP8 E4M3 caches (KV8 instances): the same kernel on byte caches, the bytes
//    converted exactly to bf16 MFMA operands; see decode_stream_kernel.
#include <hip/hip_ext.h>

#include <type_traits>
#include <utility>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr float kRescaleSlack = 8.0f;  // log2 units: lazy max, exp2 <= 256

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, in order, each with a
// compile-time index (an unrolled loop whatever the body's size).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Finished segments are staged in LDS and written out once the wave's loads are
// done (see the kernel).  A slot holds one segment: a header of 4 words, two
// floats per head, and the wave's sums (GP*D floats; with fewer than 4 heads
// the matrix-core layout leaves lanes without a head, so 4*D).  Slots per wave:
// about 8 KB of LDS, at least 2.
template <int GP, int D>
struct StageGeom {
    static constexpr int kMeta = 4 + 2 * GP;
    static constexpr int kVals = (GP < 4 ? 4 : GP) * D;
    static constexpr int kWords = kMeta + kVals;
    static constexpr int kSlots = (2048 / kVals) > 2 ? (2048 / kVals) : 2;
    static constexpr size_t kBytesPerWave = (size_t)kSlots * kWords * sizeof(float);
};

template <typename T, int D>
struct DecodeGeom {
    static constexpr int kElem = sizeof(T);
    static constexpr int kE = 16 / kElem;            // elements per 16-byte chunk
    static constexpr int kDpl = D / 8;               // dims per lane
    static constexpr int kVecs = kDpl / kE;          // 16-byte chunks per lane per token
    static_assert(kVecs >= 1, "head_dim too small");
    // global dim of element j of chunk c of lane dl
    __device__ static constexpr int dim(int c, int dl, int j) { return c * 8 * kE + dl * kE + j; }
};

// fp32: scores of the lane's two tokens for its GP heads, fully reduced over dims.
template <int GP, int KDPL, int KVECS>
__device__ __forceinline__ void qk_block(float (&sc)[2][GP], const uint4 (&kr)[2][KVECS], const float (&qf)[GP][KDPL]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < KVECS; ++c) {
                a = fmaf(__uint_as_float(kr[t][c].x), qf[g][c * 4 + 0], a);
                a = fmaf(__uint_as_float(kr[t][c].y), qf[g][c * 4 + 1], a);
                a = fmaf(__uint_as_float(kr[t][c].z), qf[g][c * 4 + 2], a);
                a = fmaf(__uint_as_float(kr[t][c].w), qf[g][c * 4 + 3], a);
            }
            sc[t][g] = sum_lanes8(a);
        }
    }
}

// O += P V for one block on the matrix cores (16x16x16 bf16 steps).  Lane
// (q, r) = (lane/16, lane%16) holds, as the A operand, the probabilities of
// score column r for tokens 4q .. 4q+3 (two bf16 pairs: pk), and vw[k], the KW
// words of its KNT = D/16 contiguous dims r*KNT .. of token 4q+k.  Step j
// takes dim j of every lane's dims as B column r, so o[j] receives output rows
// 4q .. 4q+3 (score columns) at dim r*KNT + j.  B needs the four tokens of one
// dim in one lane; v_perm pairs tokens (4q, 4q+1) and (4q+2, 4q+3) of a dim
// (bf16: word w holds dims 2w, 2w+1; fp8: dims 4w .. 4w+3, converted exactly).
template <int KNT, int KW, bool KV8>
__device__ __forceinline__ void pv_mfma(f32x4_t (&o)[KNT], uint2 pk, const uint32_t (&vw)[4][KW]) {
    if constexpr (!KV8) {
        static_assert(KNT == 2 * KW, "bf16: two dims per word");
#pragma unroll
        for (int w = 0; w < KW; ++w) {
            const uint2 ev = make_uint2(__builtin_amdgcn_perm(vw[1][w], vw[0][w], 0x05040100u),
                                        __builtin_amdgcn_perm(vw[3][w], vw[2][w], 0x05040100u));
            const uint2 od = make_uint2(__builtin_amdgcn_perm(vw[1][w], vw[0][w], 0x07060302u),
                                        __builtin_amdgcn_perm(vw[3][w], vw[2][w], 0x07060302u));
            o[2 * w] = mfma16x16x16_bf16(pk, ev, o[2 * w]);
            o[2 * w + 1] = mfma16x16x16_bf16(pk, od, o[2 * w + 1]);
        }
    } else {
        static_assert(KNT == 4 * KW, "fp8: four dims per word");
#pragma unroll
        for (int w = 0; w < KW; ++w) {
            // (token a dim d, token b dim d, token a dim d+1, token b dim d+1)
            const uint32_t lo0 = __builtin_amdgcn_perm(vw[1][w], vw[0][w], 0x05010400u);
            const uint32_t hi0 = __builtin_amdgcn_perm(vw[1][w], vw[0][w], 0x07030602u);
            const uint32_t lo1 = __builtin_amdgcn_perm(vw[3][w], vw[2][w], 0x05010400u);
            const uint32_t hi1 = __builtin_amdgcn_perm(vw[3][w], vw[2][w], 0x07030602u);
            o[4 * w + 0] = mfma16x16x16_bf16(
                pk, make_uint2(fp8x2_to_bf16x2<false>(lo0), fp8x2_to_bf16x2<false>(lo1)), o[4 * w + 0]);
            o[4 * w + 1] = mfma16x16x16_bf16(
                pk, make_uint2(fp8x2_to_bf16x2<true>(lo0), fp8x2_to_bf16x2<true>(lo1)), o[4 * w + 1]);
            o[4 * w + 2] = mfma16x16x16_bf16(
                pk, make_uint2(fp8x2_to_bf16x2<false>(hi0), fp8x2_to_bf16x2<false>(hi1)), o[4 * w + 2]);
            o[4 * w + 3] = mfma16x16x16_bf16(
                pk, make_uint2(fp8x2_to_bf16x2<true>(hi0), fp8x2_to_bf16x2<true>(hi1)), o[4 * w + 3]);
        }
    }
}

// fp32: acc[g][:] += p[0][g] * V[token 0] + p[1][g] * V[token 1]   (the lane's dims)
template <int GP, int KDPL, int KVECS>
__device__ __forceinline__ void pv_block(float (&acc)[GP][KDPL], float (&l)[GP], const float (&p)[2][GP],
                                         const uint4 (&vr)[2][KVECS]) {
#pragma unroll
    for (int g = 0; g < GP; ++g) l[g] += p[0][g] + p[1][g];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int c = 0; c < KVECS; ++c) {
            const float v[4] = {__uint_as_float(vr[t][c].x), __uint_as_float(vr[t][c].y),
                                __uint_as_float(vr[t][c].z), __uint_as_float(vr[t][c].w)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int g = 0; g < GP; ++g) acc[g][c * 4 + j] = fmaf(p[t][g], v[j], acc[g][c * 4 + j]);
            }
        }
    }
}

// A register copy the compiler cannot fold away: the result never shares a
// register with its source, so the source registers are free once it has run.
__device__ __forceinline__ uint32_t opaque_copy(uint32_t x) {
    uint32_t y;
    asm volatile("v_mov_b32 %0, %1" : "=&v"(y) : "v"(x));
    return y;
}

// Pins values in VGPRs at this point in program order: whatever computes them
// must run before it.  Placed after the P*V products of a ring stage, ahead of
// that stage's refill: without it the compiler sinks the products below the
// refill, the refilled V registers then need copies at the loop back edge, and
// each copy waits for its load -- which drains the whole ring once per unit.
template <int GP, int KDPL>
__device__ __forceinline__ void keep_in_regs(float (&acc)[GP][KDPL], float (&l)[GP]) {
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        asm volatile("" : "+v"(l[g]));
#pragma unroll
        for (int d = 0; d < KDPL; ++d) asm volatile("" : "+v"(acc[g][d]));
    }
}

// Reduce-scatter over the 8 token groups (lane bits 3..5) of the lane's
// V = GP*KDPL partial sums, flat index g*KDPL + d.  Each halving step hands
// half of the values to the partner lane and adds what comes back (the
// permlane swaps exchange the upper 32 / odd 16-lane rows of their first
// operand with the lower / even rows of the second), so lane tg ends with the
// complete sums of flat values tg*V/8 .. tg*V/8 + V/8 - 1: 7V/8 exchanges
// instead of 3V for a full all-reduce.
template <int GP, int KDPL>
__device__ __forceinline__ void reduce_scatter8(float (&red)[GP * KDPL / 8], const float (&acc)[GP][KDPL],
                                                int lane) {
    constexpr int V = GP * KDPL;
    static_assert(V % 8 == 0, "reduce-scatter needs 8 | GP*KDPL");
    float h1[V / 2];
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
        const int j = i + V / 2;
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i / KDPL][i % KDPL]),
                                                        __float_as_uint(acc[j / KDPL][j % KDPL]), false, false);
        h1[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    float h2[V / 4];
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(h1[i]), __float_as_uint(h1[i + V / 4]),
                                                        false, false);
        h2[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const bool up8 = (lane & 8) != 0;
#pragma unroll
    for (int i = 0; i < V / 8; ++i) {
        const float keep = up8 ? h2[i + V / 8] : h2[i];
        const float send = up8 ? h2[i] : h2[i + V / 8];
        red[i] = keep + dpp_f32<kDppRowRor8>(send);
    }
}

// Store P consecutive values (times mul) to dst, converted to OutT.
template <typename OutT, int P>
__device__ __forceinline__ void store_piece(OutT* dst, const float* v, float mul) {
    if constexpr (sizeof(OutT) == 2) {
        if constexpr (P == 8) {
            *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(v[0] * mul, v[1] * mul), pack_bf16x2(v[2] * mul, v[3] * mul),
                                                        pack_bf16x2(v[4] * mul, v[5] * mul), pack_bf16x2(v[6] * mul, v[7] * mul));
        } else if constexpr (P == 4) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0] * mul, v[1] * mul), pack_bf16x2(v[2] * mul, v[3] * mul));
        } else if constexpr (P == 2) {
            *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(v[0] * mul, v[1] * mul);
        } else {
            *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16_bits(v[0] * mul);
        }
    } else {
        if constexpr (P == 4) {
            *reinterpret_cast<float4*>(dst) = make_float4(v[0] * mul, v[1] * mul, v[2] * mul, v[3] * mul);
        } else if constexpr (P == 2) {
            *reinterpret_cast<float2*>(dst) = make_float2(v[0] * mul, v[1] * mul);
        } else {
            *reinterpret_cast<float*>(dst) = v[0] * mul;
        }
    }
}

// Store the lane's CH reduced values, elements d0 .. d0+CH-1 of its KDPL dims
// (element d of lane dl is dim (d/KE)*8*KE + dl*KE + d%KE), into row dst.
template <typename OutT, int KE, int CH>
__device__ __forceinline__ void store_run(OutT* dst, const float (&v)[CH], float mul, int d0, int dl) {
    constexpr int kRun = CH < KE ? CH : KE;                        // contiguous dims
    constexpr int kMaxP = 16 / (int)sizeof(OutT);
    constexpr int P = kRun < kMaxP ? kRun : kMaxP;                 // per store
#pragma unroll
    for (int i = 0; i < CH; i += P) {
        const int d = d0 + i;
        store_piece<OutT, P>(dst + (d / KE) * 8 * KE + dl * KE + d % KE, &v[i], mul);
    }
}


// Work is measured in TICKS: every unit costs unit_ticks, and every segment
// adds switch_ticks for the work of closing it (reduction, stores, a fresh
// running max).  pref[s] = blocks of sequences before s and tpref[s] = ticks of
// one head group of every sequence before s, computed by all NT threads of the
// workgroup: per-thread sums over a chunk of sequences, a scan within each
// wave, and one barrier to add the totals of the waves before.  Each context
// length is read from memory once (a thread's loads are all issued before the
// first use) and kept in lens[] for the rest of the kernel; reading it again
// after the barrier would add a dependent round trip to every wave's prologue.
// The first four loads are issued unconditionally (clamped addresses), so the
// wait for each is exact.
template <int NT>
__device__ void prefix_blocks(int* pref, int* tpref, int* lens, int2* wave_tot, const int32_t* __restrict__ ctx,
                              int S, int unit_ticks, int switch_ticks) {
    constexpr int NW = NT / kWave;
    const int t = threadIdx.x;
    const int w = t / kWave;
    const int chunk = (S + NT - 1) / NT;
    const int lo = min(S, t * chunk);
    const int hi = min(S, lo + chunk);
    auto nblk = [&](int n) { return (n + kBlockTokens - 1) / kBlockTokens; };
    auto ticks = [&](int nb) { return nb * unit_ticks + (nb > 0 ? switch_ticks : 0); };
    int sx = 0, sy = 0;
    auto take = [&](int s, int n) {
        lens[s] = n;
        const int nb = nblk(n);
        sx += nb;
        sy += ticks(nb);
    };
    int c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = ctx[min(lo + j, S - 1)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (lo + j < hi) take(lo + j, c[j]);
    }
    for (int s0 = lo + 4; s0 < hi; s0 += 4) {  // more than 4*NT sequences
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = ctx[min(s0 + j, S - 1)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (s0 + j < hi) take(s0 + j, c[j]);
        }
    }
    const int ix = wave_scan_incl(sx), iy = wave_scan_incl(sy);
    if ((t & (kWave - 1)) == kWave - 1) wave_tot[w] = make_int2(ix, iy);
    __syncthreads();
    int ox = 0, oy = 0;
#pragma unroll
    for (int k = 0; k < NW - 1; ++k) {
        if (k < w) {
            ox += wave_tot[k].x;
            oy += wave_tot[k].y;
        }
    }
    int rx = ox + ix - sx, ry = oy + iy - sy;  // exclusive prefix of this thread's chunk
    for (int s = lo; s < hi; ++s) {
        pref[s] = rx;
        tpref[s] = ry;
        const int nb = nblk(lens[s]);
        rx += nb;
        ry += ticks(nb);
    }
    if (t == NT - 1) {
        pref[S] = rx;
        tpref[S] = ry;
    }
}

// Largest s in [lo, hi) with key[s] <= t, for key nondecreasing on [lo, hi)
// and key[lo] <= t.  Wave-uniform: all 64 lanes take part (each step tests
// 64 evenly spaced candidates and keeps the last that passes), so the search
// over S keys costs ceil(log64 S) LDS round trips instead of log2 S.
__device__ __forceinline__ int wave_search(const int* key, int lo, int hi, long long t) {
    const int lane = threadIdx.x & (kWave - 1);
    int n = hi - lo;
    while (n > 1) {
        const int step = (n + kWave - 1) / kWave;
        const bool ok = lane * step < n && (long long)key[lo + lane * step] <= t;
        const uint64_t m = __builtin_amdgcn_ballot_w64(ok);  // lanes 0 .. k pass, lane 0 always
        const int k = 63 - __builtin_clzll(m);
        lo += k * step;
        n = min(step, n - k * step);
    }
    return lo;
}

// Per-lane form: largest s in [lo, hi] with key[s] <= t (key[lo] <= t).
__device__ __forceinline__ int lane_search(const int* key, int lo, int hi, long long t) {
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((long long)key[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// fp32: query rows of the GP heads of head group kvg of sequence s, this lane's dims.
template <int D, int GP, int KDPL>
__device__ __forceinline__ void load_q(float (&qf)[GP][KDPL], const DecodeArgs& a, int s, int kvg, int dl) {
    using G = DecodeGeom<float, D>;
    const int hk = kvg / a.groups_per_kv;
    const int gi0 = (kvg % a.groups_per_kv) * GP;
    const float* qrow = reinterpret_cast<const float*>(a.q) + ((size_t)s * a.num_q_heads + hk * a.group + gi0) * D;
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        // heads past the group (GP > group) reuse the first head's row: their
        // scores are computed but never stored, and the number of loads issued
        // does not depend on the group size
        const int gl = gi0 + g < a.group ? g : 0;
#pragma unroll
        for (int c = 0; c < G::kVecs; ++c) {
            const float4 v = *reinterpret_cast<const float4*>(qrow + (size_t)gl * D + G::dim(c, dl, 0));
            qf[g][c * 4 + 0] = v.x; qf[g][c * 4 + 1] = v.y;
            qf[g][c * 4 + 2] = v.z; qf[g][c * 4 + 3] = v.w;
        }
    }
}

// Range of ticks [start(g), start(g+1)) of wave group g among G groups of T
// ticks.  Tick t lies in the range of group ((t + 1) * G - 1) / T.
__device__ __forceinline__ long long range_start(long long g, long long T, long long G) { return g * T / G; }

// Index (into the concatenated blocks of all sequences) of the first block
// whose first tick is >= t, T ticks in all.  Block blk of sequence s starts at
// tick tpref[s] + blk * R.
__device__ __forceinline__ int block_at_tick(long long t, long long T, const int* pref, const int* tpref, int S,
                                             int R) {
    if (t >= T) return pref[S];
    const int s = wave_search(tpref, 0, S, t);
    const int nb = pref[s + 1] - pref[s];
    const int r = (int)(t - tpref[s]);
    return pref[s] + min((r + R - 1) / R, nb);
}

// KV8: the caches hold FP8 E4M3 (q and out stay T = bf16); dequantized values
// are k_scale * e4m3 and v_scale * e4m3, k_scale folded into scale_log2 and
// v_scale applied when a segment closes.  For the scores lane row q loads the
// 16 bytes at dims 64p + 16q of a key, which feed MFMA steps 2p and 2p+1 (the
// query rows are loaded with the same dim order); V bytes are converted in
// pv_mfma.
template <typename T, int D, int GP, int NW, int STAGES, int WIN, bool KV8>
__global__ __launch_bounds__(NW * kWave) void decode_stream_kernel(DecodeArgs a) {
    using G = DecodeGeom<T, D>;
    using KVT = typename std::conditional<KV8, uint8_t, T>::type;  // cache element
    static_assert(!KV8 || sizeof(T) == 2, "an fp8 cache goes with bf16 queries");
    constexpr int kDpl = G::kDpl;
    constexpr int kVecs = G::kVecs;
    constexpr int kE = G::kE;

    extern __shared__ int smem[];
    __shared__ int2 scan_scratch[NW];
    const int S = a.num_seqs;
    const int S4 = (S + 1 + 3) & ~3;
    int* pref = smem;
    int* tpref = smem + S4;
    int* lens = smem + 2 * S4;  // context lengths
    uint4* tabs = reinterpret_cast<uint4*>(smem + 3 * S4);

    const int R = a.unit_ticks;
    const int C = a.switch_ticks;
    prefix_blocks<NW * kWave>(pref, tpref, lens, scan_scratch, a.context_lens, S, R, C);
    __syncthreads();
    const long long TT = tpref[S];  // ticks of one head group over all sequences
    if (threadIdx.x < kWave) {
        // sequences without tokens get zero rows: wave 0 of every workgroup
        // checks 64 sequences at a time, one per lane
        for (int s0 = blockIdx.x * kWave; s0 < S; s0 += gridDim.x * kWave) {
            const int sl = s0 + (int)threadIdx.x;
            uint64_t em = __builtin_amdgcn_ballot_w64(sl < S && pref[min(sl, S - 1) + 1] == pref[min(sl, S - 1)]);
            while (em != 0) {
                const int j = __builtin_ctzll(em);
                em &= em - 1;
                T* orow = reinterpret_cast<T*>(a.out) + (size_t)(s0 + j) * a.num_q_heads * D;
                for (int i = threadIdx.x; i < a.num_q_heads * D; i += kWave) orow[i] = T(0);
            }
        }
    }
    // wave index, made wave-uniform explicitly: everything the wave decides
    // (ranges, segment walk, branches) derives from it, and the compiler would
    // otherwise treat threadIdx-derived values as per-lane and turn the whole
    // control flow into exec-masked vector code
    // Workgroups are dealt to the 8 XCDs round robin (id mod 8).  Virtual
    // workgroup ids are numbered so that consecutive ones sit on the same XCD:
    // the waves of a wave group, which read the kv-head slices of the same
    // blocks, then go through one L2.
    const int nwg = (int)gridDim.x;
    const int vwg = nwg % 8 == 0 ? (int)(blockIdx.x % 8) * (nwg / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(vwg * NW + threadIdx.x / kWave);
    if (wv >= a.waves) return;  // padding waves of the last workgroup (no barrier follows)
    const int lane = threadIdx.x & (kWave - 1);
    const int hb = a.band_heads;
    const bool band1 = wv >= a.band_groups[0] * hb;
    const int band_wave0 = band1 ? a.band_groups[0] * hb : 0;  // the band's first wave
    const int band_kvg0 = band1 ? hb : 0;                       // the band's first head group
    const long long NG = a.band_groups[band1 ? 1 : 0];          // wave groups of the band
    const int kvg = band_kvg0 + (wv - band_wave0) % hb;         // this wave's head group
    const long long grp = (wv - band_wave0) / hb;               // its wave group in the band
    const int hk = kvg / a.groups_per_kv;        // kv head
    const int gi0 = (kvg % a.groups_per_kv) * GP;  // first query head of the group within the kv head
    const int h0 = hk * a.group + gi0;           // ... among all query heads
    const int nvh = min(GP, a.group - gi0);      // query heads present (the last group may hold fewer)
    const int u_begin = block_at_tick(range_start(grp, TT, NG), TT, pref, tpref, S, R);
    const int u_end = block_at_tick(range_start(grp + 1, TT, NG), TT, pref, tpref, S, R);
    if (u_begin >= u_end) {
        // an empty range (a share smaller than a unit): a zero-weight record in
        // slot 0, in case the wave lies inside a split segment's span of waves
        if (lane < GP) *reinterpret_cast<float2*>(a.ws_ml + ((size_t)wv * 2 * GP + lane) * 2) = make_float2(-INFINITY, 0.f);
        if (lane == 0) a.ws_split[wv].seq = -1;  // no split segment starts here
        return;  // wave-uniform; no barrier follows
    }

    uint4* tab = tabs + (wv % NW) * WIN;
    const int tg = lane >> 3;
    const int dl = lane & 7;
    const int hkv_heads = a.num_kv_heads;
    const uint32_t lane_off = ((uint32_t)tg * hkv_heads) * D + dl * kE;
    const uint32_t tok8_off = 8u * hkv_heads * D;
    const KVT* kbase = reinterpret_cast<const KVT*>(a.k_cache);
    const KVT* vbase = reinterpret_cast<const KVT*>(a.v_cache);

    // consume-side position: sequence, block, blocks in sequence
    int cs = wave_search(pref, 0, S, u_begin);
    int cnb = pref[cs + 1] - pref[cs];
    int cblk = u_begin - pref[cs];
    int seg_first_blk = cblk;
    bool first_seg = true;

    // bf16 queries: both products on the matrix cores.  Lane (mrow, mtok) =
    // (l/16, l%16).  Scores come out transposed, S^T = K Q^T: K is the A
    // operand (row mtok = token mtok of the block), the query rows the B
    // operand, so lane l receives the scores of score column mtok for tokens
    // 4*mrow .. +3 -- exactly the A operand of P*V (pv_mfma) once turned into
    // probabilities, with no exchange between lanes.  Head g of the group sits
    // in score column g*kCs; the other columns carry no head (their
    // probabilities are zero).  P*V row c is score column c, so head g's
    // output lands in rows g*kCs: on lanes with mrow = g*kCs/4, accumulator
    // element g*kCs%4, dims mtok*kNt .. +kNt of the head (every lane holds a
    // whole head at 4 heads or more).
    constexpr bool kMfma = sizeof(T) == 2;
    constexpr int kMf = D / 32;         // score MFMAs per block
    constexpr int kNt = D / 16;         // P*V MFMAs per block = dims per lane
    constexpr int kVw = kNt * (int)sizeof(KVT) / 4;  // dwords of V per lane and token
    constexpr int kCs = 16 / GP;        // score columns per head
    constexpr int kU = GP > 4 ? GP / 4 : 1;  // accumulator elements holding a head
    const int mrow = lane >> 4;
    const int mtok = lane & 15;
    const uint32_t kmf_off = ((uint32_t)mtok * hkv_heads) * D + (KV8 ? 16 : 8) * mrow;
    // this lane's score column holds head mtok / kCs
    const bool real_col = mtok % kCs == 0 && mtok / kCs < nvh;
    // V: tokens 4*mrow + k (k = 0..3), dims mtok*kNt .. +kNt
    const uint32_t vmf_off = ((uint32_t)(4 * mrow) * hkv_heads) * D + (uint32_t)mtok * kNt;
    const uint32_t tok_off = (uint32_t)hkv_heads * D;
    // head of accumulator element u*kCs of this lane (rows 4*mrow + u*kCs), or -1
    auto out_head = [&](int u) -> int {
        const int row = 4 * mrow + (GP > 4 ? u * kCs : 0);
        return row % kCs == 0 && row / kCs < nvh ? row / kCs : -1;
    };

    // Staging of finished segments.  A global store holds up the completion
    // count of every load issued after it until the store itself completes,
    // which under a full read stream takes about as long as a load: a store in
    // mid-stream stalls the ring.  So finished segments wait in LDS and are
    // written after the wave's last load (or when the slots run out).
    using SG = StageGeom<GP, D>;
    constexpr int kCh = kMfma ? kU * kNt : GP * kDpl / 8;  // staged sums per lane
    float* stage = reinterpret_cast<float*>(tabs + NW * WIN) + (wv % NW) * SG::kSlots * SG::kWords;
    int nstaged = 0;
    const int gl = (tg * kCh) / kDpl;  // head of this lane's reduced sums
    const int d0 = (tg * kCh) % kDpl;  // their first element among the lane's dims
    SplitNote note;                    // written at the end
    note.seq = -1;
    note.kvg = kvg;
    note.last_wave = 0;
    note.first_slot = 0;

    auto flush = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int j = 0; j < nstaged; ++j) {
            const float* sl = stage + j * SG::kWords;
            const int kind = __builtin_amdgcn_readfirstlane(__float_as_int(sl[0]));
            const int base = __builtin_amdgcn_readfirstlane(__float_as_int(sl[1]));
            float v[kCh];
#pragma unroll
            for (int i = 0; i < kCh; ++i) v[i] = sl[SG::kMeta + i * kWave + lane];
            if constexpr (kMfma) {
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int h = out_head(u);
                    if (h < 0) continue;
                    const float x = sl[4 + h], y = sl[4 + GP + h];
                    if (kind == 0) {
                        store_piece<T, kNt>(reinterpret_cast<T*>(a.out) + (size_t)(base + h) * D + mtok * kNt,
                                            &v[u * kNt], x);
                    } else {
                        float* dst = a.ws_acc + (size_t)(base + h) * D + mtok * kNt;
#pragma unroll
                        for (int i = 0; i < kNt; i += 4) store_piece<float, 4>(dst + i, &v[u * kNt + i], 1.f);
                        if (mtok == 0) *reinterpret_cast<float2*>(a.ws_ml + (size_t)(base + h) * 2) = make_float2(x, y);
                    }
                }
            } else {
                const float x = sl[4 + gl], y = sl[4 + GP + gl];
                if (gl < nvh) {
                    if (kind == 0) {
                        store_run<T, kE, kCh>(reinterpret_cast<T*>(a.out) + (size_t)(base + gl) * D, v, x, d0, dl);
                    } else {
                        store_run<float, kE, kCh>(a.ws_acc + (size_t)(base + gl) * D, v, 1.f, d0, dl);
                        if (dl == 0 && d0 == 0) *reinterpret_cast<float2*>(a.ws_ml + (size_t)(base + gl) * 2) = make_float2(x, y);
                    }
                }
            }
        }
        nstaged = 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // every counter to zero: the stores above are a variable number, and
        // without a known count after them the compiler's waits for the ring
        // stages would turn conservative everywhere after this point
        __builtin_amdgcn_s_waitcnt(0);
    };

    float qf[GP][kDpl], qnf[GP][kDpl];
    // MFMA path: the B operands of the scores (the group's query rows in
    // their score columns; columns without a head repeat the first head's row,
    // never used) of the current segment, and of the next one, loaded during
    // the last unit of the current segment
    uint4 qm[kMf], qmn[kMf];
    auto load_qm = [&](uint4 (&dst)[kMf], int seq) __attribute__((always_inline)) {
        const uint32_t hi = real_col ? (uint32_t)(mtok / kCs) : 0u;
        const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)seq * a.num_q_heads + h0 + hi) * D;
#pragma unroll
        for (int mm = 0; mm < kMf; ++mm) {
            const int qoff = KV8 ? 64 * (mm / 2) + 16 * mrow + 8 * (mm % 2) : 8 * mrow + 32 * mm;
            dst[mm] = *reinterpret_cast<const uint4*>(qp + qoff);
        }
    };
    if constexpr (kMfma) {
        load_qm(qm, cs);
    } else {
        load_q<D, GP, kDpl>(qf, a, cs, kvg, dl);
    }

    float m[GP], l[GP], acc[GP][kDpl];
    // MFMA path: running max and partial normaliser of this lane's score
    // column (the max is the same on the column's four lanes; the normaliser
    // covers the lane's tokens), and the P*V accumulators
    float mcol = -INFINITY, lcol = 0.f;
    f32x4_t oacc[kNt];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < kDpl; ++i) acc[g][i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < kNt; ++j) oacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 kr[STAGES][2][kVecs], vr[STAGES][2][kVecs];
    uint4 kb4[STAGES][kMf];
    uint32_t vt[STAGES][4][kVw];  // MFMA path: V of tokens 4*mrow + k
    int vld[STAGES];

    auto issue = [&](int st, uint4 e) {
        const uint32_t b = __builtin_amdgcn_readfirstlane(e.x);
        const uint32_t hv = __builtin_amdgcn_readfirstlane(e.y);
        vld[st] = (int)(hv >> 16);
        const size_t base = ((size_t)b * kBlockTokens * hkv_heads + (hv & 0xFFFFu)) * D;
        // with a fused append, the block holding a sequence's new token (e.w =
        // its input row) reads that token's rows from the inputs: the lane
        // choice changes addresses only, never the number of loads
        const uint32_t nrow = __builtin_amdgcn_readfirstlane(e.w);
        const int noff = vld[st] - 1;  // the new token is the block's last valid one
        if constexpr (kMfma) {
            // K: token mtok, 16 bytes per score step; V: tokens 4*mrow + k
            const KVT* kb = kbase + base + kmf_off;
            if (!KV8 && nrow != 0xFFFFFFFFu && mtok == noff)
                kb = reinterpret_cast<const KVT*>(a.new_k) + (size_t)nrow * D + 8 * mrow;
            if constexpr (KV8) {
#pragma unroll
                for (int p = 0; p < kMf / 2; ++p) kb4[st][p] = ldg_nt(kb + 64 * p);
            } else {
#pragma unroll
                for (int mm = 0; mm < kMf; ++mm) kb4[st][mm] = ldg_nt(kb + 32 * mm);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const KVT* vp = vbase + base + vmf_off + k * tok_off;
                if (!KV8 && nrow != 0xFFFFFFFFu && 4 * mrow + k == noff)
                    vp = reinterpret_cast<const KVT*>(a.new_v) + (size_t)nrow * D + mtok * kNt;
                ldg_nt_words<kVw>(vt[st][k], vp);
            }
        } else {
            // K and V rows of the block's two token halves (tokens tg, tg + 8)
            const KVT* vb0 = vbase + base + lane_off;
            const KVT* vb1 = vb0 + tok8_off;
            const KVT* kt0 = kbase + base + lane_off;
            const KVT* kt1 = kt0 + tok8_off;
            if (nrow != 0xFFFFFFFFu) {
                const size_t in_off = (size_t)nrow * D + dl * kE;
                if (tg == noff) {
                    vb0 = reinterpret_cast<const KVT*>(a.new_v) + in_off;
                    kt0 = reinterpret_cast<const KVT*>(a.new_k) + in_off;
                }
                if (tg + 8 == noff) {
                    vb1 = reinterpret_cast<const KVT*>(a.new_v) + in_off;
                    kt1 = reinterpret_cast<const KVT*>(a.new_k) + in_off;
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int c = 0; c < kVecs; ++c) kr[st][t][c] = ldg_nt((t == 0 ? kt0 : kt1) + c * 8 * kE);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int c = 0; c < kVecs; ++c) vr[st][t][c] = ldg_nt((t == 0 ? vb0 : vb1) + c * 8 * kE);
            }
        }
    };

    // Segment (cs, kvg) is done: stage its rows, or a partial record.  MFMA
    // path: each lane holds whole sums (kNt dims of each of its kU heads).
    // fp32: the partial sums are reduce-scattered over the token groups, so
    // lane (tg, dl) ends with kCh complete sums of head gl: elements d0 ..
    // d0+kCh-1 of its dims.
    auto finish_segment = [&]() {
        const bool complete = seg_first_blk == 0 && cblk == cnb - 1;
        const int slot = first_seg ? 0 : 1;
        float red[kCh];
        float* sl = stage + nstaged * SG::kWords;
        if constexpr (kMfma) {
            // the rows of this lane's heads, whole: no reduction across lanes
#pragma unroll
            for (int u = 0; u < kU; ++u) {
#pragma unroll
                for (int j = 0; j < kNt; ++j) red[u * kNt + j] = oacc[j][GP > 4 ? u * kCs : 0];
            }
            if constexpr (KV8) {
#pragma unroll
                for (int i = 0; i < kCh; ++i) red[i] *= a.v_scale;  // dequantized V = v_scale * e4m3
            }
#pragma unroll
            for (int i = 0; i < kCh; ++i) sl[SG::kMeta + i * kWave + lane] = red[i];
            const float lt = sum_rows4(lcol);  // column total, on the column's four lanes
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                const float lg = readlane_f32(lt, g * kCs), mg = readlane_f32(mcol, g * kCs);
                if (lane == 0) {
                    sl[4 + g] = complete ? 1.f / lg : mg;
                    sl[4 + GP + g] = lg;
                }
            }
            mcol = -INFINITY;
            lcol = 0.f;
#pragma unroll
            for (int j = 0; j < kNt; ++j) oacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        } else {
            reduce_scatter8<GP, kDpl>(red, acc, lane);
#pragma unroll
            for (int i = 0; i < kCh; ++i) sl[SG::kMeta + i * kWave + lane] = red[i];
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                const float lt = sum_groups8(l[g]);  // the same on every lane
                if (lane == 0) {
                    sl[4 + g] = complete ? 1.f / lt : m[g];
                    sl[4 + GP + g] = lt;
                }
            }
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                m[g] = -INFINITY;
                l[g] = 0.f;
#pragma unroll
                for (int d = 0; d < kDpl; ++d) acc[g][d] = 0.f;
            }
        }
        if (lane == 0) {
            sl[0] = __int_as_float(complete ? 0 : 1);
            sl[1] = __int_as_float(complete ? cs * a.num_q_heads + h0 : (wv * 2 + slot) * GP);
        }
        ++nstaged;
        if (!complete && seg_first_blk == 0) {
            // this wave holds the segment's first unit: note it for the fix-up,
            // with the wave (same head group) whose group holds the first tick
            // of the segment's last block
            const long long t_last = (long long)tpref[cs] + (long long)(cnb - 1) * R;
            note.seq = cs;
            note.last_wave = band_wave0 + (int)(((t_last + 1) * NG - 1) / TT) * hb + (kvg - band_kvg0);
            note.first_slot = slot;
        }
        first_seg = false;
        if (nstaged == SG::kSlots) flush();  // rare: many short sequences in one range
    };

    for (int wb0 = u_begin; wb0 < u_end; wb0 += WIN) {
        const int wn = min(WIN, u_end - wb0);
        // ---- stage this window's block ids and valid-token counts in LDS
        // (the window's units lie in sequences s_a .. s_b)
        const int s_a = wb0 == u_begin ? cs : wave_search(pref, 0, S, wb0);
        const int s_b = wave_search(pref, s_a, S, wb0 + wn - 1);
        for (int i = lane; i < wn; i += kWave) {
            const int u = wb0 + i;
            const int s = lane_search(pref, s_a, s_b, u);
            const int blk = u - pref[s];
            const int b = a.block_tables[(size_t)s * a.max_blocks_per_seq + blk];
            const int valid = min(kBlockTokens, lens[s] - blk * kBlockTokens);
            // block id; kv head | valid tokens << 16; (unused); input row of
            // the new token if this block holds it (fused append), else ~0
            const bool holds_new = a.new_k != nullptr && blk == pref[s + 1] - pref[s] - 1;
            tab[i] = make_uint4((uint32_t)b, (uint32_t)hk | ((uint32_t)valid << 16), 0u,
                                holds_new ? (uint32_t)(s * a.num_kv_heads + hk) : 0xFFFFFFFFu);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // Every stage is (re)filled on every path -- past the window end with a
        // repeat of its last unit, never consumed -- and scheduling barriers keep
        // each stage's loads together and in ring order.  The number of loads in
        // flight is then the same on all paths, and the compiler's wait counts
        // only wait for the stage being consumed, not for the whole ring.
        static_for<STAGES>([&](auto st) {
            issue(st, tab[min((int)st, wn - 1)]);
            __builtin_amdgcn_sched_barrier(0);
        });
        // One unit: consume ring stage st (window unit ux), then refill it.
        auto unit_step = [&](const int st, const int ux) __attribute__((always_inline)) {
                const int ug = wb0 + ux;
                const bool seg_end = (cblk == cnb - 1) || (ug == u_end - 1);
                // the table entry of the unit this stage is refilled with, read
                // now so that its LDS latency hides behind this unit's work
                const uint4 e_refill = tab[min(ux + STAGES, wn - 1)];
                const bool has_next = seg_end && (ug + 1 < u_end);
                int ns = cs;
                if (has_next) {
                    ++ns;
                    while (pref[ns + 1] == pref[ns]) ++ns;
                    if constexpr (kMfma) {
                        load_qm(qmn, ns);
                    } else {
                        load_q<D, GP, kDpl>(qnf, a, ns, kvg, dl);
                    }
                }

                const int valid = vld[st];
                if constexpr (kMfma) {
                    // ---- scores on the matrix cores, transposed: S^T = K Q^T
                    f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (KV8) {
#pragma unroll
                        for (int p = 0; p < kMf / 2; ++p) {
                            const uint4 r = kb4[st][p];
                            s4 = mfma16x16x32_bf16(fp8x8_to_bf16x8(r.x, r.y), qm[2 * p], s4);
                            s4 = mfma16x16x32_bf16(fp8x8_to_bf16x8(r.z, r.w), qm[2 * p + 1], s4);
                        }
                    } else {
#pragma unroll
                        for (int mm = 0; mm < kMf; ++mm) s4 = mfma16x16x32_bf16(kb4[st][mm], qm[mm], s4);
                    }
                    // V leaves the ring for working registers, and the stage is
                    // refilled at once: the loads of unit ux + STAGES then run
                    // during this unit's softmax and P*V instead of after them.
                    uint32_t vw[4][kVw];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
#pragma unroll
                        for (int w = 0; w < kVw; ++w) vw[k][w] = opaque_copy(vt[st][k][w]);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(s4[r]));
                    __builtin_amdgcn_sched_barrier(0);
                    issue(st, e_refill);
                    __builtin_amdgcn_sched_barrier(0);
                    if (valid < kBlockTokens) {
                        // stale slots past the context: zero their V (may hold NaN)
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            if (4 * mrow + k >= valid) {
#pragma unroll
                                for (int w = 0; w < kVw; ++w) vw[k][w] = 0u;
                            }
                        }
                    }
                    // this lane's scores: column mtok, tokens 4*mrow + i
                    float sv[4];
                    bool need = false;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sv[i] = 4 * mrow + i < valid ? s4[i] * a.scale_log2 : -INFINITY;
                        need |= real_col && sv[i] > mcol + kRescaleSlack;
                    }
                    // ---- lazy running max (rare, uniform branch)
                    if (__builtin_amdgcn_ballot_w64(need) != 0) {
                        const float bm = max_rows4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
                        const float mn = fmaxf(mcol, bm);
                        // 0 when the column's max was -inf; columns without a head keep 1
                        const float alpha = real_col ? fast_exp2(mcol - mn) : 1.f;
                        mcol = mn;
                        lcol *= alpha;
                        // accumulator element i of this lane is output row
                        // 4*mrow + i, i.e. score column 4*mrow + i: its factor
                        // comes from lane 16*mrow + 4*mrow + i
#pragma unroll
                        for (int u = 0; u < kU; ++u) {
                            const int i = GP > 4 ? u * kCs : 0;
                            const float ar = __int_as_float(
                                __builtin_amdgcn_ds_bpermute((20 * mrow + i) * 4, __float_as_int(alpha)));
#pragma unroll
                            for (int jt = 0; jt < kNt; ++jt) oacc[jt][i] *= ar;
                        }
                    }
                    // ---- probabilities of the lane's four tokens: the A operand of P*V
                    float pr[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) pr[i] = real_col ? fast_exp2(sv[i] - mcol) : 0.f;
                    const uint2 pk = make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
                    lcol = dot2_bf16(pk.x, 0x3F803F80u, lcol);  // + the rounded probabilities
                    lcol = dot2_bf16(pk.y, 0x3F803F80u, lcol);
                    pv_mfma<kNt, kVw, KV8>(oacc, pk, vw);
                } else {
                    if (valid < kBlockTokens) {
                        // stale slots past the context: zero their V (may hold NaN)
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            if (tg + 8 * t >= valid) {
#pragma unroll
                                for (int c = 0; c < kVecs; ++c) vr[st][t][c] = make_uint4(0, 0, 0, 0);
                            }
                        }
                    }
                    // ---- scores of this block
                    float sc[2][GP];
                    qk_block<GP, kDpl, kVecs>(sc, kr[st], qf);
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
#pragma unroll
                        for (int g = 0; g < GP; ++g) sc[t][g] = tg + 8 * t < valid ? sc[t][g] * a.scale_log2 : -INFINITY;
                    }
                    // ---- lazy running max, probabilities, P*V
                    bool need = false;
#pragma unroll
                    for (int g = 0; g < GP; ++g) need |= fmaxf(sc[0][g], sc[1][g]) > m[g] + kRescaleSlack;
                    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
                        for (int g = 0; g < GP; ++g) {
                            const float bm = max_groups8(fmaxf(sc[0][g], sc[1][g]));
                            const float mn = fmaxf(m[g], bm);
                            const float alpha = fast_exp2(m[g] - mn);  // 0 when m was -inf
                            l[g] *= alpha;
#pragma unroll
                            for (int d = 0; d < kDpl; ++d) acc[g][d] *= alpha;
                            m[g] = mn;
                        }
                    }
                    float p[2][GP];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
#pragma unroll
                        for (int g = 0; g < GP; ++g) p[t][g] = fast_exp2(sc[t][g] - m[g]);
                    }
                    pv_block<GP, kDpl, kVecs>(acc, l, p, vr[st]);
                    // ---- refill this stage (unconditionally, see above), once
                    // its registers are no longer read
                    keep_in_regs<GP, kDpl>(acc, l);
                    __builtin_amdgcn_sched_barrier(0);
                    issue(st, e_refill);
                    __builtin_amdgcn_sched_barrier(0);
                }

                if (!seg_end) {
                    ++cblk;
                    return;
                }
                finish_segment();
                if (has_next) {
                    cs = ns;
                    cblk = 0;
                    cnb = pref[cs + 1] - pref[cs];
                    seg_first_blk = 0;
                    if constexpr (kMfma) {
#pragma unroll
                        for (int mm = 0; mm < kMf; ++mm) qm[mm] = qmn[mm];
                    } else {
#pragma unroll
                        for (int g = 0; g < GP; ++g) {
#pragma unroll
                            for (int i = 0; i < kDpl; ++i) qf[g][i] = qnf[g][i];
                        }
                    }
                }
        };
        // Whole rounds of the ring, with no exit inside a round: on every path
        // through the loop the stages are consumed and refilled in ring order,
        // so the compiler's load-counter waits at a stage only cover that
        // stage's loads.  (A conditional exit between stages gives the wait
        // placement paths on which a later stage's loads look the most recent,
        // and it then waits for the whole ring before every unit.)
        int x = 0;
        for (; x + STAGES <= wn; x += STAGES) {
            static_for<STAGES>([&](auto st) { unit_step(st, x + st); });
        }
        // the last wn % STAGES units of the window
        static_for<STAGES - 1>([&](auto st) {
            if (x + st < wn) unit_step(st, x + st);
        });
    }
    flush();
    if (lane == 0) a.ws_split[wv] = note;
}

// Merge the partial records of the split segment noted by wave w (if any):
//   M = max_v m_v,  L = sum_v l_v 2^(m_v - M),  out = sum_v acc_v 2^(m_v - M) / L
// over the waves v = w, w + band_heads, ..., last_wave (the waves of the
// segment's head group in consecutive wave groups of its band) that hold its
// units, folded in record
// order with a running maximum.  One workgroup per noting wave, one wave per
// head.  The note is one memory round trip; the (max, sum) pairs and sums of up
// to kBatch records are then loaded together, so a merge of up to kBatch parts
// costs two dependent round trips.  Segments of more than kLongMin parts (a
// long context spread over many waves) take a two-pass merge instead: the
// (max, sum) pairs of every part at once, then the sums kLongBatch parts at a
// time with precomputed weights.  In the fused call the workgroup first
// copies new K/V rows into the cache (see below).  Records of zero weight (m = -inf: waves
// whose range was empty) are skipped without touching their sums.
//
// Workgroup b merges for wave w = (b mod 8) * waves/8 + b/8: workgroups are
// dealt to the XCDs round robin (b mod 8), and the streaming kernel placed
// waves [x*waves/8, (x+1)*waves/8) on XCD x, so the note and most records are
// read on the XCD that wrote them (measured on MI355X: 0.4-0.8 us off a
// decode step).  The row copies stay dealt by b, spread over all XCDs.
template <typename T, int D, int GP>
__global__ __launch_bounds__(GP * kWave) void decode_fixup_kernel(DecodeArgs a) {
    constexpr int kPerLane = D / kWave;  // 1 or 2
    constexpr int kBatch = 8;
    constexpr int kLongMin = 16;     // segments of more parts, up to kLongChunks * 64,
    constexpr int kLongChunks = 4;   // take the two-pass merge
    constexpr int kLongBatch = 32;   // sums loaded together in the two-pass merge (divides kWave)
    const int nb = (int)gridDim.x;  // = a.waves
    const int w = nb % 8 == 0 ? (int)(blockIdx.x % 8) * (nb / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const SplitNote sn = a.ws_split[w];
    const int gi0 = sn.seq >= 0 ? (sn.kvg % a.groups_per_kv) * GP : 0;
    const bool merging = sn.seq >= 0 && gi0 + g < a.group;
    const int hb = a.band_heads;
    const int nrec = merging ? (sn.last_wave - w) / hb + 1 : 1;  // waves w, w + hb, ..., last_wave
    auto rec_of = [&](int j) __attribute__((always_inline)) -> size_t {  // record of wave w + j * hb, head g
        return ((size_t)(w + j * hb) * 2 + (j == 0 ? sn.first_slot : 0)) * GP + g;
    };
    // lane b loads the (max, sum) of record j0 + b (one vector load for the
    // batch), every lane its kPerLane sums of each record; records past nrec
    // repeat the last one and get zero weight, so every load is used and all
    // are issued before the first wait
    float2 mlv;
    float x[kBatch][kPerLane];
    auto load_batch = [&](int j0) __attribute__((always_inline)) {
        mlv = *reinterpret_cast<const float2*>(a.ws_ml + rec_of(min(j0 + (lane & (kBatch - 1)), nrec - 1)) * 2);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const size_t r = rec_of(min(j0 + b, nrec - 1));
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) x[b][i] = a.ws_acc[r * D + lane * kPerLane + i];
        }
    };
    // the two-pass merge (below) for segments of many parts
    const bool long_merge = merging && nrec > kLongMin && nrec <= kLongChunks * kWave;
    float2 mlc[kLongChunks];
    if (long_merge) {
        // (max, sum) of record j in lane j % 64 of chunk j / 64, all loaded together
#pragma unroll
        for (int c = 0; c < kLongChunks; ++c) {
            const int j = c * kWave + lane;
            mlc[c] = make_float2(-INFINITY, 0.f);
            if (c * kWave < nrec) {  // uniform
                const float2 v = *reinterpret_cast<const float2*>(a.ws_ml + rec_of(min(j, nrec - 1)) * 2);
                if (j < nrec) mlc[c] = v;
            }
        }
    } else if (merging) {
        load_batch(0);
    }
    // either is in flight while the copy below resolves its slot

    if (a.new_k != nullptr) {
        // Fused KV append: the new token's K/V rows of sequence b (and b +
        // gridDim.x, ...) go to their cache slots (position N-1).  The streaming
        // kernel took those rows from the inputs, so the copies only have to be
        // done by the end of the call.  The rows and the context length load
        // together with the records above; the copy adds the block-table read.
        constexpr int kRowVecsPerHead = D * (int)sizeof(T) / 16;
        // four vectors per thread and chunk, in named registers (an array
        // here would be placed in memory before the loops are unrolled)
        const int row_vecs = a.num_kv_heads * kRowVecsPerHead;
        const int bd = (int)blockDim.x;
        const int chunk = 4 * bd;  // one chunk at the configurations' shapes
        for (int sq = (int)blockIdx.x; sq < a.num_seqs; sq += gridDim.x) {
            const uint4* ksrc = reinterpret_cast<const uint4*>(a.new_k) + (size_t)sq * row_vecs;
            const uint4* vsrc = reinterpret_cast<const uint4*>(a.new_v) + (size_t)sq * row_vecs;
            for (int c0 = 0; c0 < row_vecs; c0 += chunk) {
                const int i0 = c0 + (int)threadIdx.x, i1 = i0 + bd, i2 = i1 + bd, i3 = i2 + bd;
                const int last = row_vecs - 1;
                const uint4 k0 = ksrc[min(i0, last)], k1 = ksrc[min(i1, last)];
                const uint4 k2 = ksrc[min(i2, last)], k3 = ksrc[min(i3, last)];
                const uint4 v0 = vsrc[min(i0, last)], v1 = vsrc[min(i1, last)];
                const uint4 v2 = vsrc[min(i2, last)], v3 = vsrc[min(i3, last)];
                const int nq = a.context_lens[sq];
                if (nq <= 0) break;
                const int bq = a.block_tables[(size_t)sq * a.max_blocks_per_seq + (nq - 1) / kBlockTokens];
                const size_t slot = (size_t)bq * kBlockTokens + (nq - 1) % kBlockTokens;
                uint4* kdst = reinterpret_cast<uint4*>(a.k_cache_w) + slot * row_vecs;
                uint4* vdst = reinterpret_cast<uint4*>(a.v_cache_w) + slot * row_vecs;
                if (i0 < row_vecs) { kdst[i0] = k0; vdst[i0] = v0; }
                if (i1 < row_vecs) { kdst[i1] = k1; vdst[i1] = v1; }
                if (i2 < row_vecs) { kdst[i2] = k2; vdst[i2] = v2; }
                if (i3 < row_vecs) { kdst[i3] = k3; vdst[i3] = v3; }
            }
        }
    }
    if (!merging) return;

    const int hk = sn.kvg / a.groups_per_kv;
    float M = -INFINITY, L = 0.f, o[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) o[i] = 0.f;
    if (long_merge) {
        // A segment of many parts (a long context over many waves): the
        // (max, sum) pairs of all its records came first; their maximum and
        // the normaliser are wave reductions, and each record's weight
        // 2^(m - M) / L stays in its lane.  The sums are then loaded
        // kLongBatch records at a time and added with those weights: a few
        // round trips in all instead of one per kBatch records, and no
        // dependency from one record to the next.
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < kLongChunks; ++c) mx = fmaxf(mx, mlc[c].x);
        M = wave_max64(mx);  // finite: the noting wave's own part holds units
        float ls = 0.f;
        float wgt[kLongChunks];
#pragma unroll
        for (int c = 0; c < kLongChunks; ++c) {
            wgt[c] = mlc[c].x != -INFINITY ? fast_exp2(mlc[c].x - M) : 0.f;  // zero-weight records stay 0
            ls += mlc[c].y * wgt[c];
        }
        L = wave_sum64(ls);
        const float invl = 1.f / L;
#pragma unroll
        for (int c = 0; c < kLongChunks; ++c) wgt[c] *= invl;
        float xs[kLongBatch][kPerLane];
        for (int j0 = 0; j0 < nrec; j0 += kLongBatch) {
#pragma unroll
            for (int b = 0; b < kLongBatch; ++b) {
                const size_t r = rec_of(min(j0 + b, nrec - 1));
#pragma unroll
                for (int i = 0; i < kPerLane; ++i) xs[b][i] = a.ws_acc[r * D + lane * kPerLane + i];
            }
            const int c = j0 / kWave;  // kLongBatch divides kWave: one chunk per batch
            float wc = wgt[0];
#pragma unroll
            for (int k = 1; k < kLongChunks; ++k) wc = c == k ? wgt[k] : wc;
#pragma unroll
            for (int b = 0; b < kLongBatch; ++b) {
                const float wb = readlane_f32(wc, (j0 % kWave) + b);  // 0 past the segment
                // a zero weight skips the record's sums (never written for empty ranges)
#pragma unroll
                for (int i = 0; i < kPerLane; ++i) o[i] = wb != 0.f ? fmaf(xs[b][i], wb, o[i]) : o[i];
            }
        }
        L = 1.f;  // the weights carried 1 / L
    } else {
      for (int j0 = 0; j0 < nrec; j0 += kBatch) {
        if (j0 > 0) load_batch(j0);
        float2 ml[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) ml[b] = make_float2(readlane_f32(mlv.x, b), readlane_f32(mlv.y, b));
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const bool live = j0 + b < nrec && ml[b].x != -INFINITY;
            const float mn = live ? fmaxf(M, ml[b].x) : M;
            const float ca = live ? fast_exp2(M - mn) : 1.f;  // 0 while M is -inf
            const float cb = live ? fast_exp2(ml[b].x - mn) : 0.f;
            L = L * ca + (live ? ml[b].y * cb : 0.f);
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) o[i] = o[i] * ca + (live ? x[b][i] * cb : 0.f);
            M = mn;
        }
      }
    }
    const float inv = 1.f / L;
    T* orow = reinterpret_cast<T*>(a.out) + ((size_t)sn.seq * a.num_q_heads + hk * a.group + gi0 + g) * D +
              lane * kPerLane;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        if constexpr (sizeof(T) == 2) {
            reinterpret_cast<uint16_t*>(orow)[i] = f32_to_bf16_bits(o[i] * inv);
        } else {
            reinterpret_cast<float*>(orow)[i] = o[i] * inv;
        }
    }
}

// ---------------------------------------------------------------- launchers
template <int GP, int D>
static size_t decode_stream_lds_bytes(int num_seqs) {
    return 3 * (size_t)((num_seqs + 1 + 3) & ~3) * sizeof(int) +
           (size_t)kDecodeWaves * kDecodeWindow * sizeof(uint4) +
           (size_t)kDecodeWaves * StageGeom<GP, D>::kBytesPerWave;
}

// Events, when given, take the kernel's own start and stop times from its
// dispatch (hipExtLaunchKernel): no extra packets on the stream.
template <typename T, int D, int GP, int STAGES, bool KV8>
static hipError_t launch_stream(const DecodeArgs& a, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
    const size_t lds = decode_stream_lds_bytes<GP, D>(a.num_seqs);
    const dim3 grid((a.waves + kDecodeWaves - 1) / kDecodeWaves), block(kDecodeWaves * kWave);
    auto kernel = decode_stream_kernel<T, D, GP, kDecodeWaves, STAGES, kDecodeWindow, KV8>;
    if (ev_start || ev_stop) {
        DecodeArgs arg = a;
        void* args[] = {&arg};
        return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, lds, stream, ev_start,
                                  ev_stop, 0);
    }
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, a);
    return hipGetLastError();
}

template <typename T, int D, int GP>
static hipError_t launch_decode_g(const DecodeArgs& a, int stages, bool kv8, hipStream_t stream, hipEvent_t ev_start,
                                  hipEvent_t ev_stop) {
    hipError_t e;
    if (kv8) {
        if constexpr (sizeof(T) == 2) {
            switch (stages) {
                case 2: e = launch_stream<T, D, GP, 2, true>(a, stream, ev_start, ev_stop); break;
                case 3: e = launch_stream<T, D, GP, 3, true>(a, stream, ev_start, ev_stop); break;
                case 6: e = launch_stream<T, D, GP, 6, true>(a, stream, ev_start, ev_stop); break;
                case 8: e = launch_stream<T, D, GP, 8, true>(a, stream, ev_start, ev_stop); break;
                default: e = launch_stream<T, D, GP, 4, true>(a, stream, ev_start, ev_stop); break;
            }
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        switch (stages) {
            case 3: e = launch_stream<T, D, GP, 3, false>(a, stream, ev_start, ev_stop); break;
            case 4: e = launch_stream<T, D, GP, 4, false>(a, stream, ev_start, ev_stop); break;
            default: e = launch_stream<T, D, GP, 2, false>(a, stream, ev_start, ev_stop); break;
        }
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_fixup_kernel<T, D, GP>), dim3(a.waves), dim3(GP * kWave), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_d(const DecodeArgs& a, int gp, int stages, bool kv8, hipStream_t stream,
                                  hipEvent_t e0, hipEvent_t e1) {
    switch (gp) {
        case 1: return launch_decode_g<T, D, 1>(a, stages, kv8, stream, e0, e1);
        case 2: return launch_decode_g<T, D, 2>(a, stages, kv8, stream, e0, e1);
        case 4: return launch_decode_g<T, D, 4>(a, stages, kv8, stream, e0, e1);
        default: return launch_decode_g<T, D, 8>(a, stages, kv8, stream, e0, e1);
    }
}

hipError_t launch_decode(const DecodeArgs& a, int dtype_bf16, int head_dim, int gp, int stages, bool kv8,
                         hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
    if (dtype_bf16) {
        return head_dim == 64 ? launch_decode_d<uint16_t, 64>(a, gp, stages, kv8, stream, e0, e1)
                              : launch_decode_d<uint16_t, 128>(a, gp, stages, kv8, stream, e0, e1);
    }
    if (kv8) return hipErrorInvalidValue;
    return head_dim == 64 ? launch_decode_d<float, 64>(a, gp, stages, false, stream, e0, e1)
                          : launch_decode_d<float, 128>(a, gp, stages, false, stream, e0, e1);
}

}  // namespace pa
