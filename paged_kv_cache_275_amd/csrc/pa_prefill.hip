// pa_prefill.hip -- causal chunked prefill over the paged KV cache (gfx950, bf16).
//
// What is computed: sequence s owns query rows query_start_loc[s] .. +c-1, its c
// newest tokens (already appended to the cache).  Row i sits at absolute
// position p = context_lens[s] - c + i and attends to the tokens 0..p of its
// sequence, each found through the block table -- exact softmax attention,
// the same formula as decode.  Prefill processes a prompt's tokens together
// (page "从零实现一个 mini vLLM--开篇", section "2. LLM 推理到底在慢什么");
// chunked prefill is named in its section 5, stage six; the position reading
// above is this library's.
//
// How (MI355X design): a dense contraction, so both products run on the
// matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//  * A workgroup owns one kv head and RT consecutive query rows of one sequence;
//    its COLS = RT * GP columns are (query row, head) pairs, all heads of the
//    GQA group side by side, so every K/V tile staged in LDS serves the whole
//    group.  Wave w owns CT tiles of 16 columns.
//  * Keys stream through LDS in tiles of 64 (four 16-token blocks, resolved
//    through the block table).  K is stored row-major; V is stored transposed
//    (V^T[dim][key]) so that it can be an MFMA A operand.  The next tile's
//    global loads are issued before the current tile is computed.
//  * Scores are computed transposed, S^T = K Q^T: lane l then holds column l%16
//    and keys 4*(l/16) .. +3 of each 16-key subtile.  Row maxima and sums are
//    per-lane work plus two lane swaps, and the probabilities of two subtiles
//    are, unchanged, the B operand of O^T = V^T P^T for a 32-key step (k-slots
//    8g .. 8g+7 of lane group g are keys 4g .. 4g+3 of the first subtile and of
//    the second; V^T is read with the same key order).
//  * Online softmax per column in the log2 domain; keys past a row's position,
//    and past the context, are masked (score -inf, V zero).
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <int D, int GP, int NW, int CT>
__global__ __launch_bounds__(NW * kWave) void prefill_kernel(PrefillArgs a) {
    constexpr int kCols = NW * 16 * CT;  // (row, head) columns per workgroup
    constexpr int kRT = kCols / GP;      // query rows per workgroup
    constexpr int kKT = 64;              // keys per tile
    constexpr int kKP = D + 8;           // K row pitch in LDS (elements)
    constexpr int kVP = kKT + 8;         // V^T row pitch in LDS (elements)
    constexpr int kMs = D / 32;          // MFMA k-steps over dims
    constexpr int kDt = D / 16;          // 16-dim tiles of the output
    constexpr int kNT = NW * kWave;
    constexpr int kKChunks = kKT * D / 8 / kNT;  // 16-byte K chunks per thread per tile
    constexpr int kVBlocks = kKT / 4 * (D / 8);  // 4-key x 8-dim V blocks per tile
    static_assert(kKChunks >= 1 && kKChunks * kNT == kKT * D / 8, "K staging must cover the tile");
    static_assert(kVBlocks <= kNT, "V staging assumes at most one block per thread");

    __shared__ __align__(16) uint16_t k_lds[kKT * kKP];
    __shared__ __align__(16) uint16_t vt_lds[D * kVP];

    const int hk = blockIdx.y;
    // ---- which sequence and row tile: flat enumeration over sequences
    int s = 0, tile = blockIdx.x, r0 = 0, c = 0;
    for (; s < a.num_seqs; ++s) {
        r0 = a.query_start_loc[s];
        c = a.query_start_loc[s + 1] - r0;
        const int nt = (c + kRT - 1) / kRT;
        if (tile < nt) break;
        tile -= nt;
    }
    if (s >= a.num_seqs) return;  // uniform: grid is an upper bound
    const int n = a.context_lens[s];
    const int i0 = tile * kRT;
    const int rows = min(kRT, c - i0);
    const int pos0 = n - c + i0;           // position of the workgroup's first row
    const int pmax = pos0 + rows - 1;      // last key any row needs
    const int ntiles = pmax / kKT + 1;
    const int32_t* bt = a.block_tables + (size_t)s * a.max_blocks_per_seq;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lg = lane >> 4;    // lane group: k-slots 8*lg .. +8, output rows 4*lg .. +3
    const int lc = lane & 15;    // column within a 16-column tile
    const int hkv_heads = a.num_kv_heads;
    const uint16_t* kcache = reinterpret_cast<const uint16_t*>(a.k_cache);
    const uint16_t* vcache = reinterpret_cast<const uint16_t*>(a.v_cache);

    // ---- this lane's columns: query row and head, causal limit, Q^T operands
    int col_row[CT], col_head[CT], col_pos[CT];
    uint4 qb[CT][kMs];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int col = (w * CT + ct) * 16 + lc;
        const int i = col / GP;
        const int g = col % GP;
        col_row[ct] = i;
        col_head[ct] = g;
        col_pos[ct] = pos0 + i;
        // rows past the chunk and heads past the group read a valid row; their
        // results are never stored
        const int ii = i0 + i < c ? i : 0;
        const int gg = g < a.group ? g : 0;
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) +
                               ((size_t)(r0 + i0 + ii) * a.num_q_heads + hk * a.group + gg) * D + 8 * lg;
#pragma unroll
        for (int m = 0; m < kMs; ++m) qb[ct][m] = *reinterpret_cast<const uint4*>(qrow + 32 * m);
    }

    f32x4_t o[CT][kDt];
    float mrun[CT], lrun[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        mrun[ct] = -INFINITY;
        lrun[ct] = 0.f;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) o[ct][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // ---- staging: K chunks (key, 16-byte chunk) and one 4-key x 8-dim V block
    uint4 kreg[kKChunks], vreg[4];
    const int v_kg = tid / (D / 8);   // keys 4*v_kg .. +3 of the tile
    const int v_dc = tid % (D / 8);   // dims 8*v_dc .. +7
    auto load_tile = [&](int t) {
        const int t0 = t * kKT;
#pragma unroll
        for (int j = 0; j < kKChunks; ++j) {
            const int q = tid + j * kNT;
            const int key = q / (D / 8);
            const int ch = q % (D / 8);
            const int tok = t0 + key;
            if (tok < n) {
                const int b = bt[tok / kBlockTokens];
                kreg[j] = *reinterpret_cast<const uint4*>(
                    kcache + (((size_t)b * kBlockTokens + tok % kBlockTokens) * hkv_heads + hk) * D + ch * 8);
            } else {
                kreg[j] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tok = t0 + 4 * v_kg + e;
            if (tid < kVBlocks && tok < n) {
                const int b = bt[tok / kBlockTokens];
                vreg[e] = *reinterpret_cast<const uint4*>(
                    vcache + (((size_t)b * kBlockTokens + tok % kBlockTokens) * hkv_heads + hk) * D + v_dc * 8);
            } else {
                vreg[e] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int j = 0; j < kKChunks; ++j) {
            const int q = tid + j * kNT;
            *reinterpret_cast<uint4*>(&k_lds[(q / (D / 8)) * kKP + (q % (D / 8)) * 8]) = kreg[j];
        }
        if (tid >= kVBlocks) return;
        // transpose the 4 keys x 8 dims block: dim e gets (k0, k1, k2, k3)
        const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
        const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
        const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
        const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // even dim 2j: low halves; odd dim 2j+1: high halves
            const uint2 ev = make_uint2(__builtin_amdgcn_perm(w1[j], w0[j], 0x05040100u),
                                        __builtin_amdgcn_perm(w3[j], w2[j], 0x05040100u));
            const uint2 od = make_uint2(__builtin_amdgcn_perm(w1[j], w0[j], 0x07060302u),
                                        __builtin_amdgcn_perm(w3[j], w2[j], 0x07060302u));
            *reinterpret_cast<uint2*>(&vt_lds[(v_dc * 8 + 2 * j) * kVP + 4 * v_kg]) = ev;
            *reinterpret_cast<uint2*>(&vt_lds[(v_dc * 8 + 2 * j + 1) * kVP + 4 * v_kg]) = od;
        }
    };

    load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();  // the previous tile is no longer being read
        store_tile();
        __syncthreads();
        if (t + 1 < ntiles) load_tile(t + 1);
        const int t0 = t * kKT;

        // ---- S^T = K Q^T for the four 16-key subtiles
        f32x4_t sacc[4][CT];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) sacc[sb][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < kMs; ++m) {
                const uint4 ka = *reinterpret_cast<const uint4*>(&k_lds[(sb * 16 + lc) * kKP + 32 * m + 8 * lg]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) sacc[sb][ct] = mfma16x16x32_bf16(ka, qb[ct][m], sacc[sb][ct]);
            }
        }
        // ---- online softmax per column
        uint4 pb[CT][2];  // B operands of the two 32-key P*V steps
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            float sv[4][4];
            float tmax = -INFINITY;
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = t0 + sb * 16 + 4 * lg + r;
                    const float x = key <= col_pos[ct] ? sacc[sb][ct][r] * a.scale_log2 : -INFINITY;
                    sv[sb][r] = x;
                    tmax = fmaxf(tmax, x);
                }
            }
            // the column's keys live in lanes lc, lc+16, lc+32, lc+48
            {
                auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
                tmax = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
                auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
                tmax = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
            }
            const float mn = fmaxf(mrun[ct], tmax);
            const float alpha = mn == -INFINITY ? 1.f : fast_exp2(mrun[ct] - mn);
            mrun[ct] = mn;
            float psum = 0.f;
            float pv[4][4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pv[sb][r] = mn == -INFINITY ? 0.f : fast_exp2(sv[sb][r] - mn);
                    psum += pv[sb][r];
                }
            }
            lrun[ct] = lrun[ct] * alpha + psum;
#pragma unroll
            for (int dt = 0; dt < kDt; ++dt) o[ct][dt] *= alpha;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                pb[ct][kk] = make_uint4(pack_bf16x2(pv[2 * kk][0], pv[2 * kk][1]),
                                        pack_bf16x2(pv[2 * kk][2], pv[2 * kk][3]),
                                        pack_bf16x2(pv[2 * kk + 1][0], pv[2 * kk + 1][1]),
                                        pack_bf16x2(pv[2 * kk + 1][2], pv[2 * kk + 1][3]));
            }
        }
        // ---- O^T += V^T P^T (32 keys per step)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int dt = 0; dt < kDt; ++dt) {
                const uint16_t* vrow = &vt_lds[(dt * 16 + lc) * kVP + 32 * kk + 4 * lg];
                const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
                const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
                const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) o[ct][dt] = mfma16x16x32_bf16(va, pb[ct][kk], o[ct][dt]);
            }
        }
    }

    // ---- normalise and store: lane holds column lc, dims dt*16 + 4*lg .. +3
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        float lt = lrun[ct];
        {
            auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(lt), __float_as_uint(lt), false, false);
            lt = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
            auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lt), __float_as_uint(lt), false, false);
            lt = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
        }
        const int i = col_row[ct];
        const int g = col_head[ct];
        if (i0 + i >= c || g >= a.group) continue;
        const float inv = 1.f / lt;
        uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) +
                         ((size_t)(r0 + i0 + i) * a.num_q_heads + hk * a.group + g) * D + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) {
            const f32x4_t x = o[ct][dt];
            *reinterpret_cast<uint2*>(orow + dt * 16) =
                make_uint2(pack_bf16x2(x[0] * inv, x[1] * inv), pack_bf16x2(x[2] * inv, x[3] * inv));
        }
    }
}

// ---------------------------------------------------------------- launchers
template <int D, int GP>
static hipError_t launch_prefill_g(const PrefillArgs& a, int total_rows, hipStream_t stream) {
    constexpr int kNW = 4, kCT = 2;
    constexpr int kRT = kNW * 16 * kCT / GP;
    const long long tiles = (long long)total_rows / kRT + a.num_seqs;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_kernel<D, GP, kNW, kCT>), dim3((unsigned)tiles, a.num_kv_heads),
                       dim3(kNW * kWave), 0, stream, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, int total_rows, int gp, hipStream_t stream) {
    switch (gp) {
        case 1: return launch_prefill_g<D, 1>(a, total_rows, stream);
        case 2: return launch_prefill_g<D, 2>(a, total_rows, stream);
        case 4: return launch_prefill_g<D, 4>(a, total_rows, stream);
        case 8: return launch_prefill_g<D, 8>(a, total_rows, stream);
        default: return launch_prefill_g<D, 16>(a, total_rows, stream);
    }
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int total_rows, int gp, hipStream_t stream) {
    return head_dim == 64 ? launch_prefill_d<64>(a, total_rows, gp, stream)
                          : launch_prefill_d<128>(a, total_rows, gp, stream);
}

}  // namespace pa
