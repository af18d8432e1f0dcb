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
//  * Work unit = one workgroup of NW waves per (sequence, kv head, head group,
//    partition of PART = NW*BPW*16 tokens).  Each wave owns BPW consecutive
//    logical blocks of the partition and ALL query heads (up to GP) that share
//    the kv head, so every K/V byte is loaded from HBM exactly once and reused
//    from registers by the whole GQA group.
//  * Lane layout inside a wave for one 16-token block: lane = 8*tg + dl.
//    Token group tg (0..7) owns tokens tg and tg+8 of the block, dl (0..7) owns
//    head_dim/8 consecutive dims.  One token's row of one kv head is
//    head_dim*elem bytes, read by 8 lanes as 16-byte loads; the loads for a
//    whole chunk of blocks are issued before any of them is consumed.
//  * Scores: v_dot2_f32_bf16 partial dot products, then a sum over the 8 lanes
//    of a token group with three DPP adds.
//  * Online softmax in the log2 domain with a wave-uniform running max per
//    head.  The max is only raised when a block holds a score more than
//    kRescaleSlack above it (a ballot decides, so the branch is uniform): the
//    result is the same softmax, the rescale of the accumulators becomes rare,
//    and exp2 never exceeds 2^kRescaleSlack.
//  * P*V: probabilities packed to bf16 pairs (token tg, token tg+8) and V
//    re-paired by v_perm so that one v_dot2 adds both tokens' contributions.
//    The normaliser l is accumulated from the same rounded probabilities.
//  * End of a work unit: token groups and waves are merged through LDS.  A
//    sequence that fits one partition is written to out directly; otherwise the
//    partition's (max, sum, unnormalised acc) go to the workspace and
//    decode_reduce_kernel merges the partitions (log-sum-exp).
//  * Tokens >= n in a sequence's last block are masked (score -inf and V
//    zeroed), so stale slots -- even NaN -- never reach the result.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr float kRescaleSlack = 8.0f;  // log2 units: lazy max, exp2 <= 256

template <typename T, int D>
struct DecodeGeom {
    static constexpr int kElem = sizeof(T);
    static constexpr int kDpl = D / 8;                   // dims per lane
    static constexpr int kVecs = kDpl * kElem / 16;      // 16-byte loads per lane per token
    static_assert(kVecs >= 1, "head_dim too small");
};

// Scores of the lane's two tokens for its GP heads, fully reduced over dims.
template <typename T, int GP, int KDPL, int KVECS, int KQB>
__device__ __forceinline__ void qk_block(float (&sc)[2][GP], const uint4 (&kr)[2][KVECS],
                                         const uint32_t (&qb)[GP][KQB], const float (&qf)[GP][KDPL]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            float a = 0.f;
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int c = 0; c < KVECS; ++c) {
                    a = dot2_bf16(kr[t][c].x, qb[g][c * 4 + 0], a);
                    a = dot2_bf16(kr[t][c].y, qb[g][c * 4 + 1], a);
                    a = dot2_bf16(kr[t][c].z, qb[g][c * 4 + 2], a);
                    a = dot2_bf16(kr[t][c].w, qb[g][c * 4 + 3], a);
                }
            } else {
#pragma unroll
                for (int c = 0; c < KVECS; ++c) {
                    a = fmaf(__uint_as_float(kr[t][c].x), qf[g][c * 4 + 0], a);
                    a = fmaf(__uint_as_float(kr[t][c].y), qf[g][c * 4 + 1], a);
                    a = fmaf(__uint_as_float(kr[t][c].z), qf[g][c * 4 + 2], a);
                    a = fmaf(__uint_as_float(kr[t][c].w), qf[g][c * 4 + 3], a);
                }
            }
            sc[t][g] = sum_lanes8(a);
        }
    }
}

// acc[g][:] += p[0][g] * V[token 0] + p[1][g] * V[token 1]   (the lane's dims)
template <typename T, int GP, int KDPL, int KVECS>
__device__ __forceinline__ void pv_block(float (&acc)[GP][KDPL], float (&l)[GP], const float (&p)[2][GP],
                                         const uint4 (&vr)[2][KVECS]) {
    if constexpr (sizeof(T) == 2) {
        uint32_t pk[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            pk[g] = pack_bf16x2(p[0][g], p[1][g]);
            l[g] = dot2_bf16(pk[g], 0x3F803F80u, l[g]);  // + p0 + p1 as rounded
        }
#pragma unroll
        for (int c = 0; c < KVECS; ++c) {
            const uint32_t v0[4] = {vr[0][c].x, vr[0][c].y, vr[0][c].z, vr[0][c].w};
            const uint32_t v1[4] = {vr[1][c].x, vr[1][c].y, vr[1][c].z, vr[1][c].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // (even dim of token 0, even dim of token 1) and the odd dims
                const uint32_t ev = __builtin_amdgcn_perm(v1[j], v0[j], 0x05040100u);
                const uint32_t od = __builtin_amdgcn_perm(v1[j], v0[j], 0x07060302u);
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    acc[g][c * 8 + 2 * j] = dot2_bf16(ev, pk[g], acc[g][c * 8 + 2 * j]);
                    acc[g][c * 8 + 2 * j + 1] = dot2_bf16(od, pk[g], acc[g][c * 8 + 2 * j + 1]);
                }
            }
        }
    } else {
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
}

template <typename T, int D, int GP, int NW, int BPW, int CH>
__global__ __launch_bounds__(NW * kWave) void decode_partition_kernel(DecodeArgs a) {
    using G = DecodeGeom<T, D>;
    constexpr int kDpl = G::kDpl;
    constexpr int kVecs = G::kVecs;
    constexpr int kPart = NW * BPW * kBlockTokens;
    static_assert(BPW % CH == 0, "chunk must divide blocks per wave");

    const int n_kvg = a.num_kv_heads * a.groups_per_kv;
    const int wg = blockIdx.x;
    const int kvg = wg % n_kvg;
    const int rest = wg / n_kvg;
    const int s = rest % a.num_seqs;
    const int part = rest / a.num_seqs;

    const int n = a.context_lens[s];
    const int np = (n + kPart - 1) / kPart;
    if (part >= (np > 0 ? np : 1)) return;  // uniform over the workgroup

    const int hk = kvg / a.groups_per_kv;
    const int gi0 = (kvg % a.groups_per_kv) * GP;   // first head within the kv head's group
    const int h0 = hk * a.group + gi0;              // first query head of this unit
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int tg = lane >> 3;
    const int dl = lane & 7;

    // ---- query rows of the GP heads, this lane's dims
    constexpr int kQb = kDpl / 2 > 0 ? kDpl / 2 : 1;
    uint32_t qb[GP][kQb];
    float qf[GP][kDpl];
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((size_t)s * a.num_q_heads + h0) * D + dl * kDpl;
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const bool valid = gi0 + g < a.group;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int c = 0; c < kVecs; ++c) {
                uint4 v = valid ? *reinterpret_cast<const uint4*>(qrow + (size_t)g * D + c * 8)
                                : make_uint4(0, 0, 0, 0);
                qb[g][c * 4 + 0] = v.x; qb[g][c * 4 + 1] = v.y;
                qb[g][c * 4 + 2] = v.z; qb[g][c * 4 + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int c = 0; c < kVecs; ++c) {
                uint4 v = valid ? *reinterpret_cast<const uint4*>(qrow + (size_t)g * D + c * 4)
                                : make_uint4(0, 0, 0, 0);
                qf[g][c * 4 + 0] = __uint_as_float(v.x); qf[g][c * 4 + 1] = __uint_as_float(v.y);
                qf[g][c * 4 + 2] = __uint_as_float(v.z); qf[g][c * 4 + 3] = __uint_as_float(v.w);
            }
        }
    }

    float m[GP], l[GP], acc[GP][kDpl];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < kDpl; ++i) acc[g][i] = 0.f;
    }

    const int nblk = (n + kBlockTokens - 1) / kBlockTokens;
    const int jb_begin = part * (NW * BPW) + w * BPW;
    const int jb_end = min(jb_begin + BPW, nblk);
    const int32_t* bt = a.block_tables + (size_t)s * a.max_blocks_per_seq;
    const size_t blk_elems = (size_t)kBlockTokens * a.num_kv_heads * D;
    // element offset of (token tg, kv head hk, lane dims) inside a block
    const uint32_t lane_off0 = ((uint32_t)tg * a.num_kv_heads + hk) * D + dl * kDpl;
    const uint32_t tok8_off = 8u * a.num_kv_heads * D;
    const T* kbase = reinterpret_cast<const T*>(a.k_cache);
    const T* vbase = reinterpret_cast<const T*>(a.v_cache);
    constexpr int kElemsPerVec = 16 / sizeof(T);

    for (int jc = jb_begin; jc < jb_end; jc += CH) {
        uint4 kr[CH][2][kVecs], vr[CH][2][kVecs];
        // issue every load of the chunk first
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            if (jc + i < jb_end) {
                const int b = bt[jc + i];
                const T* kb = kbase + (size_t)b * blk_elems + lane_off0;
                const T* vb = vbase + (size_t)b * blk_elems + lane_off0;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int c = 0; c < kVecs; ++c) {
                        kr[i][t][c] = *reinterpret_cast<const uint4*>(kb + t * tok8_off + c * kElemsPerVec);
                    }
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int c = 0; c < kVecs; ++c) {
                        vr[i][t][c] = *reinterpret_cast<const uint4*>(vb + t * tok8_off + c * kElemsPerVec);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int jb = jc + i;
            if (jb >= jb_end) break;
            float sc[2][GP];
            qk_block<T, GP, kDpl, kVecs, kQb>(sc, kr[i], qb, qf);
            const int tok0 = jb * kBlockTokens + tg;
            const bool last = (jb + 1) * kBlockTokens > n;  // uniform
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int g = 0; g < GP; ++g) sc[t][g] *= a.scale_log2;
            }
            if (last) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    if (tok0 + 8 * t >= n) {
#pragma unroll
                        for (int g = 0; g < GP; ++g) sc[t][g] = -INFINITY;
#pragma unroll
                        for (int c = 0; c < kVecs; ++c) vr[i][t][c] = make_uint4(0, 0, 0, 0);
                    }
                }
            }
            // lazy running max: raise it only when a score clears it by the slack
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
            pv_block<T, GP, kDpl, kVecs>(acc, l, p, vr[i]);
        }
    }

    // ---- merge token groups and waves through LDS
    // token groups tg and tg^1 first (DPP, within a row), then LDS holds 4 per wave
    __shared__ float sh_acc[NW][4][GP][D];
    __shared__ float sh_m[NW][GP];
    __shared__ float sh_l[NW][GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const float lt = sum_groups8(l[g]);
        if (lane == 0) {
            sh_m[w][g] = m[g];
            sh_l[w][g] = lt;
        }
#pragma unroll
        for (int d = 0; d < kDpl; ++d) acc[g][d] += dpp_f32<kDppRowRor8>(acc[g][d]);
    }
    if ((tg & 1) == 0) {
#pragma unroll
        for (int g = 0; g < GP; ++g) {
#pragma unroll
            for (int d = 0; d < kDpl; d += 4) {
                *reinterpret_cast<float4*>(&sh_acc[w][tg >> 1][g][dl * kDpl + d]) =
                    make_float4(acc[g][d], acc[g][d + 1], acc[g][d + 2], acc[g][d + 3]);
            }
        }
    }
    __syncthreads();

    const bool single = np <= 1;
    const size_t ws_row0 = ((size_t)s * a.num_q_heads + h0) * a.max_parts + part;
    for (int idx = threadIdx.x; idx < GP * D; idx += NW * kWave) {
        const int g = idx / D;
        const int d = idx % D;
        if (gi0 + g >= a.group) continue;
        float mx = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) mx = fmaxf(mx, sh_m[ww][g]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float sw = (sh_m[ww][g] == -INFINITY) ? 0.f : fast_exp2(sh_m[ww][g] - mx);
            L += sh_l[ww][g] * sw;
            A += (sh_acc[ww][0][g][d] + sh_acc[ww][1][g][d] + sh_acc[ww][2][g][d] +
                  sh_acc[ww][3][g][d]) * sw;
        }
        if (single) {
            const float o = L > 0.f ? A / L : 0.f;
            T* orow = reinterpret_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + h0 + g) * D;
            if constexpr (sizeof(T) == 2) {
                reinterpret_cast<uint16_t*>(orow)[d] = f32_to_bf16_bits(o);
            } else {
                reinterpret_cast<float*>(orow)[d] = o;
            }
        } else {
            const size_t row = ws_row0 + (size_t)g * a.max_parts;
            a.ws_acc[row * D + d] = A;
            if (d == 0) {
                a.ws_ml[row * 2 + 0] = mx;
                a.ws_ml[row * 2 + 1] = L;
            }
        }
    }
}

// Merge the partitions of every (sequence, query head) whose context spans more
// than one partition: M = max_p m_p, L = sum_p l_p 2^(m_p - M),
// out = sum_p acc_p 2^(m_p - M) / L.  One wave per (sequence, head).
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a, int part_tokens) {
    const int wave_id = blockIdx.x * 4 + threadIdx.x / kWave;
    if (wave_id >= a.num_seqs * a.num_q_heads) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int s = wave_id / a.num_q_heads;
    const int h = wave_id % a.num_q_heads;
    const int n = a.context_lens[s];
    const int np = (n + part_tokens - 1) / part_tokens;
    if (np <= 1) return;
    const size_t row0 = ((size_t)s * a.num_q_heads + h) * a.max_parts;
    float mx = -INFINITY;
    for (int p = lane; p < np; p += kWave) mx = fmaxf(mx, a.ws_ml[(row0 + p) * 2]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float L = 0.f;
    for (int p = lane; p < np; p += kWave) {
        L += a.ws_ml[(row0 + p) * 2 + 1] * fast_exp2(a.ws_ml[(row0 + p) * 2] - mx);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    constexpr int kPerLane = D / kWave;  // 1 or 2
    float A[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) A[i] = 0.f;
    for (int p = 0; p < np; ++p) {
        const float sw = fast_exp2(a.ws_ml[(row0 + p) * 2] - mx);
        const float* src = a.ws_acc + (row0 + p) * D + lane * kPerLane;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) A[i] += src[i] * sw;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    T* orow = reinterpret_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + h) * D + lane * kPerLane;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const float o = A[i] * inv;
        if constexpr (sizeof(T) == 2) {
            reinterpret_cast<uint16_t*>(orow)[i] = f32_to_bf16_bits(o);
        } else {
            reinterpret_cast<float*>(orow)[i] = o;
        }
    }
}

// ---------------------------------------------------------------- launchers
template <typename T, int D, int GP, int NW, int BPW, int CH>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    constexpr int kPart = NW * BPW * kBlockTokens;
    const long long grid = (long long)a.max_parts * a.num_seqs * a.num_kv_heads * a.groups_per_kv;
    hipLaunchKernelGGL((decode_partition_kernel<T, D, GP, NW, BPW, CH>), dim3((unsigned)grid),
                       dim3(NW * kWave), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.max_parts > 1) {
        const int waves = a.num_seqs * a.num_q_heads;
        hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3((waves + 3) / 4), dim3(256), 0, stream,
                           a, kPart);
        e = hipGetLastError();
    }
    return e;
}

template <typename T, int D, int GP>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t stream) {
    return launch_decode_t<T, D, GP, kDecodeWaves, kDecodeBlocksPerWave, kDecodeChunk>(a, stream);
}

template <typename T, int D>
static hipError_t launch_decode_d(const DecodeArgs& a, int gp, hipStream_t stream) {
    switch (gp) {
        case 1: return launch_decode_g<T, D, 1>(a, stream);
        case 2: return launch_decode_g<T, D, 2>(a, stream);
        case 4: return launch_decode_g<T, D, 4>(a, stream);
        default: return launch_decode_g<T, D, 8>(a, stream);
    }
}

hipError_t launch_decode(const DecodeArgs& a, int dtype_bf16, int head_dim, int gp, hipStream_t stream) {
    if (dtype_bf16) {
        return head_dim == 64 ? launch_decode_d<uint16_t, 64>(a, gp, stream)
                              : launch_decode_d<uint16_t, 128>(a, gp, stream);
    }
    return head_dim == 64 ? launch_decode_d<float, 64>(a, gp, stream)
                          : launch_decode_d<float, 128>(a, gp, stream);
}

}  // namespace pa
