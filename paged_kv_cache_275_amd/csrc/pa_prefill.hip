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
//  * Work items (sequence, kv head, row tile) are numbered so that the items
//    of one (sequence, kv head) are consecutive, latest rows (the most keys)
//    first, and the grid is remapped so that each XCD (workgroup id mod 8)
//    takes one contiguous eighth of the items: the workgroups that read the
//    same K/V share one L2, and each XCD starts on its longest items.
//  * Keys stream through LDS in tiles of 64 (four 16-token blocks, resolved
//    through the block table).  K is stored row-major; V is stored transposed
//    (V^T[dim][key]) so that it can be an MFMA A operand.  Two LDS buffers: a
//    step stores tile t+1 into one while the matrix cores work on tile t from
//    the other, with one barrier per tile (measured 4-5% faster than storing
//    and computing on a single buffer between two barriers).  Global loads run
//    two tiles ahead in registers, always issued (block index clamped into the
//    sequence, keys past the context masked afterwards), so the load counter
//    never has to drain and no load waits on another.
//  * Scores are computed transposed, S^T = K Q^T: lane l then holds column l%16
//    and keys 4*(l/16) .. +3 of each 16-key subtile.  Row maxima and sums are
//    per-lane work plus two lane swaps, and the probabilities of two subtiles
//    are, unchanged, the B operand of O^T = V^T P^T for a 32-key step (k-slots
//    8g .. 8g+7 of lane group g are keys 4g .. 4g+3 of the first subtile and of
//    the second; V^T is read with the same key order).
//  * Online softmax per column in the log2 domain; keys past a row's position,
//    and past the context, are masked (score -inf, V zero).
//  * FP8 E4M3 caches (KV8): each 8-element chunk is loaded as 8 bytes instead of
//    16 and converted exactly to bf16 before it is written to LDS, so the tiles
//    and everything after them are the same; k_scale is folded into the score
//    scale by the host and v_scale into the final normalisation.
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr float kSlack = 8.0f;  // log2 units: lazy running max, exp2 <= 256

template <int D, int GP, int NW, int CT, bool KV8>
__global__ __launch_bounds__(NW * kWave, 8 / NW) void prefill_kernel(PrefillArgs a) {
    constexpr int kCols = NW * 16 * CT;  // (row, head) columns per workgroup
    constexpr int kRT = kCols / GP;      // query rows per workgroup
    constexpr int kKT = 64;              // keys per tile
    // K row pitch in LDS (elements).  D + 16 (a 32-byte shift per row) measured
    // 45% fewer LDS bank-conflict cycles than D + 8 and 2.5% faster; D + 24,
    // D + 32 and D + 40 were no better than D + 8.
    constexpr int kKP = D + 16;
    // V^T row pitch in LDS (elements).  kKT + 16 measured bank conflicts in
    // 9% of the LDS-active cycles against 33% for kKT + 8 (the prefill time
    // moved by less than 0.5%: the LDS is not what bounds it).
    constexpr int kVP = kKT + 16;
    constexpr int kMs = D / 32;          // MFMA k-steps over dims
    constexpr int kDt = D / 16;          // 16-dim tiles of the output
    constexpr int kNT = NW * kWave;
    constexpr int kKChunks = kKT * D / 8 / kNT;  // 16-byte K chunks per thread per tile
    // V is staged as blocks of 2 keys x 8 dims: every thread of the
    // workgroup takes one (D = 128), and two V chunks per thread leave the
    // registers for the accumulators (measured 3-8% faster than 4-key blocks
    // on half of the threads)
    constexpr int kVK = 2;
    constexpr int kVBlocks = kKT / kVK * (D / 8);  // V blocks per tile
    static_assert(kKChunks >= 1 && kKChunks * kNT == kKT * D / 8, "K staging must cover the tile");
    static_assert(kVBlocks <= kNT, "V staging assumes at most one block per thread");

    // two LDS buffers: tile t+1 is stored while tile t is computed on
    __shared__ __align__(16) uint16_t k_lds2[2][kKT * kKP];
    __shared__ __align__(16) uint16_t vt_lds2[2][D * kVP];

    // ---- work item: see the header.  Sequence s owns items[s] = ceil(c / RT) *
    // kv heads consecutive items; the workgroup's item is found by a prefix
    // scan of items[] across the workgroup's threads, 512 sequences at a time.
    __shared__ int s_wave[NW];  // per-wave totals of a scan
    __shared__ int s_loc[2];    // the item's sequence, items before it
    const int S = a.num_seqs;
    const int hkv_heads = a.num_kv_heads;
    // The index arrays are read through the constant address space: a uniform
    // read is then a scalar load, which the loads of K and V do not wait
    // behind (the barriers of the scan would otherwise count as possible
    // writers, and the reads become vector loads).
    using cint_ptr = const __attribute__((address_space(4))) int32_t*;
    const cint_ptr qsl = (cint_ptr)a.query_start_loc;
    const cint_ptr ctxl = (cint_ptr)a.context_lens;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    auto seq_items = [&](int q) __attribute__((always_inline)) {
        const int cq = qsl[q + 1] - qsl[q];
        return (cq + kRT - 1) / kRT * hkv_heads;
    };
    // inclusive prefix over the workgroup's threads, and the total
    auto block_scan = [&](int v, int& tot) __attribute__((always_inline)) {
        const int x = wave_scan_incl(v);
        if (lane == kWave - 1) s_wave[w] = x;
        __syncthreads();
        int off = 0;
        tot = 0;
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const int t = s_wave[k];
            off += k < w ? t : 0;
            tot += t;
        }
        __syncthreads();  // s_wave is rewritten by the next scan
        return off + x;
    };
    int v = tid < S ? seq_items(tid) : 0;
    int tot;
    int incl = block_scan(v, tot);
    int total = tot;
    for (int b = kNT; b < S; b += kNT) {
        int t;
        block_scan(b + tid < S ? seq_items(b + tid) : 0, t);
        total += t;
    }
    const int per_xcd = (total + 7) / 8;
    const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if ((int)(blockIdx.x / 8) >= per_xcd || item >= total) return;  // uniform: grid is an upper bound
    for (int b = 0, carry = 0;; b += kNT) {
        if (b > 0) {
            v = b + tid < S ? seq_items(b + tid) : 0;
            incl = block_scan(v, tot);
        }
        if (v > 0 && carry + incl - v <= item && item < carry + incl) {
            s_loc[0] = b + tid;
            s_loc[1] = carry + incl - v;
        }
        carry += tot;
        if (carry > item) break;  // uniform: found in this batch
    }
    __syncthreads();
    const int s = __builtin_amdgcn_readfirstlane(s_loc[0]);
    const int base = __builtin_amdgcn_readfirstlane(s_loc[1]);
    const int r0 = qsl[s];
    const int c = qsl[s + 1] - r0;
    const int tiles = (c + kRT - 1) / kRT;
    const int hk = (item - base) / tiles;
    const int tile = tiles - 1 - (item - base) % tiles;  // latest rows first
    const int n = ctxl[s];
    const int i0 = tile * kRT;
    const int rows = min(kRT, c - i0);
    const int pos0 = n - c + i0;           // position of the workgroup's first row
    const int pmax = pos0 + rows - 1;      // last key any row needs
    const int ntiles = pmax / kKT + 1;
    const int nblk = (n + kBlockTokens - 1) / kBlockTokens;  // table entries that may be read
    const cint_ptr bt = (cint_ptr)a.block_tables + (size_t)s * a.max_blocks_per_seq;

    const int lg = lane >> 4;    // lane group: k-slots 8*lg .. +8, output rows 4*lg .. +3
    const int lc = lane & 15;    // column within a 16-column tile
    using KVT = typename std::conditional<KV8, uint8_t, uint16_t>::type;  // cache element
    const KVT* kcache = reinterpret_cast<const KVT*>(a.k_cache);
    const KVT* vcache = reinterpret_cast<const KVT*>(a.v_cache);

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
    // Scores are scaled inside the exponent, exp2(s * scale - m), with the
    // running max taken over raw scores; for a negative scale q is negated
    // (exact in bf16) so that the scale used is positive.  A zero scale makes
    // every score 0: q is zeroed and the scale set to 1 instead, so that the
    // masked scores (-inf) are not multiplied by 0.
    const bool zero_scale = a.scale_log2 == 0.f;
    const float qscale = zero_scale ? 1.f : fabsf(a.scale_log2);
    if (zero_scale) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
            for (int m = 0; m < kMs; ++m) qb[ct][m] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    if (a.scale_log2 < 0.f) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
            for (int m = 0; m < kMs; ++m) {
                qb[ct][m].x ^= 0x80008000u; qb[ct][m].y ^= 0x80008000u;
                qb[ct][m].z ^= 0x80008000u; qb[ct][m].w ^= 0x80008000u;
            }
        }
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

    // ---- staging: K chunks (key, 16-byte chunk) and one 2-key x 8-dim V block,
    // two tiles in flight
    // native vector registers (a struct copy would be lowered through memory)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    // one 8-element chunk as loaded: 16 bytes of bf16, or 8 bytes of fp8
    using Chunk = typename std::conditional<KV8, u32x2, u32x4>::type;
    Chunk kreg[2][kKChunks], vreg[2][kVK];
    // a loaded chunk as 8 bf16 (the fp8 conversion is exact)
    auto widen = [](const Chunk& c) __attribute__((always_inline)) -> u32x4 {
        if constexpr (KV8) {
            return u32x4{fp8x2_to_bf16x2<false>(c[0]), fp8x2_to_bf16x2<true>(c[0]), fp8x2_to_bf16x2<false>(c[1]),
                         fp8x2_to_bf16x2<true>(c[1])};
        } else {
            return c;
        }
    };
    const int v_kg = tid / (D / 8);   // keys kVK*v_kg .. +kVK-1 of the tile
    const int v_dc = tid % (D / 8);   // dims 8*v_dc .. +7
    // the four blocks of tile t (the same for the whole workgroup); entries past
    // the context are never read: the index is clamped, and the keys such a
    // block would hold are masked
    auto tile_blocks = [&](int t) __attribute__((always_inline)) {
        int4 b;
        b.x = bt[min(t * 4 + 0, nblk - 1)];
        b.y = bt[min(t * 4 + 1, nblk - 1)];
        b.z = bt[min(t * 4 + 2, nblk - 1)];
        b.w = bt[min(t * 4 + 3, nblk - 1)];
        return b;
    };
    static_assert(kKT == 4 * kBlockTokens, "a key tile is four blocks");
    // Per-thread element offsets inside a block, fixed for the whole kernel
    // (tiles start on block boundaries); which of the tile's four blocks a
    // load reads is the same across a wave for K, and for V when D = 128.
    constexpr size_t kBlkElems = (size_t)kBlockTokens * D;  // per kv head, times hkv_heads below
    const size_t blk_stride = kBlkElems * hkv_heads;
    uint32_t koff[kKChunks];
    int kbi[kKChunks];
#pragma unroll
    for (int j = 0; j < kKChunks; ++j) {
        const int q = tid + j * kNT;
        const int key = q / (D / 8);
        koff[j] = (uint32_t)(((key % kBlockTokens) * hkv_heads + hk) * D + (q % (D / 8)) * 8);
        kbi[j] = __builtin_amdgcn_readfirstlane(key / kBlockTokens);
    }
    // a wave's V keys (8 for D = 128, 16 for D = 64) lie in one block
    static_assert(kWave / (D / 8) * kVK <= kBlockTokens, "a wave's V keys must share a block");
    const int vk = tid < kVBlocks ? kVK * v_kg : 0;
    const int vbi = __builtin_amdgcn_readfirstlane(vk / kBlockTokens);
    uint32_t voff[kVK];
#pragma unroll
    for (int e = 0; e < kVK; ++e) voff[e] = (uint32_t)((((vk + e) % kBlockTokens) * hkv_heads + hk) * D + v_dc * 8);
    auto load_tile = [&](int t, int buf, int4 bq) __attribute__((always_inline)) {
        auto blk = [&](int j) {  // block j of the tile, without dynamic indexing
            return j == 0 ? bq.x : j == 1 ? bq.y : j == 2 ? bq.z : bq.w;
        };
#pragma unroll
        for (int j = 0; j < kKChunks; ++j) {
            const KVT* base = kcache + (size_t)blk(kbi[j]) * blk_stride;
            kreg[buf][j] = *reinterpret_cast<const Chunk*>(base + koff[j]);
        }
        const KVT* vbase = vcache + (size_t)blk(vbi) * blk_stride;
#pragma unroll
        for (int e = 0; e < kVK; ++e) {
            // waves past the V blocks load nothing (uniform per wave: kVBlocks is
            // a multiple of the wave size)
            if (kVBlocks >= kNT || tid < kVBlocks) vreg[buf][e] = *reinterpret_cast<const Chunk*>(vbase + voff[e]);
        }
    };
    auto store_tile = [&](int t, int buf, int lb) __attribute__((always_inline)) {
        uint16_t* k_lds = k_lds2[lb];
        uint16_t* vt_lds = vt_lds2[lb];
#pragma unroll
        for (int j = 0; j < kKChunks; ++j) {
            const int q = tid + j * kNT;
            *reinterpret_cast<u32x4*>(&k_lds[(q / (D / 8)) * kKP + (q % (D / 8)) * 8]) = widen(kreg[buf][j]);
        }
        if (tid >= kVBlocks) return;
        // keys past the context: V is zero (the slots may hold anything)
        u32x4 vv[kVK];
#pragma unroll
        for (int e = 0; e < kVK; ++e) vv[e] = widen(vreg[buf][e]);
        if (t * kKT + kKT > n) {  // uniform: only the tile that reaches past the context
#pragma unroll
            for (int e = 0; e < kVK; ++e) {
                if (t * kKT + kVK * v_kg + e >= n) vv[e] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        // V^T columns of this thread's two keys: within each group of 32 keys
        // the 4-key chunks are stored in the order 0,4,1,5,2,6,3,7, so that the
        // keys lane group g needs for a 32-key MFMA step (chunks g and g+4) are
        // 16 contiguous bytes.  Row r's 16-byte chunks are then permuted by XOR
        // with (r / 16) % 8, which spreads these stores over the LDS banks (the
        // reads of one MFMA step all share r / 16); this thread's 8 rows lie in
        // one 16-row band.
        const int k0 = kVK * v_kg;
        const int xk = (k0 % 32) / 4;
        const int vcol = (k0 / 32) * 32 + 4 * (xk < 4 ? 2 * xk : 2 * (xk - 4) + 1);
        const int col = (vcol ^ (8 * ((v_dc >> 1) & 7))) + k0 % 4;
        const uint32_t w0[4] = {vv[0].x, vv[0].y, vv[0].z, vv[0].w};
        const uint32_t w1[4] = {vv[1].x, vv[1].y, vv[1].z, vv[1].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // dim 2j: the low halves of the two keys; dim 2j+1: the high halves
            const int r0e = v_dc * 8 + 2 * j;
            *reinterpret_cast<uint32_t*>(&vt_lds[r0e * kVP + col]) = __builtin_amdgcn_perm(w1[j], w0[j], 0x05040100u);
            *reinterpret_cast<uint32_t*>(&vt_lds[(r0e + 1) * kVP + col]) = __builtin_amdgcn_perm(w1[j], w0[j], 0x07060302u);
        }
    };

    // Tile t uses register buffer t % 2.  The step is called with a literal
    // buffer index (the loop runs over pairs of tiles) so that the buffers stay
    // in registers.
    // tiles [0, tmask) lie entirely at or before the first row's position
    const int tmask = pos0 >= kKT - 1 ? (pos0 - (kKT - 1)) / kKT + 1 : 0;
    auto step = [&](const int t, const int lb, int4& bn) __attribute__((always_inline)) {
        // lb = t % 2: the LDS buffer (and register buffer) of tile t.  The other
        // buffers take tile t+1, whose LDS buffer was last read by tile t-1,
        // before the barrier that ended the previous step.
        if (t + 1 < ntiles) store_tile(t + 1, 1 - lb, 1 - lb);
        load_tile(min(t + 3, ntiles - 1), 1 - lb, bn);  // past the end: a repeat, never stored
        bn = tile_blocks(min(t + 4, ntiles - 1));        // requested a step before it is needed
        const uint16_t* k_lds = k_lds2[lb];
        const uint16_t* vt_lds = vt_lds2[lb];
        const int t0 = t * kKT;
        // every key of this tile is visible to every row of the workgroup
        // unless the tile reaches past the first row's position (the last
        // tile or two of a row tile)
        const bool masked = t >= tmask;

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
        // ---- causal mask, only on tiles that reach past the first row (uniform)
        if (__builtin_expect(masked, 0)) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (t0 + sb * 16 + 4 * lg + r > col_pos[ct]) sacc[sb][ct][r] = -INFINITY;
                    }
                }
            }
        }
        // ---- online softmax per column
        uint4 pb[CT][2];  // B operands of the two 32-key P*V steps
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            float sv[4][4];  // raw scores, -inf where masked
            float tmax = -INFINITY;
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sv[sb][r] = sacc[sb][ct][r];
                    tmax = fmaxf(tmax, sv[sb][r]);
                }
            }
            tmax *= qscale;
            // Lazy running max: raised only when a score exceeds it by more than
            // kSlack (log2 units), so exp2 stays <= 2^kSlack and the rescale of
            // the accumulators is rare.  Tile 0 holds key 0, visible to every
            // row, so the max is finite from then on.
            const bool need = tmax > mrun[ct] + kSlack;
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
                // the column's keys live in lanes lc, lc+16, lc+32, lc+48
                auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
                float cm = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
                auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(cm), __float_as_uint(cm), false, false);
                cm = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
                const float mn = fmaxf(mrun[ct], cm);
                const float alpha = mrun[ct] == -INFINITY ? 0.f : fast_exp2(mrun[ct] - mn);
                mrun[ct] = mn;
                lrun[ct] *= alpha;
#pragma unroll
                for (int dt = 0; dt < kDt; ++dt) o[ct][dt] *= alpha;
            }
            const float nm = -mrun[ct];
            float pv[4][4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) pv[sb][r] = fast_exp2(fmaf(sv[sb][r], qscale, nm));
            }
            float psum = lrun[ct];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                pb[ct][kk] = make_uint4(pack_bf16x2(pv[2 * kk][0], pv[2 * kk][1]),
                                        pack_bf16x2(pv[2 * kk][2], pv[2 * kk][3]),
                                        pack_bf16x2(pv[2 * kk + 1][0], pv[2 * kk + 1][1]),
                                        pack_bf16x2(pv[2 * kk + 1][2], pv[2 * kk + 1][3]));
                // the normaliser sums the probabilities as rounded for P*V
                psum = dot2_bf16(pb[ct][kk].x, 0x3F803F80u, psum);
                psum = dot2_bf16(pb[ct][kk].y, 0x3F803F80u, psum);
                psum = dot2_bf16(pb[ct][kk].z, 0x3F803F80u, psum);
                psum = dot2_bf16(pb[ct][kk].w, 0x3F803F80u, psum);
            }
            lrun[ct] = psum;
        }
        // ---- O^T += V^T P^T (32 keys per step)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int dt = 0; dt < kDt; ++dt) {
                const uint4 va = *reinterpret_cast<const uint4*>(
                    &vt_lds[(dt * 16 + lc) * kVP + ((32 * kk + 8 * lg) ^ (8 * (dt & 7)))]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) o[ct][dt] = mfma16x16x32_bf16(va, pb[ct][kk], o[ct][dt]);
            }
        }
        __syncthreads();  // tile t is no longer read; tile t+1 is in LDS
    };
    load_tile(0, 0, tile_blocks(0));
    load_tile(ntiles > 1 ? 1 : 0, 1, tile_blocks(ntiles > 1 ? 1 : 0));  // always issued
    store_tile(0, 0, 0);
    load_tile(min(2, ntiles - 1), 0, tile_blocks(min(2, ntiles - 1)));  // always issued
    int4 bnext = tile_blocks(min(3, ntiles - 1));  // blocks of the next tile to load
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
        step(t, 0, bnext);
        if (t + 1 < ntiles) step(t + 1, 1, bnext);
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
        const float inv = (KV8 ? a.v_scale : 1.f) / lt;
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
template <int D, int GP, bool KV8>
static hipError_t launch_prefill_g(const PrefillArgs& a, int total_rows, hipStream_t stream) {
    constexpr int kNW = 8, kCT = 2;
    constexpr int kRT = kNW * 16 * kCT / GP;
    // an upper bound of the work items (sequence, kv head, row tile), rounded
    // up to whole XCD shares
    const long long items = ((long long)total_rows / kRT + a.num_seqs) * a.num_kv_heads;
    const long long grid = (items + 7) / 8 * 8;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_kernel<D, GP, kNW, kCT, KV8>), dim3((unsigned)grid), dim3(kNW * kWave), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool KV8>
static hipError_t launch_prefill_d(const PrefillArgs& a, int total_rows, int gp, hipStream_t stream) {
    switch (gp) {
        case 1: return launch_prefill_g<D, 1, KV8>(a, total_rows, stream);
        case 2: return launch_prefill_g<D, 2, KV8>(a, total_rows, stream);
        case 4: return launch_prefill_g<D, 4, KV8>(a, total_rows, stream);
        case 8: return launch_prefill_g<D, 8, KV8>(a, total_rows, stream);
        default: return launch_prefill_g<D, 16, KV8>(a, total_rows, stream);
    }
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int total_rows, int gp, bool kv8, hipStream_t stream) {
    if (kv8) {
        return head_dim == 64 ? launch_prefill_d<64, true>(a, total_rows, gp, stream)
                              : launch_prefill_d<128, true>(a, total_rows, gp, stream);
    }
    return head_dim == 64 ? launch_prefill_d<64, false>(a, total_rows, gp, stream)
                          : launch_prefill_d<128, false>(a, total_rows, gp, stream);
}

}  // namespace pa
