// pa_cache.hip -- KV append: copy each new token's K and V rows into the cache
// slot named by the slot mapping (decode appends only the new token's key and
// value: page "从零实现一个 mini vLLM--开篇", section "2. LLM 推理到底在慢什么";
// blocks of 16 tokens: page "轻量级的vLLM", section 核心机制一：分页 KV Cache).
//
// One token's row ([num_kv_heads, head_dim]) is contiguous both in the input
// and in the cache (at slot * row_bytes), so the append is a gather-free row
// copy: every thread moves one 16-byte vector of K or V.  The copy is bit
// exact for any element type.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int num_tokens,
    int row_vecs) {
    const long long per_tensor = (long long)num_tokens * row_vecs;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * per_tensor;
         i += (long long)gridDim.x * blockDim.x) {
        const bool is_v = i >= per_tensor;
        const long long j = is_v ? i - per_tensor : i;
        const int tok = (int)(j / row_vecs);
        const int vec = (int)(j % row_vecs);
        const int slot = slot_mapping[tok];
        if (slot < 0) continue;
        const uint4* src = is_v ? value : key;
        uint4* dst = is_v ? v_cache : k_cache;
        dst[(long long)slot * row_vecs + vec] = src[j];
    }
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int num_tokens, int row_bytes,
                                    hipStream_t stream) {
    const int row_vecs = row_bytes / 16;
    const long long total = 2LL * num_tokens * row_vecs;
    long long blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), slot_mapping,
                       num_tokens, row_vecs);
    return hipGetLastError();
}

// One 16-element piece of a K or V row as 16 E4M3 bytes: every element
// becomes e4m3(clamp(x * inv_scale, +-448)), nearest even (x * inv_scale in
// fp32).
template <typename T>
__device__ __forceinline__ uint4 fp8_piece16(const T* src, float inv) {
    float x[16];
    if constexpr (sizeof(T) == 2) {
        const uint4 u0 = reinterpret_cast<const uint4*>(src)[0];
        const uint4 u1 = reinterpret_cast<const uint4*>(src)[1];
        const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            x[2 * k] = bf16_lo(w[k]) * inv;
            x[2 * k + 1] = bf16_hi(w[k]) * inv;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 f = reinterpret_cast<const float4*>(src)[k];
            x[4 * k] = f.x * inv;
            x[4 * k + 1] = f.y * inv;
            x[4 * k + 2] = f.z * inv;
            x[4 * k + 3] = f.w * inv;
        }
    }
    return make_uint4(pack_fp8x4(x[0], x[1], x[2], x[3]), pack_fp8x4(x[4], x[5], x[6], x[7]),
                      pack_fp8x4(x[8], x[9], x[10], x[11]), pack_fp8x4(x[12], x[13], x[14], x[15]));
}

// KV append into an FP8 E4M3 cache (fp8_piece16 per 16 elements).  Each
// thread turns 16 elements of one K or V row into 16 bytes.
template <typename T>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const T* __restrict__ key, const T* __restrict__ value, uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int num_tokens, int row_vecs, float k_inv, float v_inv) {
    const long long per_tensor = (long long)num_tokens * row_vecs;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * per_tensor;
         i += (long long)gridDim.x * blockDim.x) {
        const bool is_v = i >= per_tensor;
        const long long j = is_v ? i - per_tensor : i;
        const int tok = (int)(j / row_vecs);
        const int vec = (int)(j % row_vecs);
        const int slot = slot_mapping[tok];
        if (slot < 0) continue;
        const uint4 o = fp8_piece16((is_v ? value : key) + j * 16, is_v ? v_inv : k_inv);
        (is_v ? v_cache : k_cache)[(long long)slot * row_vecs + vec] = o;
    }
}

// The decode step's append into an FP8 cache: sequence s's new K/V row
// (row s of key / value) goes to position context_lens[s] - 1, its slot
// found through the block table; sequences with no tokens are skipped.
__global__ __launch_bounds__(256) void append_rows_fp8_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int32_t* __restrict__ block_tables, int max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, int num_seqs, int row_vecs, float k_inv, float v_inv) {
    const long long per_tensor = (long long)num_seqs * row_vecs;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * per_tensor;
         i += (long long)gridDim.x * blockDim.x) {
        const bool is_v = i >= per_tensor;
        const long long j = is_v ? i - per_tensor : i;
        const int sq = (int)(j / row_vecs);
        const int vec = (int)(j % row_vecs);
        const int n = context_lens[sq];
        if (n <= 0) continue;
        const long long slot = (long long)block_tables[(size_t)sq * max_blocks_per_seq + (n - 1) / kBlockTokens] *
                                   kBlockTokens + (n - 1) % kBlockTokens;
        const uint4 o = fp8_piece16((is_v ? value : key) + j * 16, is_v ? v_inv : k_inv);
        (is_v ? v_cache : k_cache)[slot * row_vecs + vec] = o;
    }
}

hipError_t launch_append_rows_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                                  int num_seqs, int row_elems, float k_inv, float v_inv, hipStream_t stream) {
    const int row_vecs = row_elems / 16;
    const long long total = 2LL * num_seqs * row_vecs;
    long long blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(append_rows_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, row_vecs, k_inv, v_inv);
    return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                                        const int32_t* slot_mapping, int num_tokens, int row_elems, bool src_bf16,
                                        float k_inv, float v_inv, hipStream_t stream) {
    const int row_vecs = row_elems / 16;  // 16 elements -> one 16-byte vector of the cache
    const long long total = 2LL * num_tokens * row_vecs;
    long long blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (src_bf16) {
        hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                           static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), slot_mapping, num_tokens,
                           row_vecs, k_inv, v_inv);
    } else {
        hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const float*>(key), static_cast<const float*>(value),
                           static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), slot_mapping, num_tokens,
                           row_vecs, k_inv, v_inv);
    }
    return hipGetLastError();
}

// Copy-on-write support: for every pair (src, dst) in pairs[n][2], block dst
// of both caches becomes a bit copy of block src.  Each thread moves one
// 16-byte vector.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs, int num_pairs,
                                                          int block_vecs) {
    const long long per_tensor = (long long)num_pairs * block_vecs;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * per_tensor;
         i += (long long)gridDim.x * blockDim.x) {
        const bool is_v = i >= per_tensor;
        const long long j = is_v ? i - per_tensor : i;
        const int p = (int)(j / block_vecs);
        const int vec = (int)(j % block_vecs);
        uint4* cache = is_v ? v_cache : k_cache;
        cache[(long long)pairs[2 * p + 1] * block_vecs + vec] = cache[(long long)pairs[2 * p] * block_vecs + vec];
    }
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs, int block_bytes,
                              hipStream_t stream) {
    const int block_vecs = block_bytes / 16;
    const long long total = 2LL * num_pairs * block_vecs;
    long long blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<uint4*>(k_cache),
                       static_cast<uint4*>(v_cache), pairs, num_pairs, block_vecs);
    return hipGetLastError();
}

}  // namespace pa

namespace pa {

// One streaming read of a buffer, the reference read rate of the benchmark:
// every 16-byte vector is loaded once with the non-temporal hint (as the
// decode stream loads K and V), eight in flight per thread, and every 32-bit
// word is folded by XOR into *xor_out.  The fold keeps the loads and gives a
// result a test can check exactly.
__global__ __launch_bounds__(256) void stream_read_probe_kernel(const uint4* __restrict__ src, long long n_vec,
                                                                uint32_t* __restrict__ xor_out) {
    constexpr int kU = 8;
    uint32_t acc = 0;
    const long long stride = (long long)gridDim.x * blockDim.x;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kU - 1) * stride < n_vec; i += kU * stride) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = ldg_nt(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n_vec; i += stride) {
        const uint4 v = ldg_nt(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if ((threadIdx.x & (kWave - 1)) == 0 && acc != 0) atomicXor(xor_out, acc);
}

hipError_t launch_stream_read_probe(const void* src, size_t bytes, uint32_t* xor_out, hipStream_t stream) {
    const long long n_vec = (long long)(bytes / 16);
    long long blocks = (n_vec + 255) / 256;
    // 16 workgroups of 4 waves per compute unit: 6.45 TB/s over 4 GiB, against
    // 6.27 with 8 and 5.74 with 4 (plain loads instead of non-temporal: 5.64)
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(stream_read_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(src), n_vec, xor_out);
    return hipGetLastError();
}

}  // namespace pa
