// pa_launch.h -- host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Decode work split: a workgroup of kDecodeWaves waves covers one partition of
// kDecodeWaves * kDecodeBlocksPerWave blocks of one sequence; each wave issues
// the loads of kDecodeChunk blocks before consuming them.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeBlocksPerWave = 4;
constexpr int kDecodeChunk = 2;
constexpr int kDecodePartTokens = kDecodeWaves * kDecodeBlocksPerWave * 16;

struct DecodeArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    float* ws_ml;   // [S, Hq, max_parts, 2]  (running max in log2 units, sum)
    float* ws_acc;  // [S, Hq, max_parts, D]  unnormalised partial outputs
    int max_blocks_per_seq;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;          // query heads per kv head
    int groups_per_kv;  // head groups (of up to GP heads) per kv head
    int max_parts;      // partitions per sequence the workspace holds
    float scale_log2;   // scale * log2(e)
};

hipError_t launch_decode(const DecodeArgs& a, int dtype_bf16, int head_dim, int gp, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int num_tokens, int row_bytes,
                                    hipStream_t stream);

}  // namespace pa
