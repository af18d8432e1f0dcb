// pa_launch.h -- host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Decode launch shape: a persistent grid of waves (kDecodeWaves per
// workgroup), each streaming an equal share of the (sequence, head group,
// block) units with kDecodeStages blocks in flight; block ids are staged in
// LDS kDecodeWindow units at a time.
constexpr int kDecodeWaves = 4;
// Default ring depth: 2 blocks per wave measured best, for bf16 and fp8
// caches alike (llama3_8b: 81.0 us bf16 and 46.4 us fp8 at 2, 46.7 / 47.2 /
// 48.1 us fp8 at 3 / 4 / 6); 3 and 4 are also built (fp8 caches: 2, 3, 4, 6,
// 8).
constexpr int kDecodeStages = 2;
constexpr int kDecodeWindow = 256;
// One wave per SIMD.  fp8 caches too: their units have half the bytes of a
// bf16 unit and the same matrix-core work, and a second wave per SIMD (8 per
// compute unit) measured slower (llama3_8b 48.6 against 46.4 us).
constexpr int kDecodeWavesPerCU = 4;
constexpr int kDecodeMaxWaves = 4096;   // workspace records are sized for this many waves
constexpr int kDecodeMaxSeqs = 8192;    // sequence prefix sums live in LDS
// Work-split costs: closing a segment takes about as long as streaming one
// unit, so each segment counts kDecodeSwitchTicks / kDecodeUnitTicks extra
// units when the units are shared out among the waves.
constexpr int kDecodeUnitTicks = 4;
constexpr int kDecodeSwitchTicks = 4;
// Wave groups of the second band over the first, where the head groups are
// split in two bands (pa_api.hip, decode_bands).
constexpr double kDecodeBandRatio = 1.032;

// A segment (sequence, head group) whose units were split across waves, noted
// by the wave that holds its first unit.  seq < 0: no split segment starts in
// that wave.  The segment's records are slot first_slot of the noting wave and
// slot 0 of the waves of the same head group in the following wave groups of
// its band (every band_heads-th wave) up to last_wave; waves with an empty
// range leave a record of zero weight there.
struct SplitNote {
    int seq;
    int kvg;
    int last_wave;
    int first_slot;
};

struct DecodeArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    // fused append (all null otherwise): each sequence's new token, [S, Hkv, D],
    // written to the cache at position N-1 and read from here by the attention
    const void* new_k;
    const void* new_v;
    void* k_cache_w;
    void* v_cache_w;
    SplitNote* ws_split;   // [waves] split segment starting in each wave
    float* ws_ml;   // [waves, 2, GP, 2]  (running max in log2 units, sum)
    float* ws_acc;  // [waves, 2, GP, D]  unnormalised partial outputs
    int max_blocks_per_seq;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;          // query heads per kv head
    int groups_per_kv;  // head groups (of up to GP heads) per kv head
    int n_kvg;          // num_kv_heads * groups_per_kv
    // The head groups are split into bands of band_heads consecutive head
    // groups (one band, band_heads = n_kvg, or two halves).  Band b has
    // band_groups[b] wave GROUPS of band_heads waves; group g of band b
    // streams the g-th of band_groups[b] equal shares of all blocks for the
    // band's head groups.  Waves are numbered band by band.
    int band_heads;
    int band_groups[2];  // band_groups[1] = 0 with one band
    int waves;           // working waves: (band_groups[0] + band_groups[1]) * band_heads
    int unit_ticks;     // work-split cost of one unit (one block of one head group)
    int switch_ticks;   // extra cost of closing a segment (one head group of a sequence)
    float scale_log2;   // scale * log2(e) (times k_scale for an fp8 cache)
    float v_scale;      // fp8 cache: dequantized V = v_scale * stored value (unused otherwise)
};

struct PrefillArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* query_start_loc;
    const int32_t* context_lens;
    int max_blocks_per_seq;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;          // query heads per kv head
    float scale_log2;   // scale * log2(e) (times k_scale for an fp8 cache)
    float v_scale;      // fp8 cache: dequantized V = v_scale * stored value (unused otherwise)
};

// Query heads per prefill column group: a power of two >= group, at most 16.
constexpr int kPrefillMaxGroup = 16;

// kv8: the caches hold FP8 E4M3 (k_scale already in scale_log2).
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int total_rows, int gp, bool kv8, hipStream_t stream);
// Launches the streaming kernel and the split-segment merge.  Non-null events
// receive the streaming kernel's start and stop times.  kv8: the caches hold
// FP8 E4M3 (bf16 queries only; 2, 3, 4, 6 or 8 stages).
hipError_t launch_decode(const DecodeArgs& a, int dtype_bf16, int head_dim, int gp, int stages, bool kv8,
                         hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);

// The decode step's new rows (bf16 [num_seqs, row_elems]) quantized into an
// FP8 cache at each sequence's last position, slots through the block table.
hipError_t launch_append_rows_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                                  int num_seqs, int row_elems, float k_inv, float v_inv, hipStream_t stream);
hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int num_tokens, int row_bytes,
                                    hipStream_t stream);
hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                                        const int32_t* slot_mapping, int num_tokens, int row_elems, bool src_bf16,
                                        float k_inv, float v_inv, hipStream_t stream);
hipError_t launch_stream_read_probe(const void* src, size_t bytes, uint32_t* xor_out, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs, int block_bytes,
                              hipStream_t stream);

}  // namespace pa
