// pa_api.hip -- the C ABI of libpa.so (declared in include/pa.h).
//
// Host code only: argument checks (all before anything is enqueued), workspace
// layout, grid sizing and dispatch to the kernel instances.
#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>

#include "pa.h"
#include "pa_launch.h"

namespace {

constexpr int kMaxGroup = 64;  // query heads per kv head handled (8 groups of 8)

int check_dtype(pa_dtype dtype) {
    return (dtype == PA_F32 || dtype == PA_BF16) ? PA_OK : PA_EUNSUPPORTED;
}

// Element types of a cache for the bit copies (fp8 caches included).
int check_storage_dtype(pa_dtype dtype) {
    return (dtype == PA_F32 || dtype == PA_BF16 || dtype == PA_FP8_E4M3) ? PA_OK : PA_EUNSUPPORTED;
}

int elem_bytes(pa_dtype dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_FP8_E4M3 ? 1 : 2); }

int check_cache_shape(int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks) {
    if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0) return PA_EINVAL;
    if (num_blocks > INT32_MAX / block_size) return PA_EINVAL;  // slots must fit int32
    if (block_size != 16) return PA_EUNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_EUNSUPPORTED;
    return PA_OK;
}

// FP8 cache scales: finite, positive, and with a finite reciprocal.
int check_kv_scales(float k_scale, float v_scale) {
    const float lo = 1.0f / 3.0e38f;
    if (!(isfinite(k_scale) && isfinite(v_scale) && k_scale > lo && v_scale > lo)) return PA_EINVAL;
    return PA_OK;
}

int check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return PA_EINVAL;
    if (num_q_heads / num_kv_heads > kMaxGroup) return PA_EUNSUPPORTED;
    return PA_OK;
}

// Query heads handled by one wave (a power of two, at most 8).
int heads_per_wave(int group) {
    int gp = 1;
    while (gp < group && gp < 8) gp *= 2;
    return gp;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Decode workspace: one split-segment note per wave,
// then the partial records of up to kDecodeMaxWaves waves (2 slots each):
// (max, sum) pairs, then accumulators.  Every byte the fix-up kernel reads is
// written earlier in the same call, so the workspace needs no initialisation.
struct DecodeWsLayout {
    size_t split, ml, acc, total;
};

// waves: the records of this many waves (every launch shape, by default).
DecodeWsLayout decode_ws_layout(int gp, int32_t head_dim, int waves = pa::kDecodeMaxWaves) {
    DecodeWsLayout L;
    const size_t recs = (size_t)waves * 2 * gp;
    L.split = 0;
    L.ml = L.split + align256((size_t)waves * sizeof(pa::SplitNote));
    L.acc = L.ml + align256(recs * 2 * sizeof(float));
    L.total = L.acc + align256(recs * head_dim * sizeof(float));
    return L;
}

// Launch-shape overrides set by pa_decode_set_launch (0: the built-in
// default).  Process-wide; read with relaxed loads on every decode call.
std::atomic<int> g_override_waves{0};
std::atomic<int> g_override_stages{0};
std::atomic<int> g_override_switch_ticks{-1};

// Waves of the persistent decode grid: per_cu per compute unit of the
// current device, unless pa_decode_set_launch chose a count.
int decode_waves(int per_cu) {
    // compute units per device, looked up once (any thread may fill a slot;
    // all write the same value)
    static std::atomic<int> cached_cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int slot = dev < 64 ? dev : 63;
    int cus = cached_cus[slot].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached_cus[slot].store(cus, std::memory_order_relaxed);
    }
    long long w = (long long)cus * per_cu;
    const int ov = g_override_waves.load(std::memory_order_relaxed);
    if (ov > 0) w = ov;
    if (w > pa::kDecodeMaxWaves) w = pa::kDecodeMaxWaves;
    w = (w / pa::kDecodeWaves) * pa::kDecodeWaves;
    if (w < pa::kDecodeWaves) w = pa::kDecodeWaves;
    return (int)w;
}

// Bands of the decode grid (see DecodeArgs).  With a bf16 cache, head_dim 128,
// 8 kv heads and one head group per kv head -- 2 KB token rows -- the waves
// of kv heads 4..7 stream measurably slower than those of heads 0..3 (3.5% per
// block on MI355X, whichever compute units they run on: the second half of
// every token row is slower to read).  Those heads then get their own band
// with kDecodeBandRatio times the wave groups of the first half, so that both
// halves finish together.  Otherwise (including fp8 caches, 1 KB rows, where
// the split measured slower) one band of n_kvg head groups.
void decode_bands(pa::DecodeArgs& a, int wave_groups, int num_kv_heads, bool bf16_rows_2k) {
    if (bf16_rows_2k && num_kv_heads == 8 && a.groups_per_kv == 1 && wave_groups >= 2) {
        const int total = 2 * wave_groups;  // groups of 4 waves
        int g0 = (int)std::lround(total / (1.0 + pa::kDecodeBandRatio));
        g0 = std::max(1, std::min(total - 1, g0));
        a.band_heads = 4;
        a.band_groups[0] = g0;
        a.band_groups[1] = total - g0;
    } else {
        a.band_heads = a.n_kvg;
        a.band_groups[0] = wave_groups;
        a.band_groups[1] = 0;
    }
}

// Decode records for pa_decode_append_noalloc: a fixed array on each device
// that the library keeps until the process ends (each device holds its own
// copy at its own address).  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Device address of this device's scratch, or nullptr if the runtime refuses
// the lookup.
void* scratch_address() {
    static std::atomic<void*> addr[64];
    static std::mutex lock;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> guard(lock);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
        addr[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

}  // namespace

extern "C" {

int pa_decode_set_launch(int32_t waves, int32_t stages, int32_t switch_ticks) {
    if (waves < 0 || waves > pa::kDecodeMaxWaves) return PA_EINVAL;
    if (stages != 0 && stages != 2 && stages != 3 && stages != 4 && stages != 6 && stages != 8) return PA_EINVAL;
    if (switch_ticks < -1 || switch_ticks > 64) return PA_EINVAL;
    g_override_waves.store(waves, std::memory_order_relaxed);
    g_override_stages.store(stages, std::memory_order_relaxed);
    g_override_switch_ticks.store(switch_ticks, std::memory_order_relaxed);
    return PA_OK;
}

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "PA_OK: success";
        case PA_EINVAL: return "PA_EINVAL: an argument is out of its documented range";
        case PA_EUNSUPPORTED: return "PA_EUNSUPPORTED: shape or dtype not supported by this build";
        case PA_EWORKSPACE: return "PA_EWORKSPACE: workspace missing or too small";
        case PA_ELAUNCH: return "PA_ELAUNCH: the HIP runtime refused a kernel launch";
        case PA_ENOMEM: return "PA_ENOMEM: not enough free KV blocks";
        default: return "unknown pa_status";
    }
}

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                         void* stream) {
    int rc = check_storage_dtype(dtype);
    if (rc) return rc;
    if (num_tokens < 0) return PA_EINVAL;
    rc = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks);
    if (rc) return rc;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_EINVAL;
    const long long row_bytes = (long long)num_kv_heads * head_dim * elem_bytes(dtype);
    if (row_bytes > INT32_MAX) return PA_EUNSUPPORTED;
    hipError_t e = pa::launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, num_tokens,
                                                (int)row_bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

int pa_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                             const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype src_dtype,
                             float k_scale, float v_scale, void* stream) {
    int rc = check_dtype(src_dtype);
    if (rc) return rc;
    if (num_tokens < 0) return PA_EINVAL;
    rc = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks);
    if (rc) return rc;
    rc = check_kv_scales(k_scale, v_scale);
    if (rc) return rc;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_EINVAL;
    const long long row_elems = (long long)num_kv_heads * head_dim;
    if (row_elems * 4 > INT32_MAX) return PA_EUNSUPPORTED;
    // the reciprocals, in IEEE single precision, are what multiplies the inputs
    const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
    hipError_t e = pa::launch_reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, num_tokens,
                                                    (int)row_elems, src_dtype == PA_BF16, k_inv, v_inv,
                                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype dtype, void* stream) {
    int rc = check_storage_dtype(dtype);
    if (rc) return rc;
    if (num_pairs < 0) return PA_EINVAL;
    rc = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks);
    if (rc) return rc;
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !pairs) return PA_EINVAL;
    const long long block_bytes = (long long)block_size * num_kv_heads * head_dim * elem_bytes(dtype);
    if (block_bytes > INT32_MAX) return PA_EUNSUPPORTED;
    hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, pairs, num_pairs, (int)block_bytes,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

int pa_stream_read_probe(const void* src, size_t bytes, uint32_t* xor_out, void* stream) {
    if (bytes == 0) return PA_OK;
    if (!src || !xor_out || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0) return PA_EINVAL;
    hipError_t e = pa::launch_stream_read_probe(src, bytes, xor_out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size) {
    (void)max_blocks_per_seq;
    (void)block_size;
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
    if (num_q_heads % num_kv_heads != 0) return 0;
    const int gp = heads_per_wave(num_q_heads / num_kv_heads);
    return decode_ws_layout(gp, head_dim).total;
}

namespace {

// Scales of an FP8 E4M3 cache (dequantized value = scale * stored value).
struct KvScales {
    float k, v;
};

// pa_decode and its fused-append, fp8-cache and timed variants: key/value
// non-null means fused append (the caches are then written); kv8 non-null
// means the caches hold FP8 E4M3 (q and out bf16).  With both, the new rows
// are quantized into the cache by a kernel of their own before the decode
// kernels, which then read every token from the cache.
int decode_impl(void* out, const void* q, const void* key, const void* value, const void* k_cache,
                const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                void* workspace, size_t workspace_bytes, void* stream, void* kernel_start, void* kernel_stop,
                bool fused, bool launch = true, const KvScales* kv8 = nullptr, bool static_scratch = false) {
    int rc = check_dtype(dtype);
    if (rc) return rc;
    if (kv8) {
        if (dtype != PA_BF16) return PA_EUNSUPPORTED;
        rc = check_kv_scales(kv8->k, kv8->v);
        if (rc) return rc;
    }
    if (num_seqs < 0) return PA_EINVAL;
    rc = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks);
    if (rc) return rc;
    rc = check_heads(num_q_heads, num_kv_heads);
    if (rc) return rc;
    if (max_blocks_per_seq <= 0 || max_blocks_per_seq > INT32_MAX / block_size) return PA_EINVAL;
    if (!isfinite(scale)) return PA_EINVAL;
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_EINVAL;
    if (fused && (!key || !value)) return PA_EINVAL;
    if (num_seqs > pa::kDecodeMaxSeqs) return PA_EUNSUPPORTED;
    const int group = num_q_heads / num_kv_heads;
    const int gp = heads_per_wave(group);
    pa::DecodeArgs a;
    a.groups_per_kv = (group + gp - 1) / gp;
    a.n_kvg = num_kv_heads * a.groups_per_kv;
    // wave groups of n_kvg waves (one per head group), as many as fit the
    // persistent grid and the workspace records
    const int wave_groups = std::max(1, std::min(decode_waves(pa::kDecodeWavesPerCU), pa::kDecodeMaxWaves) / a.n_kvg);
    if ((long long)wave_groups * a.n_kvg > pa::kDecodeMaxWaves) return PA_EUNSUPPORTED;
    decode_bands(a, wave_groups, num_kv_heads, dtype == PA_BF16 && !kv8 && head_dim == 128);
    a.waves = (a.band_groups[0] + a.band_groups[1]) * a.band_heads;
    // a caller's workspace is laid out for every launch shape; the fixed
    // scratch for exactly this call's waves, and it must hold them
    const DecodeWsLayout ws = static_scratch ? decode_ws_layout(gp, head_dim, a.waves) : decode_ws_layout(gp, head_dim);
    if (static_scratch) {
        if (ws.total > kNoAllocScratchBytes) return PA_EWORKSPACE;
        workspace = launch ? scratch_address() : nullptr;
        workspace_bytes = kNoAllocScratchBytes;
        if (launch && workspace == nullptr) return PA_ELAUNCH;
    } else if (workspace == nullptr || workspace_bytes < ws.total) {
        return PA_EWORKSPACE;
    }
    if (!launch) return PA_OK;  // arguments checked only

    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    if (fused && kv8) {
        const hipError_t e = pa::launch_append_rows_fp8(key, value, const_cast<void*>(k_cache),
                                                        const_cast<void*>(v_cache), block_tables, max_blocks_per_seq,
                                                        context_lens, num_seqs, num_kv_heads * head_dim,
                                                        1.0f / kv8->k, 1.0f / kv8->v, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return PA_ELAUNCH;
        fused = false;  // the decode kernels read the new token from the cache
    }
    a.new_k = fused ? key : nullptr;
    a.new_v = fused ? value : nullptr;
    a.k_cache_w = fused ? const_cast<void*>(k_cache) : nullptr;
    a.v_cache_w = fused ? const_cast<void*>(v_cache) : nullptr;
    a.ws_split = reinterpret_cast<pa::SplitNote*>(static_cast<char*>(workspace) + ws.split);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.ml);
    a.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.acc);
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = group;
    a.unit_ticks = pa::kDecodeUnitTicks;
    const int ov_ticks = g_override_switch_ticks.load(std::memory_order_relaxed);
    a.switch_ticks = ov_ticks >= 0 ? ov_ticks : pa::kDecodeSwitchTicks;
    a.scale_log2 = (kv8 ? scale * kv8->k : scale) * 1.4426950408889634f;
    a.v_scale = kv8 ? kv8->v : 1.0f;
    const int ov_stages = g_override_stages.load(std::memory_order_relaxed);
    const int stages = ov_stages > 0 ? ov_stages : pa::kDecodeStages;
    hipError_t e = pa::launch_decode(a, dtype == PA_BF16, head_dim, gp, stages, kv8 != nullptr,
                                     static_cast<hipStream_t>(stream),
                                     static_cast<hipEvent_t>(kernel_start), static_cast<hipEvent_t>(kernel_stop));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

}  // namespace

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
              int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype, void* workspace,
              size_t workspace_bytes, void* stream) {
    return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                       workspace, workspace_bytes, stream, nullptr, nullptr, false);
}

int pa_decode_timed(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype, void* workspace,
                    size_t workspace_bytes, void* stream, void* kernel_start, void* kernel_stop) {
    return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                       workspace, workspace_bytes, stream, kernel_start, kernel_stop, false);
}

int pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                  int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                  float k_scale, float v_scale, pa_dtype dtype, void* workspace, size_t workspace_bytes,
                  void* stream) {
    const KvScales kv{k_scale, v_scale};
    return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                       workspace, workspace_bytes, stream, nullptr, nullptr, false, true, &kv);
}

int pa_decode_fp8_timed(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int64_t num_blocks, float scale, float k_scale, float v_scale,
                        pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream, void* kernel_start,
                        void* kernel_stop) {
    const KvScales kv{k_scale, v_scale};
    return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                       workspace, workspace_bytes, stream, kernel_start, kernel_stop, false, true, &kv);
}

int pa_decode_append(void* out, const void* q, const void* key, const void* value, void* k_cache,
                     void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                       workspace, workspace_bytes, stream, nullptr, nullptr, true);
}

int pa_decode_append_timed(void* out, const void* q, const void* key, const void* value, void* k_cache,
                           void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream,
                           void* kernel_start, void* kernel_stop) {
    return decode_impl(out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                       workspace, workspace_bytes, stream, kernel_start, kernel_stop, true);
}

int pa_decode_append_noalloc(void* out, const void* q, const void* key, const void* value, void* k_cache,
                             void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             float scale, pa_dtype dtype, void* stream) {
    return decode_impl(out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                       nullptr, 0, stream, nullptr, nullptr, true, true, nullptr, true);
}

namespace {

// pa_decode_append_graph and its fp8 variant (kv8 non-null): the step's
// launches recorded on a private stream (default priority) in capture mode,
// then instantiated.
int append_graph_impl(void** graph_exec, void* out, const void* q, const void* key, const void* value,
                      void* k_cache, void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                      void* workspace, size_t workspace_bytes, const KvScales* kv8) {
    if (!graph_exec) return PA_EINVAL;
    *graph_exec = nullptr;
    if (num_seqs <= 0) return PA_EINVAL;  // an empty graph is of no use
    int rc = decode_impl(out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                         workspace, workspace_bytes, nullptr, nullptr, nullptr, true, false, kv8);
    if (rc != PA_OK) return rc;
    hipStream_t cs = nullptr;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return PA_ELAUNCH;
    rc = PA_ELAUNCH;
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) == hipSuccess) {
        rc = decode_impl(out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                         workspace, workspace_bytes, cs, nullptr, nullptr, true, true, kv8);
        const hipError_t e = hipStreamEndCapture(cs, &graph);
        if (rc == PA_OK && e != hipSuccess) rc = PA_ELAUNCH;
    }
    if (rc == PA_OK) {
        hipGraphExec_t ge = nullptr;
        if (hipGraphInstantiate(&ge, graph, nullptr, nullptr, 0) == hipSuccess) {
            *graph_exec = ge;
        } else {
            rc = PA_ELAUNCH;
        }
    }
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipStreamDestroy(cs);
    return rc;
}

}  // namespace

int pa_decode_append_graph(void** graph_exec, void* out, const void* q, const void* key, const void* value,
                           void* k_cache, void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes) {
    return append_graph_impl(graph_exec, out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq,
                             context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             scale, dtype, workspace, workspace_bytes, nullptr);
}

int pa_decode_append_fp8(void* out, const void* q, const void* key, const void* value, void* k_cache,
                         void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale, float k_scale,
                         float v_scale, pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
    const KvScales kv{k_scale, v_scale};
    return decode_impl(out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype, workspace,
                       workspace_bytes, stream, nullptr, nullptr, true, true, &kv);
}

int pa_decode_append_fp8_graph(void** graph_exec, void* out, const void* q, const void* key, const void* value,
                               void* k_cache, void* v_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, float scale, float k_scale, float v_scale, pa_dtype dtype,
                               void* workspace, size_t workspace_bytes) {
    const KvScales kv{k_scale, v_scale};
    return append_graph_impl(graph_exec, out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq,
                             context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             scale, dtype, workspace, workspace_bytes, &kv);
}

int pa_graph_launch(void* graph_exec, void* stream) {
    if (!graph_exec) return PA_EINVAL;
    return hipGraphLaunch(static_cast<hipGraphExec_t>(graph_exec), static_cast<hipStream_t>(stream)) == hipSuccess
               ? PA_OK
               : PA_ELAUNCH;
}

int pa_graph_destroy(void* graph_exec) {
    if (!graph_exec) return PA_OK;
    return hipGraphExecDestroy(static_cast<hipGraphExec_t>(graph_exec)) == hipSuccess ? PA_OK : PA_ELAUNCH;
}

size_t pa_prefill_workspace_size(int32_t num_seqs, int32_t total_query_rows, int32_t num_q_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size) {
    (void)num_seqs; (void)total_query_rows; (void)num_q_heads;
    (void)head_dim; (void)max_blocks_per_seq; (void)block_size;
    return 0;
}

namespace {

// pa_prefill_chunk and its fp8-cache variant (kv8 non-null).
int prefill_impl(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                 int32_t max_blocks_per_seq, const int32_t* query_start_loc, int32_t total_query_rows,
                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                 int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                 void* stream, const KvScales* kv8) {
    int rc = check_dtype(dtype);
    if (rc) return rc;
    if (kv8) {
        rc = check_kv_scales(kv8->k, kv8->v);
        if (rc) return rc;
    }
    if (num_seqs < 0 || total_query_rows < 0) return PA_EINVAL;
    rc = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks);
    if (rc) return rc;
    rc = check_heads(num_q_heads, num_kv_heads);
    if (rc) return rc;
    if (max_blocks_per_seq <= 0 || max_blocks_per_seq > INT32_MAX / block_size) return PA_EINVAL;
    if (!isfinite(scale)) return PA_EINVAL;
    if (num_seqs == 0 || total_query_rows == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start_loc || !context_lens)
        return PA_EINVAL;
    if (dtype != PA_BF16) return PA_EUNSUPPORTED;
    const int group = num_q_heads / num_kv_heads;
    if (group > pa::kPrefillMaxGroup) return PA_EUNSUPPORTED;
    int gp = 1;
    while (gp < group) gp *= 2;
    pa::PrefillArgs a;
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.query_start_loc = query_start_loc;
    a.context_lens = context_lens;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = group;
    a.scale_log2 = (kv8 ? scale * kv8->k : scale) * 1.4426950408889634f;
    a.v_scale = kv8 ? kv8->v : 1.0f;
    hipError_t e = pa::launch_prefill(a, head_dim, total_query_rows, gp, kv8 != nullptr,
                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

}  // namespace

int pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* query_start_loc, int32_t total_query_rows,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                     float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    return prefill_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, query_start_loc,
                        total_query_rows, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, scale, dtype, stream, nullptr);
}

int pa_prefill_chunk_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* query_start_loc, int32_t total_query_rows,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                         float scale, float k_scale, float v_scale, pa_dtype dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    const KvScales kv{k_scale, v_scale};
    return prefill_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, query_start_loc,
                        total_query_rows, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, scale, dtype, stream, &kv);
}

}  // extern "C"
