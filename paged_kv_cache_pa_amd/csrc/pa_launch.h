// pa_launch.h -- internal interface between the argument-checking C ABI
// (pa_abi.cpp) and the gfx950 kernels (pa_kernels.hip).  Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pa {

// One decode launch, already validated.  dense = false: paged pool.
struct DecodeLaunch {
    const void *q, *k, *v;
    const int32_t *tables;   // paged only
    const int32_t *lens;
    void *out;
    float *ws;               // split-K workspace (partials, then (m, l) pairs)
    float scale;
    int32_t S, Hq, Hkv, D, dtype;
    int32_t B, MBS, NB;      // paged only
    int32_t max_ctx;         // clamp for every context length
    int32_t PS;              // 0 = no split, else partition size (tokens)
    int32_t P;               // number of partitions (grid z), >= 1
    int64_t pos_stride;      // dense only: max_seq_len
    int32_t layout;          // 0 token-major, 1 head-major
    bool dense;
    // Append mode (paged only): newest token rows [S, Hkv, D] written to
    // position n - 1 of each sequence through k_w / v_w while attending.
    const void *k_new = nullptr, *v_new = nullptr;
    void *k_w = nullptr, *v_w = nullptr;
    // Shared prefixes (paged, 16-bit, n_groups > 0): a grouped launch first
    // computes, once per group, the leading partitions (of size PSg tokens)
    // its members share and writes each member's count of them to skip[S];
    // the usual launch then computes the rest.
    const int32_t *group_start = nullptr;   // [n_groups + 1], device
    const int32_t *group_shared = nullptr;  // [n_groups], device
    int32_t *skip = nullptr;                // [S], device (in the workspace)
    int32_t n_groups = 0;
    int32_t max_shared_blocks = 0;          // bound on group_shared (host)
    int32_t PSg = 0;
};

// Returns 0 on success, else the hipError_t of the failed launch.
int launch_decode(const DecodeLaunch &l, void *stream);

// One prefill launch (multi-token queries), already validated; 16-bit only.
struct PrefillLaunch {
    const void *q, *k, *v;
    const int32_t *tables, *lens, *qstart;
    void *out;
    float scale;
    int32_t S, Hq, Hkv, D, dtype;
    int32_t B, MBS, NB;
    int32_t max_ctx;     // clamp for every context length
    int32_t max_q;       // clamp for every chunk length; sizes the grid
    int32_t total_rows;  // rows of q and out
    int32_t layout;
};

// Query rows of a chunk one prefill workgroup covers (grid z = ceil(max_q /
// kPrefillTileRows), at most 65535).
constexpr int kPrefillTileRows = 128;

int launch_prefill(const PrefillLaunch &l, void *stream);

int launch_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       const int32_t *slots, int32_t n, int32_t num_blocks, int32_t block_size,
                       int32_t hkv, int64_t row_bytes, int32_t layout, void *stream);

// Most layers one launch of a multi-layer entry point takes (the pointer
// arrays travel by value in the kernel argument).
constexpr int kMaxLayers = 64;

// New rows of every layer (up to kMaxLayers per launch): per layer the
// token rows [n, Hkv, D] and the pools; one slot mapping for all layers.
struct CacheWriteLayers {
    const void *k_new[kMaxLayers], *v_new[kMaxLayers];
    void *k_cache[kMaxLayers], *v_cache[kMaxLayers];
    int32_t layers;  // 1 .. kMaxLayers
};
int launch_cache_write_layers(const CacheWriteLayers &w, const int32_t *slots, int32_t n,
                              int32_t num_blocks, int32_t block_size, int32_t hkv,
                              int64_t row_bytes, int32_t layout, void *stream);

// Whole-block moves between two pools (or within one) for up to
// kMaxLayers layers.
struct BlockMove {
    const void *src_k[kMaxLayers], *src_v[kMaxLayers];
    void *dst_k[kMaxLayers], *dst_v[kMaxLayers];
    const int32_t *pairs;    // [n][2] (src, dst), device-accessible
    int64_t block_bytes;     // one block of one of K / V: B * Hkv * D * e
    int32_t layers;          // 1 .. kMaxLayers
    int32_t src_blocks, dst_blocks;
};

int launch_move_blocks(const BlockMove &m, int32_t n, void *stream);

// Bytes of the fixed device array that serves pa_decode_no_alloc as its
// split-K workspace (one array per device).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;

// Device address of that array on the current device (looked up once per
// device, then cached).  Returns 0, or the hipError_t of the lookup.
int scratch_address(void **ptr);

const char *hip_error_name(int err);
const char *kernel_build_info();

}  // namespace pa
