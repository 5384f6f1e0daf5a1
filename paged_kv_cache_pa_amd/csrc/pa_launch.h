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
};

// Returns 0 on success, else the hipError_t of the failed launch.
int launch_decode(const DecodeLaunch &l, void *stream);

int launch_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       const int32_t *slots, int32_t n, int32_t num_blocks, int32_t block_size,
                       int32_t hkv, int64_t row_bytes, int32_t layout, void *stream);

int launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int32_t n,
                       int32_t num_blocks, int64_t block_bytes, void *stream);

const char *hip_error_name(int err);
const char *kernel_build_info();

}  // namespace pa
