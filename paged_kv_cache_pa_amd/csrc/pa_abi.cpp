// pa_abi.cpp -- the C ABI declared in include/pa.h: host-side argument
// checks, grid sizing, then one call into the kernel launchers.  No HIP call
// happens before every check has passed, so every error path is testable
// without a GPU.
#include <stddef.h>
#include <stdint.h>

#include "pa.h"
#include "pa_launch.h"

namespace {

// HIP error code behind the calling thread's most recent PA_ERR_HIP.
thread_local int last_hip_error = 0;

int hip_status(int e) {
    if (e == 0) return PA_OK;
    last_hip_error = e;
    return PA_ERR_HIP;
}

int elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : 2; }

bool dtype_ok(int32_t dtype) { return dtype == PA_F32 || dtype == PA_F16 || dtype == PA_BF16; }

bool pow2_in(int32_t x, int32_t lo, int32_t hi) {
    return x >= lo && x <= hi && (x & (x - 1)) == 0;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool layout_ok(int32_t layout) {
    return layout == PA_LAYOUT_TOKEN_MAJOR || layout == PA_LAYOUT_HEAD_MAJOR;
}

// Checks shared by the paged and dense decode.  ``row_limit`` is the most
// tokens a sequence can hold (MBS * B paged, max_seq_len dense); ``granule``
// is what partition_size must be a multiple of.
int check_decode_shape(const pa_decode_params *p, int64_t row_limit, int32_t granule) {
    if (!p) return PA_ERR_NULL;
    if (!dtype_ok(p->dtype)) return PA_ERR_DTYPE;
    if (p->num_seqs < 0 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1)
        return PA_ERR_SHAPE;
    if (p->num_q_heads % p->num_kv_heads) return PA_ERR_SHAPE;
    if (!layout_ok(p->layout)) return PA_ERR_SHAPE;
    if (p->max_context_len < 0 || p->max_context_len > row_limit) return PA_ERR_SHAPE;
    if (p->partition_size < 0 || (p->partition_size && p->partition_size % granule))
        return PA_ERR_SHAPE;
    if (p->head_dim != 64 && p->head_dim != 128) return PA_ERR_UNSUPPORTED;
    // Up to 8 query heads per kv head in every type; up to 16 in fp16 / bf16
    // (the matrix-core kernel's score tile has 16 head columns).
    const int32_t group = p->num_q_heads / p->num_kv_heads;
    if (group > 16 || (group > 8 && p->dtype == PA_F32)) return PA_ERR_UNSUPPORTED;
    // In-step row offsets are 32-bit: 16 token rows must span under 4 GiB.
    if ((int64_t)p->num_kv_heads * p->head_dim * elem_bytes(p->dtype) > (1 << 27))
        return PA_ERR_UNSUPPORTED;
    // (sequence, head) rows are indexed with 31 bits.  The decode grid is one
    // workgroup (of up to 512 threads) per (sequence, kv head, partition), the
    // merge grid one of 256 threads per (sequence, query head); a launch's
    // thread count must fit 32 bits.
    if ((int64_t)p->num_seqs * p->num_q_heads > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    if (p->partition_size &&
        ((int64_t)p->max_context_len + p->partition_size - 1) / p->partition_size > 65535)
        return PA_ERR_UNSUPPORTED;
    {
        const int64_t parts = p->partition_size && p->max_context_len > p->partition_size
                                  ? ((int64_t)p->max_context_len + p->partition_size - 1) /
                                        p->partition_size
                                  : 1;
        if ((int64_t)p->num_seqs * p->num_kv_heads * parts * 512 > 0xFFFFFFFFll)
            return PA_ERR_UNSUPPORTED;
        if (parts > 1 && (int64_t)p->num_seqs * p->num_q_heads * 256 > 0xFFFFFFFFll)
            return PA_ERR_UNSUPPORTED;
    }
    return PA_OK;
}

int check_paged_shape(const pa_decode_params *p) {
    if (!p) return PA_ERR_NULL;
    if (!pow2_in(p->block_size, 1, 256)) return PA_ERR_SHAPE;
    if (p->max_blocks_per_seq < 1 || p->num_blocks < 1) return PA_ERR_SHAPE;
    return check_decode_shape(p, (int64_t)p->max_blocks_per_seq * p->block_size, p->block_size);
}

int32_t num_partitions(const pa_decode_params *p) {
    if (p->partition_size == 0 || p->max_context_len <= p->partition_size) return 1;
    return (p->max_context_len + p->partition_size - 1) / p->partition_size;
}

// Partials [S, Hq, P, D] and (m, l) [S, Hq, P, 2] in fp32.
size_t workspace_bytes(const pa_decode_params *p) {
    const int32_t P = num_partitions(p);
    if (P <= 1) return 0;
    return (size_t)p->num_seqs * p->num_q_heads * P * (p->head_dim + 2) * sizeof(float);
}

// Shared-prefix decode: the partials as above, then the per-sequence count
// of leading partitions the grouped launch computed (int32 [S]), 16-byte
// aligned.
size_t skip_offset(const pa_decode_params *p) { return (workspace_bytes(p) + 15) & ~(size_t)15; }
size_t shared_workspace_bytes(const pa_decode_params *p) {
    return skip_offset(p) + (((size_t)p->num_seqs * 4 + 15) & ~(size_t)15);
}

struct Groups {
    const int32_t *start, *shared;
    int32_t n, max_shared;
};

// Pointer checks of a decode call with at least one sequence.
int check_decode_ptrs(const void *q, const void *k, const void *v, const int32_t *tables,
                      const int32_t *lens, const void *out, bool dense) {
    if (!q || !k || !v || !lens || !out || (!dense && !tables)) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PA_ERR_ALIGN;
    if (((uintptr_t)lens & 3u) || (tables && ((uintptr_t)tables & 3u))) return PA_ERR_ALIGN;
    return PA_OK;
}

int run_decode(const void *q, const void *k, const void *v, const int32_t *tables,
               const int32_t *lens, float scale, void *out, const pa_decode_params *p,
               void *ws, size_t ws_bytes, void *stream, bool dense, int32_t max_seq_len,
               const void *k_new = nullptr, const void *v_new = nullptr,
               const Groups *grp = nullptr) {
    if (p->num_seqs == 0) return PA_OK;
    const int pst = check_decode_ptrs(q, k, v, tables, lens, out, dense);
    if (pst != PA_OK) return pst;
    const size_t need = grp ? shared_workspace_bytes(p) : workspace_bytes(p);
    if (need) {
        if (!ws || ws_bytes < need) return PA_ERR_WORKSPACE;
        if (!aligned16(ws)) return PA_ERR_ALIGN;
    }
    pa::DecodeLaunch l;
    l.q = q;
    l.k = k;
    l.v = v;
    l.tables = tables;
    l.lens = lens;
    l.out = out;
    l.ws = (float *)ws;
    l.scale = scale;
    l.S = p->num_seqs;
    l.Hq = p->num_q_heads;
    l.Hkv = p->num_kv_heads;
    l.D = p->head_dim;
    l.dtype = p->dtype;
    l.B = dense ? 0 : p->block_size;
    l.MBS = dense ? 0 : p->max_blocks_per_seq;
    l.NB = dense ? 0 : p->num_blocks;
    l.max_ctx = p->max_context_len;
    l.P = num_partitions(p);
    l.PS = l.P > 1 ? p->partition_size : 0;
    l.pos_stride = dense ? max_seq_len : 0;
    l.layout = p->layout;
    l.dense = dense;
    if (k_new) {  // append mode: the pools are written too
        l.k_new = k_new;
        l.v_new = v_new;
        l.k_w = const_cast<void *>(k);
        l.v_w = const_cast<void *>(v);
    }
    if (grp && grp->n > 0) {
        l.group_start = grp->start;
        l.group_shared = grp->shared;
        l.n_groups = grp->n;
        l.max_shared_blocks = grp->max_shared;
        l.PSg = p->partition_size;
        l.skip = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + skip_offset(p));
    }
    const int e = pa::launch_decode(l, stream);
    return hip_status(e);
}

int check_cache_params(const pa_cache_params *p) {
    if (!p) return PA_ERR_NULL;
    if (!dtype_ok(p->dtype)) return PA_ERR_DTYPE;
    if (p->num_blocks < 1 || p->num_kv_heads < 1 || p->head_dim < 1) return PA_ERR_SHAPE;
    if (!pow2_in(p->block_size, 1, 256)) return PA_ERR_SHAPE;
    if (((int64_t)p->head_dim * elem_bytes(p->dtype)) % 16) return PA_ERR_SHAPE;
    if (!layout_ok(p->layout)) return PA_ERR_SHAPE;
    return PA_OK;
}

// Shared by copy_blocks (one layer, one pool), copy_blocks_layers and
// swap_blocks (two pools): validate, then one launch per kMaxLayers layers.
int move_blocks(const void *const *src_k, const void *const *src_v, int32_t src_blocks,
                void *const *dst_k, void *const *dst_v, int32_t dst_blocks, int32_t layers,
                const int32_t *pairs, int32_t n, const pa_cache_params *p, void *stream) {
    const int st = check_cache_params(p);
    if (st != PA_OK) return st;
    if (n < 0 || layers < 1) return PA_ERR_SHAPE;
    if (n == 0) return PA_OK;
    if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PA_ERR_NULL;
    for (int32_t l = 0; l < layers; ++l) {
        if (!src_k[l] || !src_v[l] || !dst_k[l] || !dst_v[l]) return PA_ERR_NULL;
        if (!aligned16(src_k[l]) || !aligned16(src_v[l]) || !aligned16(dst_k[l]) ||
            !aligned16(dst_v[l]))
            return PA_ERR_ALIGN;
    }
    if ((uintptr_t)pairs & 3u) return PA_ERR_ALIGN;
    const int64_t blk = (int64_t)p->block_size * p->num_kv_heads * p->head_dim *
                        elem_bytes(p->dtype);
    // grid x = pairs * layers * 2 workgroups of 256 threads; grid y = 16 KiB chunks
    const int32_t per = layers < pa::kMaxLayers ? layers : pa::kMaxLayers;
    if ((int64_t)n * per * 2 * 256 >= ((int64_t)1 << 32)) return PA_ERR_UNSUPPORTED;
    if (blk / 16 > (int64_t)65535 * 256 * 4) return PA_ERR_UNSUPPORTED;
    pa::BlockMove m;
    m.pairs = pairs;
    m.block_bytes = blk;
    m.src_blocks = src_blocks;
    m.dst_blocks = dst_blocks;
    for (int32_t l0 = 0; l0 < layers; l0 += pa::kMaxLayers) {
        m.layers = layers - l0 < pa::kMaxLayers ? layers - l0 : pa::kMaxLayers;
        for (int32_t l = 0; l < m.layers; ++l) {
            m.src_k[l] = src_k[l0 + l];
            m.src_v[l] = src_v[l0 + l];
            m.dst_k[l] = dst_k[l0 + l];
            m.dst_v[l] = dst_v[l0 + l];
        }
        const int e = pa::launch_move_blocks(m, n, stream);
        if (e) return hip_status(e);
    }
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode_workspace_size(const pa_decode_params *p, size_t *bytes) {
    if (!bytes || !p) return PA_ERR_NULL;
    *bytes = 0;
    // The size depends on S, Hq, D, max_context_len and partition_size only,
    // so the same call serves pa_decode and pa_decode_dense.
    const int st = check_decode_shape(p, INT32_MAX, 1);
    if (st != PA_OK) return st;
    *bytes = workspace_bytes(p);
    return PA_OK;
}

int pa_decode(const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, float scale, void *out,
              const pa_decode_params *p, void *workspace, size_t ws_bytes, void *stream) {
    const int st = check_paged_shape(p);
    if (st != PA_OK) return st;
    return run_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, p, workspace,
                      ws_bytes, stream, false, 0);
}

int pa_decode_shared_workspace_size(const pa_decode_params *p, size_t *bytes) {
    if (!bytes || !p) return PA_ERR_NULL;
    *bytes = 0;
    const int st = check_decode_shape(p, INT32_MAX, 1);
    if (st != PA_OK) return st;
    *bytes = shared_workspace_bytes(p);
    return PA_OK;
}

int pa_decode_shared(const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, const int32_t *context_lens,
                     const int32_t *group_start, const int32_t *group_shared, int32_t num_groups,
                     int32_t max_shared_blocks, float scale, void *out,
                     const pa_decode_params *p, void *workspace, size_t ws_bytes, void *stream) {
    const int st = check_paged_shape(p);
    if (st != PA_OK) return st;
    if (p->dtype != PA_F16 && p->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (p->partition_size < 1) return PA_ERR_SHAPE;
    if (num_groups < 0 || num_groups > p->num_seqs) return PA_ERR_SHAPE;
    if (max_shared_blocks < 0 || max_shared_blocks > p->max_blocks_per_seq) return PA_ERR_SHAPE;
    if (p->num_seqs == 0) return PA_OK;
    if (num_groups > 0) {
        if (!group_start || !group_shared) return PA_ERR_NULL;
        if (((uintptr_t)group_start & 3u) || ((uintptr_t)group_shared & 3u)) return PA_ERR_ALIGN;
        // grouped grid: (group, kv head, shared partition) workgroups of up to 512 threads
        const int64_t sp = (int64_t)max_shared_blocks * p->block_size / p->partition_size;
        const int64_t pg = sp < 1 ? 1 : (sp > num_partitions(p) ? num_partitions(p) : sp);
        if ((int64_t)num_groups * p->num_kv_heads * pg * 512 > 0xFFFFFFFFll)
            return PA_ERR_UNSUPPORTED;
    }
    const Groups g{group_start, group_shared, num_groups, max_shared_blocks};
    return run_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, p, workspace,
                      ws_bytes, stream, false, 0, nullptr, nullptr, &g);
}

static_assert(PA_NO_ALLOC_SCRATCH_BYTES == pa::kNoAllocScratchBytes,
              "the header states the scratch array's size");

int pa_decode_no_alloc(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       void *out, const pa_decode_params *p, void *stream) {
    const int st = check_paged_shape(p);
    if (st != PA_OK) return st;
    if (p->num_seqs == 0) return PA_OK;
    const int pst = check_decode_ptrs(q, k_cache, v_cache, block_tables, context_lens, out, false);
    if (pst != PA_OK) return pst;
    const size_t need = workspace_bytes(p);
    if (need > PA_NO_ALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
    void *ws = nullptr;
    if (need) {  // every check has passed: the first HIP call
        const int e = pa::scratch_address(&ws);
        if (e) return hip_status(e);
    }
    return run_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, p, ws,
                      need ? PA_NO_ALLOC_SCRATCH_BYTES : 0, stream, false, 0);
}

int pa_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache,
                     void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                     float scale, void *out, const pa_decode_params *p, void *workspace,
                     size_t ws_bytes, void *stream) {
    const int st = check_paged_shape(p);
    if (st != PA_OK) return st;
    if (p->num_seqs == 0) return PA_OK;
    if (!k_new || !v_new) return PA_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return PA_ERR_ALIGN;
    return run_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, p, workspace,
                      ws_bytes, stream, false, 0, k_new, v_new);
}

int pa_decode_dense(const void *q, const void *k, const void *v, const int32_t *context_lens,
                    float scale, void *out, const pa_decode_params *p, int32_t max_seq_len,
                    void *workspace, size_t ws_bytes, void *stream) {
    if (!p) return PA_ERR_NULL;
    if (max_seq_len < 1) return PA_ERR_SHAPE;
    const int st = check_decode_shape(p, max_seq_len, 16);
    if (st != PA_OK) return st;
    return run_decode(q, k, v, nullptr, context_lens, scale, out, p, workspace, ws_bytes, stream,
                      true, max_seq_len);
}

int pa_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                   const int32_t *slot_mapping, int32_t num_tokens, const pa_cache_params *p,
                   void *stream) {
    const int st = check_cache_params(p);
    if (st != PA_OK) return st;
    if (num_tokens < 0) return PA_ERR_SHAPE;
    if (num_tokens == 0) return PA_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
        ((uintptr_t)slot_mapping & 3u))
        return PA_ERR_ALIGN;
    const int64_t row = (int64_t)p->head_dim * elem_bytes(p->dtype);  // one head's row
    const int e = pa::launch_cache_write(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens,
                                         p->num_blocks, p->block_size, p->num_kv_heads, row,
                                         p->layout, stream);
    return hip_status(e);
}

int pa_prefill(const void *q, const void *k_cache, const void *v_cache,
               const int32_t *block_tables, const int32_t *context_lens,
               const int32_t *query_start, float scale, void *out,
               const pa_prefill_params *p, void *stream) {
    if (!p) return PA_ERR_NULL;
    if (!dtype_ok(p->dtype)) return PA_ERR_DTYPE;
    if (p->num_seqs < 0 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1 ||
        p->total_query_rows < 0 || p->max_query_len < 0 || p->max_context_len < 0)
        return PA_ERR_SHAPE;
    if (p->num_q_heads % p->num_kv_heads) return PA_ERR_SHAPE;
    if (!layout_ok(p->layout)) return PA_ERR_SHAPE;
    if (!pow2_in(p->block_size, 1, 256)) return PA_ERR_SHAPE;
    if (p->max_blocks_per_seq < 1 || p->num_blocks < 1) return PA_ERR_SHAPE;
    if (p->max_context_len > (int64_t)p->max_blocks_per_seq * p->block_size) return PA_ERR_SHAPE;
    if (p->max_query_len > p->max_context_len) return PA_ERR_SHAPE;
    if (p->dtype == PA_F32) return PA_ERR_UNSUPPORTED;
    if (p->head_dim != 64 && p->head_dim != 128) return PA_ERR_UNSUPPORTED;
    // grid (heads, sequences, row tiles): y and z are limited to 65535
    if (p->num_seqs > 65535) return PA_ERR_UNSUPPORTED;
    if (((int64_t)p->max_query_len + pa::kPrefillTileRows - 1) / pa::kPrefillTileRows > 65535)
        return PA_ERR_UNSUPPORTED;
    if ((int64_t)p->total_query_rows * p->num_q_heads > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    if (p->num_seqs == 0 || p->total_query_rows == 0 || p->max_query_len == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
        return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return PA_ERR_ALIGN;
    if (((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u) ||
        ((uintptr_t)query_start & 3u))
        return PA_ERR_ALIGN;
    pa::PrefillLaunch l;
    l.q = q;
    l.k = k_cache;
    l.v = v_cache;
    l.tables = block_tables;
    l.lens = context_lens;
    l.qstart = query_start;
    l.out = out;
    l.scale = scale;
    l.S = p->num_seqs;
    l.Hq = p->num_q_heads;
    l.Hkv = p->num_kv_heads;
    l.D = p->head_dim;
    l.dtype = p->dtype;
    l.B = p->block_size;
    l.MBS = p->max_blocks_per_seq;
    l.NB = p->num_blocks;
    l.max_ctx = p->max_context_len;
    l.max_q = p->max_query_len;
    l.total_rows = p->total_query_rows;
    l.layout = p->layout;
    return hip_status(pa::launch_prefill(l, stream));
}

int pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *block_pairs, int32_t num_pairs,
                   const pa_cache_params *p, void *stream) {
    void *k[1] = {k_cache}, *v[1] = {v_cache};
    return pa_copy_blocks_layers(k, v, 1, block_pairs, num_pairs, p, stream);
}

int pa_cache_write_layers(const void *const *k_new, const void *const *v_new,
                          void *const *k_caches, void *const *v_caches, int32_t num_layers,
                          const int32_t *slot_mapping, int32_t num_tokens,
                          const pa_cache_params *p, void *stream) {
    const int st = check_cache_params(p);
    if (st != PA_OK) return st;
    if (num_tokens < 0 || num_layers < 1) return PA_ERR_SHAPE;
    if (num_tokens == 0) return PA_OK;
    if (!k_new || !v_new || !k_caches || !v_caches || !slot_mapping) return PA_ERR_NULL;
    for (int32_t l = 0; l < num_layers; ++l) {
        if (!k_new[l] || !v_new[l] || !k_caches[l] || !v_caches[l]) return PA_ERR_NULL;
        if (!aligned16(k_new[l]) || !aligned16(v_new[l]) || !aligned16(k_caches[l]) ||
            !aligned16(v_caches[l]))
            return PA_ERR_ALIGN;
    }
    if ((uintptr_t)slot_mapping & 3u) return PA_ERR_ALIGN;
    const int64_t row = (int64_t)p->head_dim * elem_bytes(p->dtype);  // one head's row
    pa::CacheWriteLayers w;
    for (int32_t l0 = 0; l0 < num_layers; l0 += pa::kMaxLayers) {
        w.layers = num_layers - l0 < pa::kMaxLayers ? num_layers - l0 : pa::kMaxLayers;
        for (int32_t l = 0; l < w.layers; ++l) {
            w.k_new[l] = k_new[l0 + l];
            w.v_new[l] = v_new[l0 + l];
            w.k_cache[l] = k_caches[l0 + l];
            w.v_cache[l] = v_caches[l0 + l];
        }
        const int e = pa::launch_cache_write_layers(w, slot_mapping, num_tokens, p->num_blocks,
                                                    p->block_size, p->num_kv_heads, row,
                                                    p->layout, stream);
        if (e) return hip_status(e);
    }
    return PA_OK;
}

int pa_copy_blocks_layers(void *const *k_caches, void *const *v_caches, int32_t num_layers,
                          const int32_t *block_pairs, int32_t num_pairs,
                          const pa_cache_params *p, void *stream) {
    return move_blocks(k_caches, v_caches, p ? p->num_blocks : 0, k_caches, v_caches,
                       p ? p->num_blocks : 0, num_layers, block_pairs, num_pairs, p, stream);
}

int pa_swap_blocks(void *const *dst_k, void *const *dst_v, int32_t dst_num_blocks,
                   const void *const *src_k, const void *const *src_v, int32_t src_num_blocks,
                   int32_t num_layers, const int32_t *block_pairs, int32_t num_pairs,
                   const pa_cache_params *p, void *stream) {
    if (dst_num_blocks < 1 || src_num_blocks < 1) return PA_ERR_SHAPE;
    return move_blocks(src_k, src_v, src_num_blocks, dst_k, dst_v, dst_num_blocks, num_layers,
                       block_pairs, num_pairs, p, stream);
}

const char *pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "PA_OK: success";
        case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
        case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size is out of range or inconsistent";
        case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unknown element type";
        case PA_ERR_ALIGN: return "PA_ERR_ALIGN: a data pointer is not aligned";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim or head grouping not built";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: split-K workspace missing or too small";
        case PA_ERR_HIP: return "PA_ERR_HIP: the HIP launch failed";
        case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: the block pool cannot supply the call";
        case PA_ERR_STATE: return "PA_ERR_STATE: sequence handle not live, repeated or on the wrong side";
        case PA_ERR_SCRATCH:
            return "PA_ERR_SCRATCH: the split-K partials need more than the fixed scratch array "
                   "of pa_decode_no_alloc holds (PA_NO_ALLOC_SCRATCH_BYTES)";
    }
    return "unknown pa_status";
}

const char *pa_build_info(void) { return pa::kernel_build_info(); }

const char *pa_last_hip_error(void) {
    return last_hip_error ? pa::hip_error_name(last_hip_error) : "";
}

}  // extern "C"
