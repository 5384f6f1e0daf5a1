/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-KV-cache attention library.
 *
 * Pages cited (by title, then section / equation / figure):
 *   [Kwon] "Efficient Memory Management for Large Language Model Serving
 *          with PagedAttention" (paper summary page)
 *   [Int]  "vLLM Internals: PagedAttention, Continuous Batching, and Where
 *          the 2-4x Comes From"
 *   [Res]  "Paged Attention: Managing the KV Cache Like Virtual Memory"
 *   [Os]   the blog.teliaz.com page on PagedAttention as OS paging, section
 *          "PagedAttention: the OS metaphor, made literal"
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers named as device pointers must point to GPU memory on the
 *    current HIP device; parameter structs are host memory read during the
 *    call only.  The caller owns every buffer, including the split-K
 *    workspace.  The library allocates, frees and synchronises nothing.
 *    Between calls it keeps only a cache of per-device occupancy figures
 *    (filled on first use, guarded by a lock), per thread the name of the
 *    last HIP error (pa_last_hip_error), and for pa_decode_no_alloc a fixed
 *    16 MiB device array per device with its cached address (see there);
 *    calls are reentrant, except that pa_decode_no_alloc calls overlapping
 *    on one device share that array.
 *  - Work is enqueued on ``stream`` (a hipStream_t; NULL = the legacy default
 *    stream) and the call returns at once.  Buffers must stay valid until the
 *    stream has passed the work.
 *  - Every call returns a pa_status.  All argument checks run on the host
 *    before any HIP call, so a non-PA_OK status means nothing was enqueued.
 *    Only PA_ERR_HIP reports a failure of the launch itself.
 *  - Element types: PA_F32, PA_F16 (IEEE binary16), PA_BF16.  q, the caches,
 *    the new tokens and out share one dtype.  Indices are int32.
 *  - Conditions that live in device memory (context lengths, table entries,
 *    slots, pair ids) cannot be checked on the host.  Out-of-range values
 *    never cause an out-of-bounds access: each is clamped or skipped as
 *    stated per entry point, and the result for that sequence / token /
 *    pair is then unspecified.
 *
 * Layouts (row-major, innermost last):
 *   q, out              [num_seqs, num_q_heads, head_dim]
 *   k_cache, v_cache    token-major: [num_blocks, block_size, num_kv_heads, head_dim]
 *                       head-major:  [num_blocks, num_kv_heads, block_size, head_dim]
 *   block_tables        [num_seqs, max_blocks_per_seq]   int32
 *   context_lens        [num_seqs]                       int32
 *   dense k, v          token-major: [num_seqs, max_seq_len, num_kv_heads, head_dim]
 *                       head-major:  [num_seqs, num_kv_heads, max_seq_len, head_dim]
 *   k_new, v_new        [num_tokens, num_kv_heads, head_dim]
 *   slot_mapping        [num_tokens]                     int32
 *   block_pairs         [num_pairs, 2] (src, dst)        int32
 * In the token-major layout one block is exactly block_size consecutive
 * token rows of the token-major dense layout, so paged and dense inputs can
 * hold identical bytes.  The head-major layout keeps each (block, kv head)
 * contiguous ([Res] "A paged KV cache, in code": a pool of [blocks, kv
 * heads, 16 tokens, head dimension]); the decode kernel streams it faster.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* Order of the dimensions inside a block (paged) or a sequence (dense). */
typedef enum { PA_LAYOUT_TOKEN_MAJOR = 0, PA_LAYOUT_HEAD_MAJOR = 1 } pa_kv_layout;

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL                   */
    PA_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be,
                                or inconsistent with another                 */
    PA_ERR_DTYPE = -3,       /* dtype is not one of pa_dtype                 */
    PA_ERR_ALIGN = -4,       /* a data pointer is not 16-byte aligned        */
    PA_ERR_UNSUPPORTED = -5, /* valid but not built: head_dim not 64/128,
                                query heads per kv head above 8 (fp32) or
                                16 (fp16 / bf16), more than
                                65535 partitions or 2^31 - 1 (seq, head) rows,
                                a token row (all kv heads) above 128 MiB      */
    PA_ERR_WORKSPACE = -6,   /* split-K workspace missing or too small       */
    PA_ERR_HIP = -7,         /* the HIP launch failed                         */
    PA_ERR_NO_BLOCKS = -8,   /* block manager: the pool cannot supply the
                                blocks a call needs (nothing was changed)    */
    PA_ERR_STATE = -9,       /* block manager: a sequence handle is not live,
                                repeated, or on the wrong side for the call  */
    PA_ERR_SCRATCH = -10     /* pa_decode_no_alloc: the split-K partials need
                                more than PA_NO_ALLOC_SCRATCH_BYTES          */
} pa_status;

/* Shape of one decode call (host struct). */
typedef struct {
    int32_t num_seqs;           /* S >= 0; S == 0 enqueues nothing           */
    int32_t num_q_heads;        /* Hq >= 1                                    */
    int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0; Hq / Hkv <= 8,    */
                                /* <= 16 for fp16 / bf16 (PA_ERR_UNSUPPORTED) */
    int32_t head_dim;           /* D in {64, 128}                             */
    int32_t block_size;         /* B, a power of two in [1, 256]; paged only  */
    int32_t max_blocks_per_seq; /* row stride of block_tables; paged only     */
    int32_t num_blocks;         /* NB, pool size; paged only                  */
    int32_t max_context_len;    /* host-known bound on every context_lens[s]; */
                                /* sizes the split-K grid. Paged: <= MBS * B  */
    int32_t partition_size;     /* 0: one workgroup covers a whole sequence;  */
                                /* else split-K over partitions of this many  */
                                /* tokens, a multiple of B (paged) / of 16    */
    int32_t dtype;              /* pa_dtype                                   */
    int32_t layout;             /* pa_kv_layout of the K and V buffers        */
} pa_decode_params;

/* Shape of the pool for cache_write / copy_blocks (host struct). */
typedef struct {
    int32_t num_blocks;   /* NB >= 1                                          */
    int32_t block_size;   /* B, a power of two in [1, 256]                    */
    int32_t num_kv_heads; /* Hkv >= 1                                         */
    int32_t head_dim;     /* D >= 1 with D * element bytes a multiple of 16   */
    int32_t dtype;        /* pa_dtype                                         */
    int32_t layout;       /* pa_kv_layout of the pool                         */
} pa_cache_params;

/*
 * Bytes of workspace pa_decode / pa_decode_dense need for ``p``: zero when
 * partition_size == 0 or max_context_len <= partition_size, otherwise
 * num_seqs * num_q_heads * ceil(max_context_len / partition_size)
 * * (head_dim + 2) * 4 (fp32 partials).  Only the fields the size depends on are checked
 * (dtype, the head counts, head_dim, num_seqs, max_context_len >= 0,
 * partition_size >= 0); block_size, max_blocks_per_seq and num_blocks are
 * not read.  Writes the size to *bytes (0 on error); returns a pa_status.
 */
int pa_decode_workspace_size(const pa_decode_params *p, size_t *bytes);

/*
 * Paged single-query (decode) attention.  For every sequence s and query
 * head h, with n = context_lens[s] and g = h / (Hq / Hkv):
 *   out[s][h] = sum_{t<n} a_t v_t,  a_t = exp(x_t) / sum_{u<n} exp(x_u),
 *   x_t = scale * q[s][h] . k_t,
 * where token t is read from physical block block_tables[s][t / B], offset
 * t % B, kv head g of k_cache / v_cache in p->layout ([Kwon] §3.4 "PagedAttention
 * Algorithm", the per-token and block-wise equations; block table mapping
 * in "KV Cache Manager: Block Table Mapping"; [Int] "PagedAttention: page
 * tables, for KV", address translation).  K and V are gathered straight
 * through the table with no compaction pass ([Os]).  Query heads sharing a
 * kv head form contiguous groups ([Res] "Attention over scattered blocks").
 * Slots at t >= n and table entries at index >= ceil(n / B) are never read.
 * n == 0 gives a zero row.  Arithmetic is fp32 with the result rounded to
 * the dtype (round to nearest even).
 *
 * q, k_cache, v_cache, block_tables, context_lens, out: device pointers.
 * workspace: device pointer (16-byte aligned) to at least
 * pa_decode_workspace_size() bytes when that size is non-zero (may be NULL
 * otherwise); its contents on entry do not matter and are left unspecified.
 * With a split, each partition stores its unnormalised partial there and a
 * second kernel on the same stream (the merge) combines them by the
 * log-sum-exp identity.  Calls that share a workspace must not overlap
 * (order them on one stream).
 * Device-side conditions: 0 <= context_lens[s] <= max_context_len and
 * 0 <= block_tables[s][j] < num_blocks for j < ceil(n / B).  A longer
 * context is clamped to max_context_len (and to MBS * B); a table entry
 * outside [0, NB) is clamped into it.
 * Results are bitwise deterministic for fixed inputs and launch
 * configuration, and independent of where the blocks sit in the pool.
 */
int pa_decode(const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, float scale,
              void *out, const pa_decode_params *p, void *workspace, size_t ws_bytes,
              void *stream);

/*
 * pa_decode without a workspace argument, for callers that cannot allocate
 * device memory or pass a buffer they own: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid allocation.  The split-K
 * partials go to a fixed array of PA_NO_ALLOC_SCRATCH_BYTES (16 MiB) that
 * the library holds in device memory, one per device, from the library's
 * load until the process ends.  The call allocates and frees nothing; its
 * first call with a split on a device looks up that device's array address
 * (hipGetSymbolAddress) and caches it.
 *
 * Same parameters, checks, preconditions and results as pa_decode (the same
 * kernels, with the array as their workspace: bitwise the same output).
 * Returns PA_ERR_SCRATCH, before any HIP call, when
 * pa_decode_workspace_size(p) exceeds PA_NO_ALLOC_SCRATCH_BYTES (e.g. 64
 * sequences x 40 query heads x 12 partitions x 130 x 4 bytes = 16 MB fits;
 * 13 partitions do not).
 *
 * Every call on a device shares that device's array, and the array keeps
 * the last call's partials; nothing in it needs to start at zero.  Calls
 * whose work overlaps on one device (different streams, or other host
 * threads) race on the array and give unspecified results: order them on
 * one stream, or use pa_decode with a workspace of each caller's own.
 */
#define PA_NO_ALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int pa_decode_no_alloc(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       void *out, const pa_decode_params *p, void *stream);

/*
 * Bytes of workspace pa_decode_shared needs for ``p``: the split-K partials
 * as in pa_decode_workspace_size (rounded up to 16 bytes), then
 * 4 * num_seqs bytes (rounded up to 16) for each sequence's count of
 * partitions the grouped pass computed.  Same checks as
 * pa_decode_workspace_size; writes the size to *bytes (0 on error).
 */
int pa_decode_shared_workspace_size(const pa_decode_params *p, size_t *bytes);

/*
 * pa_decode for batches whose sequences share leading blocks: parallel
 * samples of one prompt, beam candidates with common ancestors, requests
 * with a common system prefix ([Kwon] "Memory Sharing for Complex Decoding
 * Algorithms": parallel sampling, beam search, shared prefix; [Res] "Sharing
 * blocks: parallel sampling and copy-on-write").  In the pages the attention
 * kernel sees only physical block ids and knows nothing of sharing ([Kwon]
 * "Logical-to-physical separation"), so a shared block is read once per
 * sequence.  Here the caller, who made the sharing (fork), passes the
 * groups, and every block in a group's shared prefix is read once per group.
 *
 * Groups: group i is sequences group_start[i] .. group_start[i+1] - 1, and
 * they name the same physical blocks in their first group_shared[i] table
 * entries (group_start [num_groups + 1] and group_shared [num_groups],
 * int32 device arrays, 4-byte aligned).  The groups must cover the batch in
 * order: group_start[0] == 0, non-decreasing, group_start[num_groups] ==
 * num_seqs (single-sequence groups are fine).  max_shared_blocks (host) is
 * at least every group_shared[i] and at most max_blocks_per_seq; it sizes
 * the first launch's grid.
 *
 * Work: with split-K partitions of p->partition_size tokens (required > 0),
 * the partitions that lie wholly inside a group's shared prefix are computed
 * once per (group, kv head) by a first launch, the group's query heads
 * (members x query heads per kv head, at most 16) as the score columns of
 * one matrix-core tile, each column masked at its own member's context
 * length; it also records, per sequence, how many leading partitions it
 * computed (in the workspace).  A second launch computes every sequence's
 * other partitions as pa_decode does, and the merge combines them.  A group
 * of one sequence, or with more than 16 query heads in all, or whose shared
 * prefix holds no whole partition, is computed as pa_decode would.
 *
 * The result equals pa_decode's within floating-point rounding (the shared
 * partitions are summed in a different order), and is bitwise deterministic
 * for fixed inputs, groups and launch configuration.  Every other parameter,
 * precondition and clamp is pa_decode's; the table entries group members
 * share are read from the group's first sequence.
 *
 * workspace: device pointer (16-byte aligned) to at least
 * pa_decode_shared_workspace_size(p) bytes; contents on entry do not matter.
 * Returns PA_ERR_UNSUPPORTED for fp32; PA_ERR_SHAPE for partition_size 0,
 * num_groups < 0 or > num_seqs, or max_shared_blocks outside [0,
 * max_blocks_per_seq]; PA_ERR_NULL / PA_ERR_ALIGN for the group arrays when
 * num_groups > 0; otherwise as pa_decode.  num_groups == 0 computes plain
 * pa_decode (split-K).  Calls that share a workspace must not overlap.
 */
int pa_decode_shared(const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, const int32_t *context_lens,
                     const int32_t *group_start, const int32_t *group_shared, int32_t num_groups,
                     int32_t max_shared_blocks, float scale, void *out,
                     const pa_decode_params *p, void *workspace, size_t ws_bytes, void *stream);

/*
 * decode_append: the decode iteration's write and attention in one launch.
 * For every sequence s with n = context_lens[s] >= 1 the newest token's rows
 * k_new[s], v_new[s] ([num_seqs, num_kv_heads, head_dim], the token at
 * position n - 1) are written to that position's slot -- block
 * block_tables[s][(n - 1) / B], offset (n - 1) % B, what pa_cache_write
 * does with that slot ([Kwon] §3.4 "Kernel-Level Optimizations", item 1) --
 * and out is what pa_decode computes over the n tokens afterwards.  The
 * attention takes position n - 1 from k_new / v_new, so no workgroup waits
 * for the write.  Pool contents are bit for bit those of pa_cache_write
 * followed by pa_decode; out is too on the matrix-core path (grouped query
 * heads, 16-bit types), while the other path adds position n - 1 as a last
 * online-softmax step and may differ from pa_decode in rounding order only
 * (deterministic, within pa_decode's tolerance).  Same parameters, layouts, checks,
 * workspace and preconditions as pa_decode; k_new, v_new: device pointers,
 * 16-byte aligned.  The newest slot must belong to sequence s alone (a
 * shared last block is copied first: pa_copy_blocks).
 */
int pa_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache,
                     void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                     float scale, void *out, const pa_decode_params *p, void *workspace,
                     size_t ws_bytes, void *stream);

/*
 * The same attention over a contiguous cache: token t of sequence s is row
 * (s, t) of k, v ([Res] "Attention over scattered blocks": the contiguous
 * cache addressed directly, no table).  Built from the same kernel source as
 * pa_decode with only the address function changed, so on identical bytes
 * the two return bitwise-identical outputs for equal partition_size and
 * max_context_len (whatever the paged block_size).  block_size, max_blocks_per_seq and
 * num_blocks in ``p`` are ignored; max_seq_len (>= 1) is the position
 * stride of k and v and clamps every context length.
 */
int pa_decode_dense(const void *q, const void *k, const void *v,
                    const int32_t *context_lens, float scale, void *out,
                    const pa_decode_params *p, int32_t max_seq_len,
                    void *workspace, size_t ws_bytes, void *stream);

/*
 * cache_write: for every new token i < num_tokens with slot = slot_mapping[i]
 * in [0, NB * B), copies its K row and V row ([Hkv, D] each, byte for byte)
 * into block slot / B, offset slot % B of k_cache / v_cache ([Kwon] §3.4
 * "Kernel-Level Optimizations", item 1, the fused reshape and block write:
 * one launch, the scheduler names block and slot; [Res] "A paged KV cache,
 * in code": the slot mapping).  Negative slots are padding and are skipped;
 * slots >= NB * B are skipped too.  Slots must be distinct within one call
 * (two tokens for one slot race).  In the head-major layout each kv head's
 * row lands in its own (block, head) plane.
 * k_new, v_new, slot_mapping, k_cache, v_cache: device pointers.
 * num_tokens == 0 enqueues nothing.
 */
int pa_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                   const int32_t *slot_mapping, int32_t num_tokens,
                   const pa_cache_params *p, void *stream);

/*
 * copy_blocks: for every pair (src, dst) of block_pairs, copies the whole K
 * block and the whole V block ([B, Hkv, D] each, byte for byte) from src to
 * dst, all pairs in one launch ([Kwon] §3.4 "Kernel-Level Optimizations",
 * item 3, the fused block copy taking (source, destination) pairs; "Memory
 * Sharing ...": copy-on-write copies the entire block).  Destinations must
 * be distinct and none may also be a source within one call; pairs with an
 * id outside [0, NB) are skipped.
 * k_cache, v_cache, block_pairs: device pointers.  num_pairs == 0 enqueues
 * nothing.
 */
int pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *block_pairs,
                   int32_t num_pairs, const pa_cache_params *p, void *stream);

/*
 * copy_blocks for every layer of a model at once: one block id names the
 * same position in every layer's pool ([Res] "A paged KV cache, in code"),
 * so one list of pairs serves all layers, and the copies of all layers run
 * in one launch per 64 layers ([Kwon] §3.4 "Kernel-Level Optimizations",
 * item 3: block copies fused across layers).  Same rules as pa_copy_blocks
 * per layer.
 * k_caches, v_caches: HOST arrays of num_layers device pointers, one pool
 * per layer, all with the geometry ``p``; read during the call only.
 * block_pairs: device pointer.  PA_ERR_UNSUPPORTED if num_pairs * min(
 * num_layers, 64) * 512 reaches 2^32 (split the call).
 */
int pa_copy_blocks_layers(void *const *k_caches, void *const *v_caches, int32_t num_layers,
                          const int32_t *block_pairs, int32_t num_pairs,
                          const pa_cache_params *p, void *stream);

/*
 * cache_write for every layer of a model at once: layer l's new rows
 * k_new[l], v_new[l] ([num_tokens, Hkv, D] each) go to the slots of
 * slot_mapping in layer l's pools k_caches[l], v_caches[l].  One slot
 * mapping serves all layers, because a block id names the same position in
 * every layer's pool ([Res] "A paged KV cache, in code"); the writes of all
 * layers run in one launch per 64 layers (the fused write of [Kwon] §3.4
 * "Kernel-Level Optimizations", item 1, across layers, as item 3 fuses the
 * copies).  Same rules per layer as pa_cache_write.
 * k_new, v_new, k_caches, v_caches: HOST arrays of num_layers device
 * pointers, read during the call only; all pools have the geometry ``p``.
 * slot_mapping: device pointer.  num_tokens == 0 enqueues nothing.
 */
int pa_cache_write_layers(const void *const *k_new, const void *const *v_new,
                          void *const *k_caches, void *const *v_caches, int32_t num_layers,
                          const int32_t *slot_mapping, int32_t num_tokens,
                          const pa_cache_params *p, void *stream);

/*
 * swap_blocks: moves whole blocks between two pools of the same block
 * geometry, for every layer, in one launch per 64 layers: for each pair
 * (src, dst), layer l: dst_k[l][dst] = src_k[l][src], dst_v[l][dst] =
 * src_v[l][src] ([Kwon] §3.4 "Scheduling and Preemption": swapping copies
 * the evicted blocks to CPU memory and back; the pairs come from the block
 * manager's pa_bm_swap_out / pa_bm_swap_in).  Either pool may live in device
 * memory or in pinned host memory that the device can access (e.g.
 * hipHostMalloc); one kernel reads and writes both, so many small blocks do
 * not cost one DMA transfer each.  Pairs with src outside [0,
 * src_num_blocks) or dst outside [0, dst_num_blocks) are skipped.  The two
 * pools must not overlap; destinations must be distinct.
 * dst_k, dst_v, src_k, src_v: HOST arrays of num_layers pool pointers.
 * block_pairs: device-accessible.  p: block geometry (its num_blocks is not
 * used).
 */
int pa_swap_blocks(void *const *dst_k, void *const *dst_v, int32_t dst_num_blocks,
                   const void *const *src_k, const void *const *src_v, int32_t src_num_blocks,
                   int32_t num_layers, const int32_t *block_pairs, int32_t num_pairs,
                   const pa_cache_params *p, void *stream);

/*
 * prefill: attention for a chunk of new tokens per sequence over the paged
 * cache -- the prompt phase, and chunked prefill where a long prompt arrives
 * in pieces ([Kwon] §3.4 "PagedAttention Algorithm" and the prompt phase of
 * §2: each prompt token attends to itself and every earlier token; the keys
 * and values are read through the block table).  Sequence s owns the query
 * rows query_start[s] .. query_start[s+1] - 1 (T_s rows), which are the
 * LAST T_s of its context_lens[s] cached tokens: their keys and values must
 * already be in the pool (pa_cache_write).  Chunk row r sits at position
 * n_s - T_s + r and attends to positions 0 .. n_s - T_s + r, with the
 * decode softmax and scale.
 * Layouts: q, out [total_query_rows, Hq, D]; pools and tables as pa_decode;
 * query_start [num_seqs + 1] int32, query_start[0] = 0, non-decreasing,
 * query_start[num_seqs] = total_query_rows.  Device pointers.
 * Host-checked: dtype fp16 or bf16 (fp32: PA_ERR_UNSUPPORTED), head_dim 64
 * or 128 (else PA_ERR_UNSUPPORTED), num_seqs <= 65535 and max_query_len <=
 * 65535 * 128 (else PA_ERR_UNSUPPORTED), Hq a multiple of Hkv, block_size a
 * power of two in [1, 256],
 * max_context_len <= max_blocks_per_seq * block_size, 16-byte aligned q,
 * caches and out, 4-byte aligned int arrays.
 * Preconditions (device data, not checked): 0 <= T_s <= max_query_len,
 * T_s <= context_lens[s] <= max_context_len, table entries of the first
 * ceil(n / B) blocks in [0, NB).  Violations never cause an out-of-range
 * access (rows, lengths and ids are clamped); the rows concerned are then
 * unspecified.
 */
typedef struct {
    int32_t num_seqs;
    int32_t num_q_heads, num_kv_heads, head_dim;
    int32_t block_size, max_blocks_per_seq, num_blocks;
    int32_t total_query_rows;   /* rows of q and out */
    int32_t max_query_len;      /* bound on every chunk length; sizes the grid */
    int32_t max_context_len;    /* bound on every context length */
    int32_t dtype;              /* pa_dtype: PA_F16 or PA_BF16 */
    int32_t layout;             /* pa_kv_layout */
} pa_prefill_params;

int pa_prefill(const void *q, const void *k_cache, const void *v_cache,
               const int32_t *block_tables, const int32_t *context_lens,
               const int32_t *query_start, float scale, void *out,
               const pa_prefill_params *p, void *stream);

/* Static text for a pa_status value (never NULL). */
const char *pa_status_string(int status);

/* Static text naming the build: target, kernel variants, compiler. */
const char *pa_build_info(void);

/* Name of the HIP error (e.g. "hipErrorInvalidValue") behind the calling
 * thread's most recent PA_ERR_HIP, or "" if this thread has had none.  The
 * string is static; it stays valid for the life of the process. */
const char *pa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
