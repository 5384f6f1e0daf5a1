/*
 * pa_block_manager.h -- host-side KV block manager (C ABI).
 *
 * The bookkeeping that runs on the CPU before each forward pass and produces
 * the inputs of the device entry points in pa.h: the copy-on-write pairs for
 * pa_copy_blocks, the slot mapping for pa_cache_write, and the block tables
 * and context lengths for pa_decode.
 *
 * Pages cited (by title, then section / figure):
 *   [Kwon] "Efficient Memory Management for Large Language Model Serving
 *          with PagedAttention" (paper summary page)
 *   [Int]  "vLLM Internals: PagedAttention, Continuous Batching, and Where
 *          the 2-4x Comes From"
 *   [Res]  "Paged Attention: Managing the KV Cache Like Virtual Memory"
 *
 * Model ([Kwon] section 3.4 "KV Cache Manager" and "Memory Sharing": the
 * fork / append / free primitives, reference counts and copy-on-write;
 * [Int] "PagedAttention: page tables, for KV" and "Ref counts and
 * copy-on-write"; [Res] "A paged KV cache, in code" and "Sharing blocks"):
 *   - A pool of num_gpu_blocks physical blocks of block_size token slots,
 *     each with a reference count (the number of block-table entries that
 *     name it).  A block with count 0 is on the free list.  A second pool of
 *     num_cpu_blocks host blocks receives swapped-out blocks ([Kwon] section
 *     3.4 "Scheduling and Preemption": swapping, the CPU block allocator).
 *   - A sequence holds a block table (physical ids, logical order) and its
 *     token count n; every slot t < n holds a stored token, slot
 *     t lives in block table[t / block_size] at offset t % block_size, and
 *     the table has exactly ceil(n / block_size) entries.
 *   - Free list order: a stack.  A new manager hands out the ids of
 *     gpu_free_order in the order given (ascending ids when it is NULL); a
 *     released block is pushed on top and is the next one handed out.
 *
 * Conventions
 * -----------
 *  - All memory is host memory.  The manager owns its state; the caller
 *    owns every array passed in or out.  No call touches the GPU.
 *  - One manager must not be used by two threads at once.
 *  - Every call returns a pa_status (pa.h).  A call that fails changes
 *    nothing: checks, including the count of blocks the call needs, run
 *    before any state is modified (all-or-nothing).
 *      PA_ERR_NULL       a required pointer is NULL
 *      PA_ERR_SHAPE      a size is out of range, or an output array is too
 *                        small for what the call would write
 *      PA_ERR_NO_BLOCKS  the pool cannot supply the blocks the call needs
 *      PA_ERR_STATE      a sequence handle is not live, is listed twice, or
 *                        is in the wrong pool for the call
 *  - Sequence handles are small non-negative integers.  A new sequence
 *    (pa_bm_new_seq, pa_bm_fork) takes the most recently freed handle, or
 *    else the next unused integer counting from 0.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_bm pa_bm; /* opaque */

/* Where a live sequence's blocks are. */
typedef enum { PA_SEQ_ON_GPU = 0, PA_SEQ_SWAPPED = 1 } pa_seq_where;

/* Create a manager.  block_size: a power of two in [1, 256];
 * num_gpu_blocks >= 1; num_cpu_blocks >= 0 (0: no swapping).
 * gpu_free_order: NULL, or a permutation of 0 .. num_gpu_blocks - 1 giving
 * the order in which a new pool hands out its blocks (PA_ERR_SHAPE if it is
 * not a permutation).  *out receives the handle. */
int pa_bm_create(int32_t num_gpu_blocks, int32_t num_cpu_blocks, int32_t block_size,
                 const int32_t *gpu_free_order, pa_bm **out);

/* Release the manager and everything it holds.  NULL is accepted. */
void pa_bm_destroy(pa_bm *bm);

/* A new empty sequence (n = 0, no blocks) on the GPU side. */
int pa_bm_new_seq(pa_bm *bm, int32_t *seq);

/* fork ([Kwon] section 3.4, the three primitive operations; [Res] "A paged
 * KV cache, in code"): a child with a copy of the parent's block table and
 * token count; every block of the parent gains one reference.  Nothing is
 * copied.  The parent must be on the GPU side. */
int pa_bm_fork(pa_bm *bm, int32_t parent, int32_t *child);

/* free, for a sequence group ([Kwon] section 3.4, free; "Scheduling and
 * Preemption": all-or-nothing, gang-scheduled groups): every listed sequence
 * drops one reference per table entry, in list order then table order;
 * blocks that reach zero are pushed on the free stack in that order.  The
 * handles become invalid.  Sequences may be on either side. */
int pa_bm_free(pa_bm *bm, const int32_t *seqs, int32_t n);

/* Reserve slots for num_new[i] new tokens of each listed sequence, for one
 * forward pass ([Kwon] section 3.4 append and copy-on-write; [Int] "Ref
 * counts and copy-on-write"; [Res] "A paged KV cache, in code", reserve).
 * Sequences are handled in list order; for each one with num_new > 0:
 *   1. if its last block is partly filled (n % block_size != 0) and shared
 *      (count > 1), a new block is taken from the pool, the pair
 *      (old, new) is appended to block_pairs, the old block loses one
 *      reference and the table's last entry becomes the new block;
 *   2. new blocks are appended until the table covers n + num_new tokens;
 *   3. the slots block * block_size + offset of tokens n .. n + num_new - 1
 *      are appended to slot_mapping, and n grows by num_new.
 * Outputs: slot_mapping[sum(num_new)] (capacity slot_cap), block_pairs
 * [*n_pairs][2] as (src, dst) (capacity pair_cap pairs).  The pairs must be
 * applied (pa_copy_blocks) before the slots are written (pa_cache_write).
 * Every listed sequence must be live, on the GPU side and listed once;
 * num_new[i] >= 0.  PA_ERR_NO_BLOCKS if the copies plus the new blocks of
 * the whole batch exceed the free GPU blocks. */
int pa_bm_reserve(pa_bm *bm, const int32_t *seqs, const int32_t *num_new, int32_t n,
                  int32_t *slot_mapping, int64_t slot_cap, int32_t *block_pairs,
                  int32_t pair_cap, int32_t *n_pairs);

/* The decode batch view of the listed GPU-side sequences, as pa_decode reads
 * it: block_tables [n, max_blocks_per_seq] (row i = sequence seqs[i]'s
 * table, unused entries -1) and context_lens [n] (= each n).  PA_ERR_SHAPE
 * if a table is longer than max_blocks_per_seq.  Sequences may repeat. */
int pa_bm_tables(const pa_bm *bm, const int32_t *seqs, int32_t n, int32_t *block_tables,
                 int32_t max_blocks_per_seq, int32_t *context_lens);

/* Swap a group out to the host pool ([Kwon] section 3.4 "Scheduling and
 * Preemption": swapping, all-or-nothing per group).  Every distinct GPU
 * block named by the group's tables (first-appearance order: list order,
 * then table order) gets one host block; the pair (gpu, cpu) is appended to
 * pairs (capacity cap pairs).  The group's references move to the host
 * block; a GPU block with no reference left returns to the GPU free stack
 * (blocks still named by a sequence outside the group stay).  The group's
 * tables then name host blocks.  GPU blocks left with no reference are
 * pushed on the GPU free stack in the pairs' order.  The pairs' data must be
 * copied before any later call hands those GPU blocks out again.
 * PA_ERR_NO_BLOCKS if the host pool is too small.  Every listed sequence
 * must be live, on the GPU side, listed once. */
int pa_bm_swap_out(pa_bm *bm, const int32_t *seqs, int32_t n, int32_t *pairs, int32_t cap,
                   int32_t *n_pairs);

/* The reverse of pa_bm_swap_out: pairs are (cpu, gpu); the group's tables
 * then name GPU blocks.  PA_ERR_NO_BLOCKS if the GPU pool is too small.
 * Every listed sequence must be live, swapped, listed once. */
int pa_bm_swap_in(pa_bm *bm, const int32_t *seqs, int32_t n, int32_t *pairs, int32_t cap,
                  int32_t *n_pairs);

/* Introspection (for tests and schedulers). */
int pa_bm_num_free(const pa_bm *bm, int32_t *gpu_free, int32_t *cpu_free);
/* Reference count of a block of the GPU pool (on_cpu = 0) or host pool (1). */
int pa_bm_ref_count(const pa_bm *bm, int32_t block, int32_t on_cpu, int32_t *refs);
/* Token count, table length and side (pa_seq_where) of a live sequence. */
int pa_bm_seq_info(const pa_bm *bm, int32_t seq, int32_t *num_tokens, int32_t *num_blocks,
                   int32_t *where);
/* A live sequence's table (cap entries available; PA_ERR_SHAPE if short). */
int pa_bm_block_table(const pa_bm *bm, int32_t seq, int32_t *table, int32_t cap);
/* The free stack of one pool, next-to-be-handed-out first (cap entries
 * available; *n receives the stack depth; PA_ERR_SHAPE if cap is short). */
int pa_bm_free_list(const pa_bm *bm, int32_t on_cpu, int32_t *ids, int32_t cap, int32_t *n);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
