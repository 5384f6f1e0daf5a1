// Host-side KV block manager: reference-counted block pools, per-sequence
// block tables, fork / reserve (append with copy-on-write) / free, group
// swap between the GPU pool and a host pool.  It emits exactly the inputs of
// the device entry points: copy pairs (pa_copy_blocks), slot mapping
// (pa_cache_write), block tables and context lengths (pa_decode).
//
// Semantics follow [Kwon] section 3.4 ("KV Cache Manager", "Memory Sharing":
// fork, append, free, reference counts, copy-on-write; "Scheduling and
// Preemption": all-or-nothing groups, swapping), [Int] "Ref counts and
// copy-on-write" and [Res] "A paged KV cache, in code" (reserve before the
// forward pass; copy a shared partly-filled last block before writing).
// The C ABI and every rule it states are in include/pa_block_manager.h.
//
// Every entry point validates, then counts what it needs, and only then
// mutates: a failing call leaves the manager unchanged.  Per-call scratch
// (a per-block counter) is kept in the manager and restored to zero before
// the call returns, so no call allocates in proportion to the pool size.

#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "pa_block_manager.h"

namespace {

struct Pool {
    std::vector<int32_t> refs;   // table entries naming each block
    std::vector<int32_t> stack;  // free blocks; back() is handed out next
    std::vector<int32_t> mark;   // per-call scratch, all zero between calls

    void init(int32_t nb) {
        refs.assign((size_t)nb, 0);
        mark.assign((size_t)nb, 0);
        stack.clear();
        stack.reserve((size_t)nb);
    }
    int32_t size() const { return (int32_t)refs.size(); }
    int32_t take() {
        const int32_t b = stack.back();
        stack.pop_back();
        refs[(size_t)b] = 1;
        return b;
    }
    void drop(int32_t b, int32_t count) {
        refs[(size_t)b] -= count;
        if (refs[(size_t)b] == 0) stack.push_back(b);
    }
};

struct Seq {
    std::vector<int32_t> table;
    int64_t n = 0;
    bool live = false;
    bool on_cpu = false;
};

}  // namespace

struct pa_bm {
    int32_t block_size = 16;
    Pool gpu, cpu;
    std::vector<Seq> seqs;
    std::vector<int32_t> spare;    // handles free for reuse (stack)
    std::vector<uint32_t> listed;  // per-handle stamp for duplicate checks
    uint32_t stamp = 0;

    Pool &pool(bool on_cpu) { return on_cpu ? cpu : gpu; }

    int32_t new_handle() {
        int32_t h;
        if (!spare.empty()) {
            h = spare.back();
            spare.pop_back();
        } else {
            h = (int32_t)seqs.size();
            listed.reserve(seqs.size() + 1);  // both grow or neither
            seqs.emplace_back();
            listed.push_back(0);
        }
        Seq &s = seqs[(size_t)h];
        s.table.clear();
        s.n = 0;
        s.live = true;
        s.on_cpu = false;
        return h;
    }

    bool is_live(int32_t h) const {
        return h >= 0 && (size_t)h < seqs.size() && seqs[(size_t)h].live;
    }

    // side: 0 = GPU side only, 1 = swapped only, -1 = either.
    int check_group(const int32_t *ids, int32_t n, int side) {
        if (n < 0) return PA_ERR_SHAPE;
        if (n > 0 && !ids) return PA_ERR_NULL;
        if (++stamp == 0) {  // wrapped: clear the stamps once
            std::fill(listed.begin(), listed.end(), 0u);
            stamp = 1;
        }
        for (int32_t i = 0; i < n; ++i) {
            const int32_t h = ids[i];
            if (!is_live(h)) return PA_ERR_STATE;
            if (side >= 0 && seqs[(size_t)h].on_cpu != (side == 1)) return PA_ERR_STATE;
            if (listed[(size_t)h] == stamp) return PA_ERR_STATE;
            listed[(size_t)h] = stamp;
        }
        return PA_OK;
    }
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

bool pow2_in(int32_t x, int32_t lo, int32_t hi) {
    return x >= lo && x <= hi && (x & (x - 1)) == 0;
}

// Move a group's distinct blocks from pool `from` to pool `to`, emitting
// (from, to) pairs in first-appearance order.
int move_group(pa_bm *bm, const int32_t *ids, int32_t n, bool to_cpu, int32_t *pairs,
               int32_t cap, int32_t *n_pairs) {
    if (!n_pairs) return PA_ERR_NULL;
    if (cap < 0) return PA_ERR_SHAPE;
    int st = bm->check_group(ids, n, to_cpu ? 0 : 1);
    if (st != PA_OK) return st;
    Pool &from = bm->pool(!to_cpu);
    Pool &to = bm->pool(to_cpu);
    // Count the group's references per block; list distinct blocks in order.
    std::vector<int32_t> order;
    size_t entries = 0;
    for (int32_t i = 0; i < n; ++i) entries += bm->seqs[(size_t)ids[i]].table.size();
    order.reserve(entries);  // may throw; nothing is marked yet
    for (int32_t i = 0; i < n; ++i)
        for (int32_t b : bm->seqs[(size_t)ids[i]].table)
            if (from.mark[(size_t)b]++ == 0) order.push_back(b);
    const int64_t need = (int64_t)order.size();
    st = PA_OK;
    if (need > (int64_t)to.stack.size()) st = PA_ERR_NO_BLOCKS;
    else if (need > cap) st = PA_ERR_SHAPE;
    else if (need > 0 && !pairs) st = PA_ERR_NULL;
    if (st != PA_OK) {
        for (int32_t b : order) from.mark[(size_t)b] = 0;
        return st;
    }
    // mark[b] becomes the destination id + 1 after its references move.
    for (size_t k = 0; k < order.size(); ++k) {
        const int32_t b = order[k];
        const int32_t cnt = from.mark[(size_t)b];
        const int32_t d = to.take();
        to.refs[(size_t)d] = cnt;
        from.drop(b, cnt);
        pairs[2 * k] = b;
        pairs[2 * k + 1] = d;
        from.mark[(size_t)b] = d + 1;
    }
    for (int32_t i = 0; i < n; ++i) {
        Seq &s = bm->seqs[(size_t)ids[i]];
        for (int32_t &b : s.table) b = from.mark[(size_t)b] - 1;
        s.on_cpu = to_cpu;
    }
    for (int32_t b : order) from.mark[(size_t)b] = 0;
    *n_pairs = (int32_t)need;
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_bm_create(int32_t num_gpu_blocks, int32_t num_cpu_blocks, int32_t block_size,
                 const int32_t *gpu_free_order, pa_bm **out) {
    if (!out) return PA_ERR_NULL;
    if (num_gpu_blocks < 1 || num_cpu_blocks < 0 || !pow2_in(block_size, 1, 256))
        return PA_ERR_SHAPE;
    pa_bm *bm = new (std::nothrow) pa_bm;
    if (!bm) return PA_ERR_NO_BLOCKS;
    try {
        bm->block_size = block_size;
        bm->gpu.init(num_gpu_blocks);
        bm->cpu.init(num_cpu_blocks);
        if (gpu_free_order) {
            std::vector<uint8_t> seen((size_t)num_gpu_blocks, 0);
            for (int32_t i = 0; i < num_gpu_blocks; ++i) {
                const int32_t b = gpu_free_order[i];
                if (b < 0 || b >= num_gpu_blocks || seen[(size_t)b]) {
                    delete bm;
                    return PA_ERR_SHAPE;
                }
                seen[(size_t)b] = 1;
            }
            for (int32_t i = num_gpu_blocks - 1; i >= 0; --i) bm->gpu.stack.push_back(gpu_free_order[i]);
        } else {
            for (int32_t b = num_gpu_blocks - 1; b >= 0; --b) bm->gpu.stack.push_back(b);
        }
        for (int32_t b = num_cpu_blocks - 1; b >= 0; --b) bm->cpu.stack.push_back(b);
    } catch (...) {
        delete bm;
        return PA_ERR_NO_BLOCKS;
    }
    *out = bm;
    return PA_OK;
}

void pa_bm_destroy(pa_bm *bm) { delete bm; }

int pa_bm_new_seq(pa_bm *bm, int32_t *seq) {
    if (!bm || !seq) return PA_ERR_NULL;
    try {
        *seq = bm->new_handle();
    } catch (...) {
        return PA_ERR_NO_BLOCKS;
    }
    return PA_OK;
}

int pa_bm_fork(pa_bm *bm, int32_t parent, int32_t *child) {
    if (!bm || !child) return PA_ERR_NULL;
    if (!bm->is_live(parent) || bm->seqs[(size_t)parent].on_cpu) return PA_ERR_STATE;
    int32_t h;
    try {
        std::vector<int32_t> table = bm->seqs[(size_t)parent].table;
        h = bm->new_handle();  // may grow seqs: index again below
        Seq &c = bm->seqs[(size_t)h];
        c.table.swap(table);
        c.n = bm->seqs[(size_t)parent].n;
    } catch (...) {
        return PA_ERR_NO_BLOCKS;
    }
    for (int32_t b : bm->seqs[(size_t)h].table) bm->gpu.refs[(size_t)b] += 1;
    *child = h;
    return PA_OK;
}

int pa_bm_free(pa_bm *bm, const int32_t *seqs, int32_t n) {
    if (!bm) return PA_ERR_NULL;
    int st = bm->check_group(seqs, n, -1);
    if (st != PA_OK) return st;
    try {
        bm->spare.reserve(bm->spare.size() + (size_t)n);
    } catch (...) {
        return PA_ERR_NO_BLOCKS;
    }
    for (int32_t i = 0; i < n; ++i) {
        Seq &s = bm->seqs[(size_t)seqs[i]];
        Pool &p = bm->pool(s.on_cpu);
        for (int32_t b : s.table) p.drop(b, 1);
        s.table.clear();
        s.n = 0;
        s.live = false;
        bm->spare.push_back(seqs[i]);
    }
    return PA_OK;
}

int pa_bm_reserve(pa_bm *bm, const int32_t *seqs, const int32_t *num_new, int32_t n,
                  int32_t *slot_mapping, int64_t slot_cap, int32_t *block_pairs,
                  int32_t pair_cap, int32_t *n_pairs) {
    if (!bm || !n_pairs) return PA_ERR_NULL;
    if (n > 0 && !num_new) return PA_ERR_NULL;
    if (slot_cap < 0 || pair_cap < 0) return PA_ERR_SHAPE;
    int st = bm->check_group(seqs, n, 0);
    if (st != PA_OK) return st;
    const int32_t bs = bm->block_size;
    Pool &g = bm->gpu;
    // Count: slots, copy-on-write copies (a shared last block loses one
    // reference per copy, so the last sharer to write finds count 1 and
    // writes in place), and new blocks.
    int64_t slots = 0, copies = 0, fresh = 0;
    std::vector<int32_t> touched;
    try {
        touched.reserve((size_t)n);
    } catch (...) {
        return PA_ERR_NO_BLOCKS;
    }
    for (int32_t i = 0; i < n && st == PA_OK; ++i) {
        const int32_t k = num_new[i];
        if (k < 0) { st = PA_ERR_SHAPE; break; }
        if (k == 0) continue;
        const Seq &s = bm->seqs[(size_t)seqs[i]];
        if (s.n + k > INT32_MAX) { st = PA_ERR_SHAPE; break; }
        slots += k;
        if (s.n % bs) {
            const int32_t b = s.table.back();
            if (g.refs[(size_t)b] - g.mark[(size_t)b] > 1) {
                ++copies;
                if (g.mark[(size_t)b]++ == 0) touched.push_back(b);
            }
        }
        fresh += blocks_for(s.n + k, bs) - (int64_t)s.table.size();
    }
    for (int32_t b : touched) g.mark[(size_t)b] = 0;
    if (st != PA_OK) return st;
    if (slots > slot_cap || copies > pair_cap) return PA_ERR_SHAPE;
    if ((slots > 0 && !slot_mapping) || (copies > 0 && !block_pairs)) return PA_ERR_NULL;
    if (copies + fresh > (int64_t)g.stack.size()) return PA_ERR_NO_BLOCKS;
    try {  // the tables may grow; reserve first so that nothing throws midway
        for (int32_t i = 0; i < n; ++i) {
            Seq &s = bm->seqs[(size_t)seqs[i]];
            s.table.reserve((size_t)blocks_for(s.n + num_new[i], bs));
        }
    } catch (...) {
        return PA_ERR_NO_BLOCKS;
    }
    int64_t w = 0;
    int32_t np = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t k = num_new[i];
        if (k == 0) continue;
        Seq &s = bm->seqs[(size_t)seqs[i]];
        if (s.n % bs) {
            const int32_t old = s.table.back();
            if (g.refs[(size_t)old] > 1) {
                const int32_t nb = g.take();
                g.drop(old, 1);
                s.table.back() = nb;
                block_pairs[2 * np] = old;
                block_pairs[2 * np + 1] = nb;
                ++np;
            }
        }
        while ((int64_t)s.table.size() * bs < s.n + k) s.table.push_back(g.take());
        for (int64_t t = s.n; t < s.n + k; ++t)
            slot_mapping[w++] = s.table[(size_t)(t / bs)] * bs + (int32_t)(t % bs);
        s.n += k;
    }
    *n_pairs = np;
    return PA_OK;
}

int pa_bm_tables(const pa_bm *bm, const int32_t *seqs, int32_t n, int32_t *block_tables,
                 int32_t max_blocks_per_seq, int32_t *context_lens) {
    if (!bm) return PA_ERR_NULL;
    if (n < 0 || max_blocks_per_seq < 1) return PA_ERR_SHAPE;
    if (n > 0 && (!seqs || !block_tables || !context_lens)) return PA_ERR_NULL;
    for (int32_t i = 0; i < n; ++i) {
        if (!bm->is_live(seqs[i]) || bm->seqs[(size_t)seqs[i]].on_cpu) return PA_ERR_STATE;
        if (bm->seqs[(size_t)seqs[i]].table.size() > (size_t)max_blocks_per_seq)
            return PA_ERR_SHAPE;
    }
    for (int32_t i = 0; i < n; ++i) {
        const Seq &s = bm->seqs[(size_t)seqs[i]];
        int32_t *row = block_tables + (int64_t)i * max_blocks_per_seq;
        const size_t m = s.table.size();
        std::copy(s.table.begin(), s.table.end(), row);
        std::fill(row + m, row + max_blocks_per_seq, -1);
        context_lens[i] = (int32_t)s.n;
    }
    return PA_OK;
}

int pa_bm_swap_out(pa_bm *bm, const int32_t *seqs, int32_t n, int32_t *pairs, int32_t cap,
                   int32_t *n_pairs) {
    if (!bm) return PA_ERR_NULL;
    try {
        return move_group(bm, seqs, n, true, pairs, cap, n_pairs);
    } catch (...) {
        return PA_ERR_NO_BLOCKS;
    }
}

int pa_bm_swap_in(pa_bm *bm, const int32_t *seqs, int32_t n, int32_t *pairs, int32_t cap,
                  int32_t *n_pairs) {
    if (!bm) return PA_ERR_NULL;
    try {
        return move_group(bm, seqs, n, false, pairs, cap, n_pairs);
    } catch (...) {
        return PA_ERR_NO_BLOCKS;
    }
}

int pa_bm_num_free(const pa_bm *bm, int32_t *gpu_free, int32_t *cpu_free) {
    if (!bm || !gpu_free || !cpu_free) return PA_ERR_NULL;
    *gpu_free = (int32_t)bm->gpu.stack.size();
    *cpu_free = (int32_t)bm->cpu.stack.size();
    return PA_OK;
}

int pa_bm_ref_count(const pa_bm *bm, int32_t block, int32_t on_cpu, int32_t *refs) {
    if (!bm || !refs) return PA_ERR_NULL;
    const Pool &p = on_cpu ? bm->cpu : bm->gpu;
    if (block < 0 || block >= p.size() || (on_cpu != 0 && on_cpu != 1)) return PA_ERR_SHAPE;
    *refs = p.refs[(size_t)block];
    return PA_OK;
}

int pa_bm_seq_info(const pa_bm *bm, int32_t seq, int32_t *num_tokens, int32_t *num_blocks,
                   int32_t *where) {
    if (!bm || !num_tokens || !num_blocks || !where) return PA_ERR_NULL;
    if (!bm->is_live(seq)) return PA_ERR_STATE;
    const Seq &s = bm->seqs[(size_t)seq];
    *num_tokens = (int32_t)s.n;
    *num_blocks = (int32_t)s.table.size();
    *where = s.on_cpu ? PA_SEQ_SWAPPED : PA_SEQ_ON_GPU;
    return PA_OK;
}

int pa_bm_block_table(const pa_bm *bm, int32_t seq, int32_t *table, int32_t cap) {
    if (!bm) return PA_ERR_NULL;
    if (!bm->is_live(seq)) return PA_ERR_STATE;
    const Seq &s = bm->seqs[(size_t)seq];
    if (cap < 0 || (size_t)cap < s.table.size()) return PA_ERR_SHAPE;
    if (!s.table.empty() && !table) return PA_ERR_NULL;
    std::copy(s.table.begin(), s.table.end(), table);
    return PA_OK;
}

int pa_bm_free_list(const pa_bm *bm, int32_t on_cpu, int32_t *ids, int32_t cap, int32_t *n) {
    if (!bm || !n) return PA_ERR_NULL;
    if (on_cpu != 0 && on_cpu != 1) return PA_ERR_SHAPE;
    const Pool &p = on_cpu ? bm->cpu : bm->gpu;
    const size_t m = p.stack.size();
    if (cap < 0 || (size_t)cap < m) return PA_ERR_SHAPE;
    if (m > 0 && !ids) return PA_ERR_NULL;
    for (size_t i = 0; i < m; ++i) ids[i] = p.stack[m - 1 - i];
    *n = (int32_t)m;
    return PA_OK;
}

}  // extern "C"
