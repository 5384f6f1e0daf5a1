// pa_kernels.hip -- gfx950 (CDNA4) kernels for paged decode attention (and
// its split-K merge), prefill over the paged cache, cache_write and block
// copies.
//
// Pages cited (by title, then section / equation / figure):
//   [Kwon] "Efficient Memory Management for Large Language Model Serving with
//          PagedAttention" (paper summary page)
//   [Int]  "vLLM Internals: PagedAttention, Continuous Batching, and Where the
//          2-4x Comes From"
//   [Res]  "Paged Attention: Managing the KV Cache Like Virtual Memory"
//
// Decode design (one workgroup of 4 or 8 wave64 per (sequence, kv head,
// partition); the launcher picks the wave count from the kernel's occupancy,
// see pick_waves):
//  * A token row of one kv head is D * e bytes (256 B for fp16/bf16 D=128
//    and fp32 D=64).  LPR = D*e/16 lanes read it with one 16-byte load each,
//    so one wave load instruction covers R = 64/LPR whole rows and every
//    byte fetched is used.  A wave step is 16 consecutive tokens (U = 16/R
//    loads of K and U of V); the waves take steps round robin and
//    issue their next step's loads before computing the current one.  K and
//    V are streamed once, so they are read with non-temporal loads.
//  * Two pool layouts are addressed through strides: token-major blocks
//    [NB, B, Hkv, D] and head-major blocks [NB, Hkv, B, D] ([Res] "A paged
//    KV cache, in code" keeps [blocks, kv heads, 16 tokens, head dim]).  In
//    the head-major layout a 16-token step of one head is 4 KiB contiguous.
//  * The sequence's block-table slice is staged in LDS (up to 1024 entries
//    at a time), so address translation ([Int] "PagedAttention: page
//    tables, for KV") costs an LDS read per step, not a dependent HBM read.
//  * q.k: per-lane partial dot (v_dot2_f32_f16 / v_dot2_f32_bf16 on the
//    unscaled inputs, fp32 FMA for fp32), then a DPP butterfly inside each
//    LPR-lane row group; every lane of the group ends with the same bits.
//    The G query heads sharing the kv head ([Res] "Attention over scattered
//    blocks") are all served from the same K/V registers.
//  * Softmax: each row group keeps its own running (max, sum, acc) in the
//    base-2 domain (scale * log2 e folded into the score), updated once per
//    step; the R row groups of a wave are merged with lane exchanges and the
//    waves through LDS at the end.  This is the one-pass form of the
//    [Kwon] §3.4 two-pass softmax; both equal the defining equation in exact
//    arithmetic.  The reduction order depends only on logical token order,
//    never on where blocks sit, so paged and dense results are bitwise equal
//    and invariant to block placement.
//  * Scheduling: for unsplit launches of up to 256 sequences with more than
//    512 (sequence, kv head) items (more than the chip holds at once), every
//    workgroup ranks the sequences by context length (longest first, ties
//    by index) and takes the sequence whose rank matches its grid position,
//    so the longest sequences start first and the tail of the launch is
//    short.  Which workgroup computes a row never changes its arithmetic.
//  * Split-K: partition p covers tokens [p*PS, (p+1)*PS) and writes its
//    unnormalised partial (acc, m, l) to the workspace; a merge kernel then
//    combines the partitions by the log-sum-exp identity ([Int] "The kernel
//    pays for the indirection": a grid dimension over partitions; [Res]:
//    slices and a merge kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pa_launch.h"

namespace pa {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef uint32_t vec4 __attribute__((ext_vector_type(4)));  // 16 bytes

constexpr int kThreads = 256;       // cache_write / copy_blocks workgroups
constexpr int kMaxWaves = 8;        // decode workgroups have 4 or 8 waves (chosen per launch)
constexpr int kStepTokens = 16;     // tokens per wave step
constexpr int kTableChunk = 1024;   // block-table entries staged in LDS at once
constexpr int kRankMaxSeqs = 256;   // longest-first scheduling up to this batch
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -3.402823466e38f;  // running-max start (finite)

// ---------------------------------------------------------------- lane helpers

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR lanes of a row group (LPR in {8, 16, 32}); every lane of
// the group receives the same bits (each step adds two equal-valued operands
// in swapped order, and fp addition is commutative).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm(1,0,3,2): lane ^ 1
    x += dpp<0x4E>(x);   // quad_perm(2,3,0,1): lane ^ 2
    x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8
    if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror: the other 8 of the 16
    if constexpr (LPR >= 32)
        x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // lane ^ 16
    return x;
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Largest of three finite-or-infinite scores in one instruction (the
// library's maxnum would first quiet each input, which scores never need:
// they are products of finite values or -inf from a mask).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ vec4 load_stream(const char *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const vec4 *>(p));
}

__device__ __forceinline__ vec4 load_cached(const char *p) {
    return *reinterpret_cast<const vec4 *>(p);
}

// ---------------------------------------------------------------- element traits

template <typename T>
struct Elem;

template <>
struct Elem<float> {
    static constexpr int kEPL = 4;  // elements per 16 bytes
    __device__ static float dot(const vec4 &a, const vec4 &b) {
        float s = __uint_as_float(a.x) * __uint_as_float(b.x);
        s = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), s);
        s = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), s);
        s = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), s);
        return s;
    }
    __device__ static void widen(const vec4 &v, float *f) {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
    __device__ static void store(void *out, int64_t i, float x) { ((float *)out)[i] = x; }
};

// Reinterpret one 32-bit lane value as two 16-bit elements.  The value is
// taken by copy: bit-casting an ext_vector element in place (v.y, v.z, ...)
// reads element 0 with this compiler.
__device__ __forceinline__ half2_t as_half2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ __forceinline__ bf162_t as_bf162(uint32_t w) { return __builtin_bit_cast(bf162_t, w); }

template <>
struct Elem<_Float16> {
    static constexpr int kEPL = 8;
    __device__ static float dot(const vec4 &a, const vec4 &b) {
        // fp16 x fp16 products are exact in fp32; the sum accumulates in fp32.
        float s = __builtin_amdgcn_fdot2(as_half2(a.x), as_half2(b.x), 0.0f, false);
        s = __builtin_amdgcn_fdot2(as_half2(a.y), as_half2(b.y), s, false);
        s = __builtin_amdgcn_fdot2(as_half2(a.z), as_half2(b.z), s, false);
        s = __builtin_amdgcn_fdot2(as_half2(a.w), as_half2(b.w), s, false);
        return s;
    }
    __device__ static void widen1(uint32_t w, float *f) {
        const half2_t h = as_half2(w);
        f[0] = (float)h.x;
        f[1] = (float)h.y;
    }
    __device__ static void widen(const vec4 &v, float *f) {
        widen1(v.x, f);
        widen1(v.y, f + 2);
        widen1(v.z, f + 4);
        widen1(v.w, f + 6);
    }
    __device__ static void store(void *out, int64_t i, float x) { ((_Float16 *)out)[i] = (_Float16)x; }
};

template <>
struct Elem<__bf16> {
    static constexpr int kEPL = 8;
    __device__ static float dot(const vec4 &a, const vec4 &b) {
        // bf16 x bf16 products are exact in fp32; the sum accumulates in fp32.
        float s = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(a.x), as_bf162(b.x), 0.0f, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(a.y), as_bf162(b.y), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(a.z), as_bf162(b.z), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(a.w), as_bf162(b.w), s, false);
        return s;
    }
    __device__ static void widen1(uint32_t w, float *f) {
        f[0] = __uint_as_float(w << 16);          // bf16 is the top half of an fp32
        f[1] = __uint_as_float(w & 0xFFFF0000u);
    }
    __device__ static void widen(const vec4 &v, float *f) {
        widen1(v.x, f);
        widen1(v.y, f + 2);
        widen1(v.z, f + 4);
        widen1(v.w, f + 6);
    }
    __device__ static void store(void *out, int64_t i, float x) { ((__bf16 *)out)[i] = (__bf16)x; }
};

// ---------------------------------------------------------------- decode

struct DecodeArgs {
    const char *q;
    const char *k;
    const char *v;
    const int32_t *tables;
    const int32_t *lens;
    void *out;
    float *ws_acc;   // [S, Hq, P, D]
    float *ws_ml;    // [S, Hq, P, 2]
    float qk_scale;  // scale * log2(e)
    // Append mode (k_new != nullptr): the newest token of each sequence,
    // rows [S, Hkv, D], is read from here for position n - 1 and written to
    // its slot through k_w / v_w (the same pools as k / v).
    const char *k_new;
    const char *v_new;
    char *k_w;
    char *v_w;
    int32_t S, Hq, Hkv, NB, MBS, log2B, max_ctx, PS, P;
    // Shared prefixes: skip[s] leading partitions of sequence s are computed
    // by the grouped launch (null: none).  The grouped launch itself reads
    // groups [group_start[i], group_start[i+1]) sharing group_shared[i]
    // leading table entries, Gh query heads per kv head, Pg partitions per
    // group in its grid, and writes skip[] for every member.
    const int32_t *skip;
    const int32_t *group_start;
    const int32_t *group_shared;
    int32_t *skip_out;
    int32_t Gh, Pg;
    int32_t hg;         // kv heads per workgroup (VALU kernel: 1 or 2)
    int32_t ips;        // workgroup items per sequence (Hkv / hg)
    int32_t rank;       // 1: longest-first sequence order (S <= kRankMaxSeqs)
    int32_t spec_blocks;  // table entries a partition can need (fetched before its length)
    int64_t tok_bytes;  // bytes between consecutive tokens of one head
    int64_t head_bytes; // bytes between kv heads at a fixed token
    int64_t blk_bytes;  // paged: bytes per block
    int64_t seq_bytes;  // dense: bytes per sequence
};

// Address modes of the decode kernel.
enum : int {
    kDense = 0,      // contiguous cache, one base per sequence
    kPagedWide = 1,  // paged, B >= 16: every 16-token step lies inside one block
    kPagedNarrow = 2 // paged, B < 16: a step spans several blocks
};

__device__ __forceinline__ int clamp_len(int x, int max_ctx) {
    return x < 0 ? 0 : (x > max_ctx ? max_ctx : x);
}

// Longest-first order: rank(t) = #{u : n_u > n_t} + #{u < t : n_u == n_t}.
// Stages every clamped length in s_len and returns the sequence of rank
// `want` (a permutation, so exactly one thread finds it).
__device__ int rank_pick(const DecodeArgs &a, int32_t *s_len, int32_t *s_pick, int want, int tid,
                         int nt_) {
    for (int t = tid; t < a.S; t += nt_) s_len[t] = clamp_len(a.lens[t], a.max_ctx);
    __syncthreads();
    // The rank of sequence t (how many are longer, or as long with a lower
    // index) is counted by k consecutive lanes, each over a contiguous
    // k-th of the lengths, and summed by lane exchanges (k <= 8, k * S <=
    // threads, so the k lanes of t share a wave and every t has its lanes).
    int k = 1;
    while (k < 8 && 2 * k * a.S <= nt_) k *= 2;
    const int t = tid / k, j = tid % k;
    if (t < a.S) {
        const int nt = s_len[t];
        // Each lane's part starts at a multiple of 4 and is read four
        // lengths per 16-byte LDS read, several reads in flight (one read
        // per length, each waited for, cost ~100 cycles a length); entries
        // past the part are masked out by index.
        const int per = ((a.S + k - 1) / k + 3) & ~3;
        const int u0 = j * per, u1 = min(a.S, u0 + per);
        const int4 *l4 = reinterpret_cast<const int4 *>(s_len);
        auto longer = [&](int nu, int u) {
            return (int)((u < u1) & ((nu > nt) | ((nu == nt) & (u < t))));
        };
        int r = 0;
#pragma unroll 4
        for (int u = u0; u < u1; u += 4) {
            const int4 L = l4[u >> 2];
            r += longer(L.x, u) + longer(L.y, u + 1) + longer(L.z, u + 2) + longer(L.w, u + 3);
        }
        for (int off = 1; off < k; off <<= 1) r += __shfl_xor(r, off, 64);
        if (j == 0 && r == want) *s_pick = t;
    }
    __syncthreads();
    return *s_pick;
}

// Block-table entries [b0, b0 + cnt) of one row into LDS, clamped into [0, NB).
__device__ void stage_table(const int32_t *trow, int b0, int cnt, int NB, int32_t *s_tab, int tid,
                            int nt_) {
    for (int i = tid; i < cnt; i += nt_) {
        const int32_t b = trow[b0 + i];
        s_tab[i] = b < 0 ? 0 : (b >= NB ? NB - 1 : b);
    }
}

// Append mode: the workgroup whose token range ends at n writes the newest
// token's K and V rows of its kv head into the slot of position n - 1 ([Kwon]
// §3.4 "Kernel-Level Optimizations", item 1: the new token's keys and values
// go to the block and slot the table names).  Its own attention reads that
// token from k_new / v_new, so nothing waits for the write.
template <typename T, int D>
__device__ void append_write(const DecodeArgs &a, const int32_t *trow, int s, int h, int n,
                             int64_t head0, int tid) {
    constexpr int VPR = D * (int)sizeof(T) / 16;  // 16-byte pieces of a row
    if (tid >= VPR) return;
    const int last = n - 1;
    int32_t b = trow[last >> a.log2B];
    b = b < 0 ? 0 : (b >= a.NB ? a.NB - 1 : b);
    const int64_t dst = head0 + (int64_t)b * a.blk_bytes +
                        (int64_t)(last & ((1 << a.log2B) - 1)) * a.tok_bytes + tid * 16;
    const int64_t src = ((int64_t)s * a.Hkv + h) * D * (int64_t)sizeof(T) + tid * 16;
    *reinterpret_cast<vec4 *>(a.k_w + dst) = load_cached(a.k_new + src);
    *reinterpret_cast<vec4 *>(a.v_w + dst) = load_cached(a.v_new + src);
}

// The VALU kernel's form of the same write: the caller already holds its
// 16-byte pieces of the rows (piece_off = the piece's byte offset in a row).
__device__ __forceinline__ void append_store(const DecodeArgs &a, const int32_t *trow, int n,
                                             int64_t head0, uint32_t piece_off, vec4 kn,
                                             vec4 vn) {
    const int last = n - 1;
    int32_t b = trow[last >> a.log2B];
    b = b < 0 ? 0 : (b >= a.NB ? a.NB - 1 : b);
    const int64_t dst = head0 + (int64_t)b * a.blk_bytes +
                        (int64_t)(last & ((1 << a.log2B) - 1)) * a.tok_bytes + piece_off;
    *reinterpret_cast<vec4 *>(a.k_w + dst) = kn;
    *reinterpret_cast<vec4 *>(a.v_w + dst) = vn;
}

// Position of a workgroup in the one-dimensional decode grid: item = (sequence
// slot, kv head) pair, part = its context partition.  The partitions of one
// item take consecutive workgroup ids, and the dispatcher deals consecutive
// ids to the eight XCDs in turn, so every item's partitions are spread over
// all XCDs (with the partition as the slow index, each item's whole context
// landed on one XCD and the XCDs' loads differed up to 2x on mixed lengths).
__device__ __forceinline__ void grid_pos(const DecodeArgs &a, int &item, int &part) {
    const int wg = (int)blockIdx.x;
    part = a.P > 1 ? wg % a.P : 0;
    item = a.P > 1 ? wg / a.P : wg;
}

// Which sequence a workgroup serves.  Without ranking, the first table chunk
// does not depend on the context length, so it is fetched together with the
// length instead of after it (*staged = true; a barrier publishes it).
template <int MODE>
__device__ void pick_work(const DecodeArgs &a, int32_t *s_len, int32_t *s_pick, int32_t *s_tab,
                          int item, int part, int tid, int nt_, int &s, int &n, bool &staged) {
    const int want = item / a.ips;
    staged = false;
    if (a.rank) {
        s = rank_pick(a, s_len, s_pick, want, tid, nt_);
        n = s_len[s];
        return;
    }
    s = want;
    if constexpr (MODE != kDense) {
        const int b0 = (a.PS ? part * a.PS : 0) >> a.log2B;
        const int cnt = min(min(kTableChunk, a.spec_blocks), a.MBS - b0);
        stage_table(a.tables + (int64_t)s * a.MBS, b0, cnt, a.NB, s_tab, tid, nt_);
        staged = true;
    }
    n = clamp_len(a.lens[s], a.max_ctx);
}

// End of a decode workgroup: combine the waves' running states (red[w][g] =
// acc[0..D), m, l) and store either the output row (a single partition
// covers the sequence) or the partition's unnormalised partial, which the
// merge kernel combines.  hg kv heads per workgroup, nw waves each (head k's
// waves are k nw .. k nw + nw - 1; its query rows follow head k - 1's).
template <typename T, int D, int G>
__device__ void finish_workgroup(const DecodeArgs &a, const float *red, int nw, int hg,
                                 int64_t qrow0, int part, int n, int tid, int nthr) {
    const bool direct = a.PS == 0 || n <= a.PS;
    for (int i = tid; i < hg * G * D; i += nthr) {
        const int k = i / (G * D), ri = i - k * (G * D);
        const int g = ri / D, d = ri % D;
        const float *rk = red + k * nw * G * (D + 2);
        float M = kNegBig;
        for (int w = 0; w < nw; ++w) M = fmaxf(M, rk[(w * G + g) * (D + 2) + D]);
        float L = 0.0f, A = 0.0f;
        for (int w = 0; w < nw; ++w) {
            const float *r = rk + (w * G + g) * (D + 2);
            const float cw = fexp2(r[D] - M);
            L = fmaf(r[D + 1], cw, L);
            A = fmaf(r[d], cw, A);
        }
        const int64_t qh = qrow0 + k * G + g;
        if (direct) {
            Elem<T>::store(a.out, qh * D + d, A / L);
        } else {
            const int64_t pi = qh * a.P + part;
            a.ws_acc[pi * D + d] = A;
            if (d == 0) {
                a.ws_ml[pi * 2] = M;
                a.ws_ml[pi * 2 + 1] = L;
            }
        }
    }
}

// End of a grouped (shared-prefix) workgroup: red[w][c] for score column c =
// member c / Gh, head c % Gh; lim[c] is that member's length.  A member whose
// context ends inside the first partition gets its output row, others the
// partition's partial; partitions past a member's end are not its own.
template <typename T, int D>
__device__ void finish_group(const DecodeArgs &a, const float *red, int nw, int ncol, int s0,
                             int h, int part, int cols, const int32_t *lim, int tid, int nthr) {
    for (int i = tid; i < cols * D; i += nthr) {
        const int c = i / D, d = i % D;
        const int np = (lim[c] + a.PS - 1) / a.PS;
        if (part >= np) continue;
        float M = kNegBig;
        for (int w = 0; w < nw; ++w) M = fmaxf(M, red[(w * ncol + c) * (D + 2) + D]);
        float L = 0.0f, A = 0.0f;
        for (int w = 0; w < nw; ++w) {
            const float *r = red + (w * ncol + c) * (D + 2);
            const float cw = fexp2(r[D] - M);
            L = fmaf(r[D + 1], cw, L);
            A = fmaf(r[d], cw, A);
        }
        const int64_t qh = (int64_t)(s0 + c / a.Gh) * a.Hq + (int64_t)h * a.Gh + c % a.Gh;
        if (np <= 1) {
            Elem<T>::store(a.out, qh * D + d, A / L);
        } else {
            const int64_t pi = qh * a.P + part;
            a.ws_acc[pi * D + d] = A;
            if (d == 0) {
                a.ws_ml[pi * 2] = M;
                a.ws_ml[pi * 2 + 1] = L;
            }
        }
    }
}

// fp32 rows need twice the registers per token, so fp32 workgroups keep 4 waves.
template <typename T>
constexpr int max_waves() { return sizeof(T) == 4 ? 4 : kMaxWaves; }

template <typename T, int D, int G, int MODE>
__global__ __launch_bounds__(max_waves<T>() * 64) void decode_kernel(DecodeArgs a) {
    using E = Elem<T>;
    constexpr int EPL = E::kEPL;
    constexpr int LPR = D / EPL;               // lanes per token row
    constexpr int R = 64 / LPR;                // rows per wave load
    constexpr int U = kStepTokens / R;         // loads per step (K and V each)
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row must be 128, 256 or 512 bytes");
    static_assert(U * R == kStepTokens, "step shape");

    // Dynamic LDS (sized by the launcher): the block-table chunk during the
    // loop, then the cross-wave merge buffer [waves][G][D + 2].
    extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
    float *smem = reinterpret_cast<float *>(dyn_smem);
    __shared__ __attribute__((aligned(16))) int32_t s_len[kRankMaxSeqs];
    __shared__ int32_t s_pick;
    int32_t *s_tab = reinterpret_cast<int32_t *>(smem);

    const int nthr = blockDim.x;   // 64 * waves
    const int nw = nthr >> 6;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int rg = lane / LPR;   // row group
    const int c = lane % LPR;    // 16-byte chunk of the row
    // With hg = 2 a workgroup serves two adjacent kv heads of one sequence,
    // nw / 2 waves each: on a token-major pool their rows of a token are
    // adjacent, so the two halves read 512 contiguous bytes per token.
    const int hg = a.hg;
    const int nwh = nw >> (hg - 1);       // waves per kv head (2, 4 or 8)
    const int lwh = 31 - __builtin_clz(nwh);
    const int sub = wave >> lwh;          // this wave's kv head within the workgroup
    const int wh = wave & (nwh - 1);      // its index among that head's waves
    int item, part;
    grid_pos(a, item, part);
    const int h = (item % a.ips) * hg + sub;
    // Leading partitions of a shared prefix are the grouped launch's (its
    // count is requested first, so a workgroup with nothing to do leaves
    // after one round trip; no ranking with a shared prefix, so the
    // sequence is item / Hkv).
    const int skip_s = a.skip ? a.skip[item / a.ips] : 0;

    int s, n;
    bool staged;
    pick_work<MODE>(a, s_len, &s_pick, s_tab, item, part, tid, nthr, s, n, staged);
    if (part < skip_s) return;
    const int tb = a.PS ? part * a.PS : 0;
    const int te = a.PS ? min(n, tb + a.PS) : n;
    const int64_t qrow0 = (int64_t)s * a.Hq + (int64_t)h * G;  // first query head of the group
    const int64_t qrow_wg = qrow0 - (int64_t)sub * G;          // the workgroup's first query head

    // q for the G heads of the group: this lane's 16-byte chunk, unscaled
    // (issued before the length test so it overlaps the other first loads).
    vec4 qv[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        qv[g] = load_cached(a.q + ((qrow0 + g) * D + (int64_t)c * EPL) * sizeof(T));
    // Append mode: the workgroup whose range ends at n takes position n - 1
    // from k_new / v_new after the loop (the head's first wave), so the loop stops before it;
    // its 16-byte pieces are requested here, with q.
    const bool app = MODE != kDense && a.k_new != nullptr && te == n;
    const uint32_t chunk_off = (uint32_t)(c * EPL * (int)sizeof(T));
    vec4 kn = {}, vn = {};
    if (app && wh == 0 && tb < te) {
        const int64_t nsrc = ((int64_t)s * a.Hkv + h) * D * (int64_t)sizeof(T) + chunk_off;
        kn = load_cached(a.k_new + nsrc);
        vn = load_cached(a.v_new + nsrc);
    }

    if (tb >= te) {
        // Only an empty sequence reaches here with part == 0: its row is zero.
        if (part == 0)
            for (int i = tid; i < hg * G * D; i += nthr) E::store(a.out, qrow_wg * D + i, 0.0f);
        return;
    }

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegBig;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
    }

    // Per-lane byte offset of its 16-byte chunk of token u*R + rg of a step.
    const uint32_t tok_bytes = (uint32_t)a.tok_bytes;
    uint32_t voff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) voff[u] = (uint32_t)(u * R + rg) * tok_bytes + chunk_off;
    const int B = 1 << a.log2B;
    const int32_t *trow = MODE == kDense ? nullptr : a.tables + (int64_t)s * a.MBS;
    // Base of kv head h (and, dense, of sequence s).
    const int64_t head0 = (int64_t)h * a.head_bytes + (MODE == kDense ? (int64_t)s * a.seq_bytes : 0);
    const char *kh = a.k + head0;
    const char *vh = a.v + head0;

    const int le = app ? te - 1 : te;
    const int nblk = (le - tb + B - 1) >> a.log2B;
    const int chunk_blocks = MODE == kDense ? nblk : kTableChunk;

    for (int cb = 0; cb < nblk; cb += chunk_blocks) {
        const int cn = min(chunk_blocks, nblk - cb);
        const int ctb = tb + cb * B;                 // first token of this chunk
        const int cte = min(le, ctb + cn * B);       // one past its last token
        if constexpr (MODE != kDense) {
            __syncthreads();  // the previous chunk's readers are done / the first chunk is out
            if (!(cb == 0 && staged)) {
                stage_table(trow, (tb >> a.log2B) + cb, cn, a.NB, s_tab, tid, nthr);
                __syncthreads();
            }
        }
        const int nfull = (cte - ctb) / kStepTokens;      // steps with 16 valid tokens
        const int tail = (cte - ctb) % kStepTokens;        // valid tokens of the last step

        // Issue the K and V loads of step j (tokens ctb + 16 j ...).  With
        // MASKED, rows past the end re-read the last valid token.
        auto issue = [&]<bool MASKED>(vec4 (&kb)[U], vec4 (&vb)[U], int j) {
            const int t0 = ctb + j * kStepTokens;
            if constexpr (MODE == kPagedNarrow) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    int t = t0 + u * R + rg;
                    if (MASKED) t = t < cte ? t : cte - 1;
                    const int64_t off = (int64_t)s_tab[(t - ctb) >> a.log2B] * a.blk_bytes +
                                        (int64_t)(t & (B - 1)) * a.tok_bytes + chunk_off;
                    kb[u] = load_stream(kh + off);
                    vb[u] = load_stream(vh + off);
                }
            } else {
                int64_t base;
                if constexpr (MODE == kDense) {
                    base = (int64_t)t0 * a.tok_bytes;
                } else {
                    const int phys = __builtin_amdgcn_readfirstlane(s_tab[(t0 - ctb) >> a.log2B]);
                    base = (int64_t)phys * a.blk_bytes + (int64_t)(t0 & (B - 1)) * a.tok_bytes;
                }
                const char *kp = kh + base;
                const char *vp = vh + base;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    uint32_t o = voff[u];
                    if (MASKED) {
                        const int r = min(u * R + rg, cte - 1 - t0);
                        o = (uint32_t)r * tok_bytes + chunk_off;
                    }
                    kb[u] = load_stream(kp + o);
                    vb[u] = load_stream(vp + o);
                }
            }
        };
        // Online-softmax update with the 16 tokens of step j.
        auto compute = [&]<bool MASKED>(const vec4 (&kb)[U], const vec4 (&vb)[U], int j) {
            float sc[U][G];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool valid = !MASKED || ctb + j * kStepTokens + u * R + rg < cte;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float x = group_sum<LPR>(E::dot(qv[g], kb[u])) * a.qk_scale;
                    sc[u][g] = valid ? x : -__builtin_inff();
                }
            }
            float vf[U][EPL];
#pragma unroll
            for (int u = 0; u < U; ++u) E::widen(vb[u], vf[u]);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float mx = sc[0][g];
#pragma unroll
                for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][g]);
                const float mn = fmaxf(m[g], mx);
                const float alpha = fexp2(m[g] - mn);
                float lsum = l[g] * alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float p = fexp2(sc[u][g] - mn);
                    lsum += p;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, vf[u][e], acc[g][e]);
                }
                l[g] = lsum;
                m[g] = mn;
            }
        };

        // Steps: the wave with index wh among its head's nwh waves takes
        // steps wh, wh + nwh, ... of the nst steps, the partly filled last
        // one (index nfull, if any) included.  The next
        // step's loads are always issued before the current step is
        // computed, so exactly one step of loads is outstanding while a step
        // is computed, the partly filled one too.  Only the last step of a
        // wave can be that one: it is issued with MASKED where it can occur
        // (a wave-uniform test) and computed with MASKED at the two places a
        // wave's last step is computed.
        const int nst = nfull + (tail ? 1 : 0);
        auto issue_any = [&](vec4 (&kb)[U], vec4 (&vb)[U], int jj) {
            if (jj < nfull)
                issue.template operator()<false>(kb, vb, jj);
            else
                issue.template operator()<true>(kb, vb, jj);
        };
        auto compute_last = [&](const vec4 (&kb)[U], const vec4 (&vb)[U], int jj) {
            if (jj < nfull)
                compute.template operator()<false>(kb, vb, jj);
            else
                compute.template operator()<true>(kb, vb, jj);
        };
        vec4 ka[U], va[U], kb2[U], vb2[U];
        int j = wh;
        if (j < nst) {
            issue_any(ka, va, j);
            while (j + 2 * nwh < nst) {
                issue.template operator()<false>(kb2, vb2, j + nwh);   // j + nwh < nst - nwh <= nfull
                __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
                compute.template operator()<false>(ka, va, j);
                issue_any(ka, va, j + 2 * nwh);
                __builtin_amdgcn_sched_barrier(0);
                compute.template operator()<false>(kb2, vb2, j + nwh);
                j += 2 * nwh;
            }
            if (j + nwh < nst) {
                issue_any(kb2, vb2, j + nwh);
                __builtin_amdgcn_sched_barrier(0);
                compute.template operator()<false>(ka, va, j);      // j < j + nwh <= nfull
                compute_last(kb2, vb2, j + nwh);
            } else {
                compute_last(ka, va, j);
            }
        }
    }

    // Merge the R row groups of the wave (lanes rg*LPR + c, same c).
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mo = __shfl_xor(m[g], off, 64);
            const float lo = __shfl_xor(l[g], off, 64);
            const float mn = fmaxf(m[g], mo);
            const float c1 = fexp2(m[g] - mn), c2 = fexp2(mo - mn);
            l[g] = l[g] * c1 + lo * c2;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float ao = __shfl_xor(acc[g][e], off, 64);
                acc[g][e] = acc[g][e] * c1 + ao * c2;
            }
            m[g] = mn;
        }
    }

    if (app && wh == 0) {
        // Every row group of the head's first wave now holds the wave's merged state: add
        // position n - 1 as one more online-softmax step, and store its rows
        // in their slot (lanes 0 .. LPR - 1 hold the whole row).
        float vf[EPL];
        E::widen(vn, vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float x = group_sum<LPR>(E::dot(qv[g], kn)) * a.qk_scale;
            const float mn = fmaxf(m[g], x);
            const float alpha = fexp2(m[g] - mn);
            const float pn = fexp2(x - mn);
            l[g] = l[g] * alpha + pn;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pn, vf[e], acc[g][e] * alpha);
            m[g] = mn;
        }
        if (lane < LPR) append_store(a, trow, n, head0, chunk_off, kn, vn);
    }

    // Merge the waves through LDS: red[w][g][0..D) = acc, [D] = m, [D+1] = l.
    __syncthreads();  // s_tab is dead; reuse its LDS
    float *red = smem;
    if (lane < LPR) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float *r = red + (wave * G + g) * (D + 2);
#pragma unroll
            for (int e = 0; e < EPL; ++e) r[c * EPL + e] = acc[g][e];
            if (lane == 0) {
                r[D] = m[g];
                r[D + 1] = l[g];
            }
        }
    }
    __syncthreads();
    finish_workgroup<T, D, G>(a, red, nwh, hg, qrow_wg, part, n, tid, nthr);
}

// ---------------------------------------------------------------- grouped-query decode on MFMA

// For 16-bit K/V with G >= 2 query heads per kv head the scores of a 16-token
// step form a [16 tokens x G heads] tile, so both products run on the matrix
// cores (the VALU form spends ~700 instructions per step at G = 6):
//   S^T = K Q^T   v_mfma_f32_16x16x32: A = K (row = token, 8 dims per lane),
//                 B = Q^T (column = head, heads >= G are zero);
//   O^T += V^T P^T  v_mfma_f32_16x16x16: B = P^T is the S^T result in place
//                 (lane l holds tokens 4*(l/16)..+3 of head l%16), A = V^T
//                 from the transposing LDS read ds_read_b64_tr_b16.
// K and V are loaded as whole rows per instruction (the decode kernel's
// pattern: every 128-byte line a load instruction touches is used whole by
// it) and pass through a per-wave LDS tile of unpadded, swizzled rows, from
// which both operands are read.  Loading the A operand of K straight from
// the pool instead (16 rows x 64 bytes per instruction, each line split over
// two instructions) streamed ~12% slower.
// Lane layouts (A[l%16][k-block l/16], B[k-block l/16][l%16],
// C[4*(l/16)+j][l%16]) were checked against a host product on gfx950.
// The per-head running max is shared by the 16 tokens of a step (two lane
// exchanges), so P can feed one product; it moves lazily (kLazy below).  The
// weights enter the product in the input type: fp16 once (11-bit
// significand), bf16 as a high part plus the bf16 rounding of the remainder,
// two products that together carry ~16 significant bits (one bf16 rounding
// alone, 2^-9 per weight, can exceed the output tolerance for short
// sequences).  The running sum uses the fp32 weights.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef short short4_t2 __attribute__((ext_vector_type(4)));
// Lazy running max of the matrix-core kernels: the max of a score column
// moves only when a score exceeds it by more than 2^kLazy, so weights stay
// <= 2^kLazy (exact in fp16 / bf16), the final division by the running sum
// is unchanged in exact arithmetic, and the accumulator rescale is rare.
constexpr float kLazy = 8.0f;
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t vec2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Mma;

template <>
struct Mma<_Float16> {
    static constexpr bool kSplit = false;
    __device__ static float4_t qk(vec4 a, vec4 b, float4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    }
    __device__ static float4_t pv(vec2 a, vec2 b, float4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a),
                                                     __builtin_bit_cast(half4_t, b), c, 0, 0, 0);
    }
    __device__ static vec4 ones() { return vec4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u}; }
    __device__ static float4_t pv32(vec4 a, vec4 b, float4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    }
    __device__ static vec2 pack(float x0, float x1, float x2, float x3) {
        half4_t h = {(_Float16)x0, (_Float16)x1, (_Float16)x2, (_Float16)x3};
        return __builtin_bit_cast(vec2, h);
    }
    __device__ static vec2 rest(float, float, float, float, vec2) { return vec2{0u, 0u}; }
};

template <>
struct Mma<__bf16> {
    static constexpr bool kSplit = true;
    __device__ static float4_t qk(vec4 a, vec4 b, float4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a),
                                                       __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
    }
    __device__ static float4_t pv(vec2 a, vec2 b, float4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                         __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
    }
    __device__ static vec4 ones() { return vec4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}; }
    __device__ static float4_t pv32(vec4 a, vec4 b, float4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a),
                                                       __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
    }
    __device__ static vec2 pack(float x0, float x1, float x2, float x3) {
        typedef __bf16 bf164_t __attribute__((ext_vector_type(4)));
        bf164_t h = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
        return __builtin_bit_cast(vec2, h);
    }
    // bf16 of x - hi for each weight, hi the packed high parts
    __device__ static vec2 rest(float x0, float x1, float x2, float x3, vec2 hi) {
        const float h0 = __uint_as_float(hi.x << 16), h1 = __uint_as_float(hi.x & 0xFFFF0000u);
        const float h2 = __uint_as_float(hi.y << 16), h3 = __uint_as_float(hi.y & 0xFFFF0000u);
        return pack(x0 - h0, x1 - h1, x2 - h2, x3 - h3);
    }
};

// Position of 16-byte piece p of a K / V row r in an LDS tile of unpadded
// rows: p ^ row_swz(r).  The swizzle spreads the pieces that one read phase
// of the matrix-core kernels touches over distinct banks: 16 rows at one
// piece (a K operand read) and 8 rows x 2 adjacent pieces (the transposing
// V read).  Head dim 128 (16 pieces per row) or 64 (8).
template <int D>
__device__ __forceinline__ int row_swz(int r) {
    if constexpr (D == 128) return 2 * (r & 7) + ((r >> 3) & 1);
    else return 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
}

template <typename T, int D, int G, int MODE, bool GROUPED = false>
__global__ __launch_bounds__(kMaxWaves * 64) void decode_mma_kernel(DecodeArgs a) {
    using E = Elem<T>;
    using M = Mma<T>;
    static_assert(sizeof(T) == 2 && G >= 2 && G <= 16 && D % 32 == 0, "16-bit grouped-query tile");
    constexpr int KL = D / 32;            // 32-dim slices of the score product
    constexpr int DS = D / 16;            // 16-wide slices of the output rows
    constexpr int ROWB = D * 2;           // bytes of a K / V row
    constexpr int LPR = ROWB / 16;        // lanes per row in a load (16-byte pieces)
    constexpr int RPL = 64 / LPR;         // rows per load instruction
    constexpr int U = kStepTokens / RPL;  // loads per step, of K and of V
    constexpr int TILE = kStepTokens * ROWB;  // one step's K (or V) tile
    constexpr int TAB_BYTES = kTableChunk * 4;

    // Dynamic LDS (sized by the launcher): block-table chunk + one K and one
    // V tile per wave during the loop, then the cross-wave merge buffer.
    extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
    char *smem = dyn_smem;
    __shared__ __attribute__((aligned(16))) int32_t s_len[kRankMaxSeqs];
    __shared__ int32_t s_pick;
    int32_t *s_tab = reinterpret_cast<int32_t *>(smem);

    const int nthr = blockDim.x;   // 64 * waves
    const int nw = nthr >> 6;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tok = lane & 15;   // token of the step this lane loads; head of its score column
    const int kb = lane >> 4;    // k-block: 8 dims of each 32-dim slice; 4 tokens of the score tile
    int item, part;
    if constexpr (GROUPED) {  // grid (group, kv head) items x Pg partitions
        part = (int)blockIdx.x % a.Pg;
        item = (int)blockIdx.x / a.Pg;
    } else {
        grid_pos(a, item, part);
    }
    const int h = item % a.Hkv;
    char *ktile = smem + TAB_BYTES + wave * 2 * TILE;
    char *vtile = ktile + TILE;

    int s, n;
    bool staged;
    int64_t qrow_tok;    // q / out row of score column tok
    int cols = G;        // score columns in use
    int lim = INT32_MAX; // grouped: keys at or past it are hidden from column tok
    if constexpr (GROUPED) {
        // Shared prefix ([Kwon] "Memory Sharing for Complex Decoding
        // Algorithms"; [Res] "Sharing blocks: parallel sampling and
        // copy-on-write"): the members of a group name the same physical
        // blocks in their first shared table entries, so a partition inside
        // that prefix is read once, with the members' query heads as the
        // score columns (member tok / Gh, head tok % Gh), each column masked
        // at its own member's length.  The first member's table row
        // addresses the blocks.
        const int gi = item / a.Hkv;
        const int s0 = min(max(a.group_start[gi], 0), a.S);
        const int s1 = min(max(a.group_start[gi + 1], s0), a.S);
        const int members = s1 - s0;
        cols = members * a.Gh;
        const int shared = min(max(a.group_shared[gi], 0), a.MBS);
        // whole partitions inside the prefix, at most the grid's Pg
        const int sp = members >= 2 && cols <= G
                           ? (int)min((int64_t)shared * (1 << a.log2B) / a.PS, (int64_t)a.Pg)
                           : 0;
        // every member's count of partitions computed here, for the launch
        // that computes the rest (an empty member is left to it entirely)
        if (h == 0 && part == 0)
            for (int i = tid; i < members; i += nthr)
                a.skip_out[s0 + i] = clamp_len(a.lens[s0 + i], a.max_ctx) > 0 ? sp : 0;
        if (part >= sp) return;
        const int mi = tok / a.Gh;
        lim = tok < cols ? clamp_len(a.lens[s0 + mi], a.max_ctx) : 0;
        qrow_tok = (int64_t)(s0 + mi) * a.Hq + (int64_t)h * a.Gh + tok % a.Gh;
        int nmax = lim;  // the longest member bounds the keys read
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) nmax = max(nmax, __shfl_xor(nmax, off, 64));
        n = __builtin_amdgcn_readfirstlane(nmax);
        s = s0;
        // the partition's table entries, requested with the lengths (they
        // do not depend on them; the loop's first chunk uses them)
        if constexpr (MODE != kDense) {
            const int b0 = (part * a.PS) >> a.log2B;
            stage_table(a.tables + (int64_t)s0 * a.MBS, b0,
                        min(min(kTableChunk, a.spec_blocks), a.MBS - b0), a.NB, s_tab, tid, nthr);
        }
        staged = true;
        if (tid < 16) s_len[tid] = lim;  // for the epilogue
    } else {
        // (as in decode_kernel: the shared-prefix count first)
        const int skip_s = a.skip ? a.skip[item / a.Hkv] : 0;
        pick_work<MODE>(a, s_len, &s_pick, s_tab, item, part, tid, nthr, s, n, staged);
        if (part < skip_s) return;
        qrow_tok = (int64_t)s * a.Hq + (int64_t)h * G + tok;
    }
    const int tb = a.PS ? part * a.PS : 0;
    const int te = a.PS ? min(n, tb + a.PS) : n;
    const int64_t qrow0 = (int64_t)s * a.Hq + (int64_t)h * G;

    // B operand of S^T = K Q^T: column tok (zero for tok >= cols), dims 32 i + 8 kb ...
    vec4 qb[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i)
        qb[i] = tok < cols ? load_cached(a.q + (qrow_tok * D + 32 * i + 8 * kb) * 2)
                           : vec4{0u, 0u, 0u, 0u};

    if (tb >= te) {
        if (!GROUPED && part == 0)
            for (int i = tid; i < G * D; i += nthr) E::store(a.out, qrow0 * D + i, 0.0f);
        return;
    }

    float m = kNegBig, lsum = 0.0f;
    float4_t acc[DS];
#pragma unroll
    for (int d = 0; d < DS; ++d) acc[d] = float4_t{0.f, 0.f, 0.f, 0.f};

    // Loads: lane l moves piece l % LPR of rows l / LPR + RPL u (whole rows
    // per instruction, every fetched line used by it); the rows land in the
    // wave's tiles with their pieces swizzled.
    const int lrow = lane / LPR, lpiece = lane % LPR;
    uint32_t soff[U];  // LDS offset of this lane's piece of load u
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = lrow + RPL * u;
        soff[u] = (uint32_t)(r * ROWB + ((lpiece ^ row_swz<D>(r)) << 4));
    }
    // K operand: row tok, piece 4 i + kb; transposing V read: row lane / 4,
    // piece 2 d + (lane % 4) / 2, half lane % 2
    const int kswz = row_swz<D>(tok), vswz = row_swz<D>(lane >> 2);
    const uint32_t kbase = (uint32_t)(tok * ROWB), vbase = (uint32_t)((lane >> 2) * ROWB + 8 * (lane & 1));
    const int vpc = (lane & 3) >> 1;
    const int B = 1 << a.log2B;
    const int32_t *trow = MODE == kDense ? nullptr : a.tables + (int64_t)s * a.MBS;
    const int64_t head0 = (int64_t)h * a.head_bytes + (MODE == kDense ? (int64_t)s * a.seq_bytes : 0);
    const char *kh = a.k + head0;
    const char *vh = a.v + head0;

    const int nblk = (te - tb + B - 1) >> a.log2B;
    const int chunk_blocks = MODE == kDense ? nblk : kTableChunk;

    for (int cb = 0; cb < nblk; cb += chunk_blocks) {
        const int cn = min(chunk_blocks, nblk - cb);
        const int ctb = tb + cb * B;
        const int cte = min(te, ctb + cn * B);
        if constexpr (MODE != kDense) {
            __syncthreads();  // the previous chunk's readers are done / the first chunk is out
            if (!(cb == 0 && staged)) {
                stage_table(trow, (tb >> a.log2B) + cb, cn, a.NB, s_tab, tid, nthr);
                __syncthreads();
            }
        }
        const int nfull = (cte - ctb) / kStepTokens;
        const int tail = (cte - ctb) % kStepTokens;

        // K and V of step j: load u of lane l is piece lpiece of row lrow +
        // RPL u (rows clamped to the range when MASKED, so they re-read its
        // last token).
        auto issue = [&]<bool MASKED>(vec4 (&kb_)[U], vec4 (&vb_)[U], int j) {
            const int t0 = ctb + j * kStepTokens;
            int64_t base;   // first row of the step (paged wide / dense)
            if constexpr (MODE == kDense) {
                base = (int64_t)t0 * a.tok_bytes;
            } else if constexpr (MODE == kPagedWide) {
                const int phys = __builtin_amdgcn_readfirstlane(s_tab[(t0 - ctb) >> a.log2B]);
                base = (int64_t)phys * a.blk_bytes + (int64_t)(t0 & (B - 1)) * a.tok_bytes;
            } else {
                base = 0;
            }
            // Append mode, the step that holds position n - 1 (a wave-uniform
            // test): that row's lanes load from k_new / v_new instead.
            const bool app = MODE != kDense && a.k_new && (unsigned)(n - 1 - t0) < (unsigned)kStepTokens;
            const int64_t nsrc = ((int64_t)s * a.Hkv + h) * D * 2 + lpiece * 16;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int r = lrow + RPL * u;
                if (MASKED) r = min(r, cte - 1 - t0);
                int64_t row;
                if constexpr (MODE == kPagedNarrow) {
                    const int t = t0 + r;
                    row = (int64_t)s_tab[(t - ctb) >> a.log2B] * a.blk_bytes +
                          (int64_t)(t & (B - 1)) * a.tok_bytes;
                } else {
                    row = base + (int64_t)r * a.tok_bytes;
                }
                const char *kq = kh + row + lpiece * 16;
                const char *vq = vh + row + lpiece * 16;
                if (app && t0 + r == n - 1) {
                    kq = a.k_new + nsrc;
                    vq = a.v_new + nsrc;
                }
                kb_[u] = load_stream(kq);
                vb_[u] = load_stream(vq);
            }
        };
        auto compute = [&]<bool MASKED>(const vec4 (&kb_)[U], const vec4 (&vb_)[U], int j) {
            // the step's K and V rows into this wave's tiles; LDS operations
            // of a wave run in order, so the previous step's reads are done
            // and the reads below see these writes
#pragma unroll
            for (int u = 0; u < U; ++u) {
                *reinterpret_cast<vec4 *>(ktile + soff[u]) = kb_[u];
                *reinterpret_cast<vec4 *>(vtile + soff[u]) = vb_[u];
            }
            vec4 ka[KL];
#pragma unroll
            for (int i = 0; i < KL; ++i)
                ka[i] = *reinterpret_cast<const vec4 *>(ktile + kbase + (((4 * i + kb) ^ kswz) << 4));
            // S^T[token 4 kb + jj][head tok]
            float4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < KL; ++i) sc = M::qk(ka[i], qb[i], sc);
            float x[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                x[jj] = sc[jj] * a.qk_scale;
                if (MASKED && ctb + j * kStepTokens + 4 * kb + jj >= cte) x[jj] = -__builtin_inff();
                if (GROUPED && ctb + j * kStepTokens + 4 * kb + jj >= lim) x[jj] = -__builtin_inff();
            }
            // lazy running max: the rescale is a rare wave-uniform branch
            float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            if (__any(mx > m + kLazy)) {
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float mn = fmaxf(m, mx);
                const float alpha = fexp2(m - mn);
                lsum *= alpha;
#pragma unroll
                for (int d = 0; d < DS; ++d) acc[d] = acc[d] * alpha;
                m = mn;
            }
            float p[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) p[jj] = fexp2(x[jj] - m);
            lsum += (p[0] + p[1]) + (p[2] + p[3]);
            const vec2 pb = M::pack(p[0], p[1], p[2], p[3]);
            const vec2 pr = M::rest(p[0], p[1], p[2], p[3], pb);
#pragma unroll
            for (int d = 0; d < DS; ++d) {
                // O^T += V^T P^T: A operand V[token 4 kb + jj][dim 16 d + tok]
                const short4_t2 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (short4_t2 __attribute__((address_space(3))) *)(vtile + vbase +
                                                                     (((2 * d + vpc) ^ vswz) << 4)));
                const vec2 va = __builtin_bit_cast(vec2, t4);
                acc[d] = M::pv(va, pb, acc[d]);
                if constexpr (M::kSplit) acc[d] = M::pv(va, pr, acc[d]);
            }
        };

        vec4 ka[U], va[U], kc[U], vc[U];
        int j = wave;
        if (j < nfull) {
            issue.template operator()<false>(ka, va, j);
            while (j + 2 * nw < nfull) {
                issue.template operator()<false>(kc, vc, j + nw);
                __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
                compute.template operator()<false>(ka, va, j);
                issue.template operator()<false>(ka, va, j + 2 * nw);
                __builtin_amdgcn_sched_barrier(0);
                compute.template operator()<false>(kc, vc, j + nw);
                j += 2 * nw;
            }
            if (j + nw < nfull) {
                issue.template operator()<false>(kc, vc, j + nw);
                __builtin_amdgcn_sched_barrier(0);
                compute.template operator()<false>(ka, va, j);
                compute.template operator()<false>(kc, vc, j + nw);
            } else {
                compute.template operator()<false>(ka, va, j);
            }
        }
        if (tail && wave == nfull % nw) {
            issue.template operator()<true>(ka, va, nfull);
            compute.template operator()<true>(ka, va, nfull);
        }
    }

    // The four lanes of a head (tok, tok + 16, tok + 32, tok + 48) hold the
    // same max and partial sums over their tokens.
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);

    if constexpr (MODE != kDense)
        if (a.k_new && te == n) append_write<T, D>(a, trow, s, h, n, head0, tid);

    __syncthreads();  // table and V tiles are dead; reuse the LDS
    float *red = reinterpret_cast<float *>(smem);
    if (tok < G) {
        float *r = red + (wave * G + tok) * (D + 2);
#pragma unroll
        for (int d = 0; d < DS; ++d)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) r[16 * d + 4 * kb + jj] = acc[d][jj];
        if (kb == 0) {
            r[D] = m;
            r[D + 1] = lsum;
        }
    }
    __syncthreads();
    if constexpr (GROUPED)
        finish_group<T, D>(a, red, nw, G, s, h, part, cols, s_len, tid, nthr);
    else
        finish_workgroup<T, D, G>(a, red, nw, 1, qrow0, part, n, tid, nthr);
}

// Combines the partitions of one (sequence, query head): with M the largest
// partition max, out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
// Sequences that fit one partition were written by the decode kernel.
// 256 threads: thread t owns the 4-float chunk c = t % (D/4) of the row and
// partitions pg, pg + NG, ... (pg = t / (D/4)).  Up to NG * kMergeRegs
// partitions every thread issues all its loads before using any, so the
// kernel waits for memory once; the groups are summed in a fixed order
// through LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeRegs = 8;

template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    const float *ws_acc, const float *ws_ml, const int32_t *lens, void *out, int32_t Hq, int32_t P,
    int32_t PS, int32_t max_ctx) {
    constexpr int C4 = D / 4;                // float4 chunks per row
    constexpr int NG = kMergeThreads / C4;   // partition groups
    __shared__ float s_red[kMergeThreads / 64];
    __shared__ float4 s_acc[NG][C4];
    __shared__ float s_l[NG];
    const int qh = blockIdx.x;  // s * Hq + h
    const int s = qh / Hq;
    const int t = threadIdx.x;
    const float *ml = ws_ml + (int64_t)qh * P * 2;
    const float4 *ac = reinterpret_cast<const float4 *>(ws_acc + (int64_t)qh * P * D);
    const int c = t % C4, pg = t / C4;
    // Up to NG * kMergeRegs partitions the partials are requested together
    // with the length (addresses clamped to the P allocated partitions, so
    // they do not wait for it); entries past the sequence's own partitions
    // are dropped by selects below.
    const bool regs = P <= NG * kMergeRegs;
    float mp[kMergeRegs], lp[kMergeRegs];
    float4 x[kMergeRegs];
    if (regs) {
#pragma unroll
        for (int k = 0; k < kMergeRegs; ++k) {
            int pc = pg + k * NG;
            pc = pc < P ? pc : P - 1;
            mp[k] = ml[2 * pc];
            lp[k] = ml[2 * pc + 1];
            x[k] = ac[(int64_t)pc * C4 + c];
        }
    }
    const int n = clamp_len(lens[s], max_ctx);
    const int np = (n + PS - 1) / PS;
    if (np <= 1) return;

    auto block_max = [&](float x) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
        if ((t & 63) == 0) s_red[t >> 6] = x;
        __syncthreads();
        float M = s_red[0];
#pragma unroll
        for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, s_red[w]);
        return M;
    };

    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float lsum = 0.0f;
    if (regs) {
#pragma unroll
        for (int k = 0; k < kMergeRegs; ++k) {
            const bool ok = pg + k * NG < np;
            mp[k] = ok ? mp[k] : kNegBig;
            lp[k] = ok ? lp[k] : 0.0f;
            x[k] = ok ? x[k] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float mx = kNegBig;
#pragma unroll
        for (int k = 0; k < kMergeRegs; ++k) mx = fmaxf(mx, mp[k]);
        const float M = block_max(mx);
#pragma unroll
        for (int k = 0; k < kMergeRegs; ++k) {
            const float w = fexp2(mp[k] - M);  // 0 for the padding entries
            a.x = fmaf(x[k].x, w, a.x);
            a.y = fmaf(x[k].y, w, a.y);
            a.z = fmaf(x[k].z, w, a.z);
            a.w = fmaf(x[k].w, w, a.w);
            lsum = fmaf(lp[k], w, lsum);
        }
    } else {
        float mx = kNegBig;
        for (int p = t; p < np; p += kMergeThreads) mx = fmaxf(mx, ml[2 * p]);
        const float M = block_max(mx);
#pragma unroll 4
        for (int p = pg; p < np; p += NG) {
            const float w = fexp2(ml[2 * p] - M);
            const float4 x = ac[(int64_t)p * C4 + c];
            a.x = fmaf(x.x, w, a.x);
            a.y = fmaf(x.y, w, a.y);
            a.z = fmaf(x.z, w, a.z);
            a.w = fmaf(x.w, w, a.w);
            lsum = fmaf(ml[2 * p + 1], w, lsum);
        }
    }
    s_acc[pg][c] = a;
    if (c == 0) s_l[pg] = lsum;
    __syncthreads();
    if (t < C4) {
        float4 r = s_acc[0][t];
        float L = s_l[0];
#pragma unroll
        for (int g = 1; g < NG; ++g) {
            const float4 x = s_acc[g][t];
            r.x += x.x;
            r.y += x.y;
            r.z += x.z;
            r.w += x.w;
            L += s_l[g];
        }
        const int64_t o = (int64_t)qh * D + 4 * t;
        Elem<T>::store(out, o + 0, r.x / L);
        Elem<T>::store(out, o + 1, r.y / L);
        Elem<T>::store(out, o + 2, r.z / L);
        Elem<T>::store(out, o + 3, r.w / L);
    }
}

// The same combination for up to kMergeRowsP partitions, several rows per
// workgroup: thread t takes chunk t % (D/4) of row t / (D/4) and all its
// partitions (requested together with the length, addresses clamped to the
// P allocated partitions), summed in partition order; no LDS, no barrier.
constexpr int kMergeRowsP = 8;

template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_rows_kernel(
    const float *ws_acc, const float *ws_ml, const int32_t *lens, void *out, int32_t rows,
    int32_t Hq, int32_t P, int32_t PS, int32_t max_ctx) {
    constexpr int C4 = D / 4;
    constexpr int RPW = kMergeThreads / C4;  // rows per workgroup
    const int t = threadIdx.x;
    const int64_t qh = (int64_t)blockIdx.x * RPW + t / C4;
    if (qh >= rows) return;
    const int c = t % C4;
    const int s = (int)(qh / Hq);
    const float *ml = ws_ml + qh * P * 2;
    const float4 *ac = reinterpret_cast<const float4 *>(ws_acc + qh * P * D);
    float mp[kMergeRowsP], lp[kMergeRowsP];
    float4 x[kMergeRowsP];
#pragma unroll
    for (int k = 0; k < kMergeRowsP; ++k) {
        const int pc = k < P ? k : P - 1;
        mp[k] = ml[2 * pc];
        lp[k] = ml[2 * pc + 1];
        x[k] = ac[(int64_t)pc * C4 + c];
    }
    const int n = clamp_len(lens[s], max_ctx);
    const int np = (n + PS - 1) / PS;
    if (np <= 1) return;  // written by the decode kernel
    float M = kNegBig;
#pragma unroll
    for (int k = 0; k < kMergeRowsP; ++k) M = k < np ? fmaxf(M, mp[k]) : M;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.0f;
#pragma unroll
    for (int k = 0; k < kMergeRowsP; ++k) {
        if (k < np) {
            const float w = fexp2(mp[k] - M);
            a.x = fmaf(x[k].x, w, a.x);
            a.y = fmaf(x[k].y, w, a.y);
            a.z = fmaf(x[k].z, w, a.z);
            a.w = fmaf(x[k].w, w, a.w);
            L = fmaf(lp[k], w, L);
        }
    }
    const int64_t o = qh * D + 4 * c;
    Elem<T>::store(out, o + 0, a.x / L);
    Elem<T>::store(out, o + 1, a.y / L);
    Elem<T>::store(out, o + 2, a.z / L);
    Elem<T>::store(out, o + 3, a.w / L);
}

// Four consecutive output elements in one store, each rounded as
// Elem<T>::store rounds it (the index is a multiple of 4 and the row start
// 16-byte aligned, so the store is aligned).
template <typename T>
__device__ __forceinline__ void store4(void *out, int64_t i, float x0, float x1, float x2, float x3) {
    if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<float4 *>((float *)out + i) = make_float4(x0, x1, x2, x3);
    } else {
        typedef T t4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<t4 *>((T *)out + i) = t4{(T)x0, (T)x1, (T)x2, (T)x3};
    }
}

// The same combination with one wave per (sequence, query head) and up to
// kMergeWaveRegs partitions per lane: lane l takes the 4-float chunk
// l % (D/4) of the row and partitions l / (D/4), l / (D/4) + NG, ... (NG =
// 64 / (D/4) lane groups), all requested at once together with the length
// (addresses clamped to the P allocated partitions); the largest partition
// max and the group sums are combined by lane exchanges, so there is no LDS
// and no barrier, and each chunk leaves in one store.  The sum runs in a
// fixed order (partition order inside a lane, then the groups' butterfly).
constexpr int kMergeWaveRegs = 16;

template <typename T, int D>
__global__ __launch_bounds__(64) void merge_wave_kernel(
    const float *ws_acc, const float *ws_ml, const int32_t *lens, void *out, int32_t Hq, int32_t P,
    int32_t PS, int32_t max_ctx) {
    constexpr int C4 = D / 4;       // float4 chunks per row
    constexpr int NG = 64 / C4;     // lane groups (2 for D 128, 4 for D 64)
    const int64_t qh = blockIdx.x;  // s * Hq + h
    const int lane = threadIdx.x;
    const int c = lane % C4, grp = lane / C4;
    const float *ml = ws_ml + qh * P * 2;
    const float4 *ac = reinterpret_cast<const float4 *>(ws_acc + qh * P * D);
    float mp[kMergeWaveRegs], lp[kMergeWaveRegs];
    float4 x[kMergeWaveRegs];
#pragma unroll
    for (int k = 0; k < kMergeWaveRegs; ++k) {
        int pc = grp + k * NG;
        pc = pc < P ? pc : P - 1;
        mp[k] = ml[2 * pc];
        lp[k] = ml[2 * pc + 1];
        x[k] = ac[(int64_t)pc * C4 + c];
    }
    const int n = clamp_len(lens[qh / Hq], max_ctx);
    const int np = (n + PS - 1) / PS;
    if (np <= 1) return;  // written by the decode kernel
    float M = kNegBig;
#pragma unroll
    for (int k = 0; k < kMergeWaveRegs; ++k) M = grp + k * NG < np ? fmaxf(M, mp[k]) : M;
#pragma unroll
    for (int off = C4; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.0f;
#pragma unroll
    for (int k = 0; k < kMergeWaveRegs; ++k) {
        if (grp + k * NG < np) {
            const float w = fexp2(mp[k] - M);
            a.x = fmaf(x[k].x, w, a.x);
            a.y = fmaf(x[k].y, w, a.y);
            a.z = fmaf(x[k].z, w, a.z);
            a.w = fmaf(x[k].w, w, a.w);
            L = fmaf(lp[k], w, L);
        }
    }
    // Butterfly over the groups: every lane of a chunk ends with the same
    // bits (each step adds two equal-valued operands in swapped order).
#pragma unroll
    for (int off = C4; off < 64; off <<= 1) {
        a.x += __shfl_xor(a.x, off, 64);
        a.y += __shfl_xor(a.y, off, 64);
        a.z += __shfl_xor(a.z, off, 64);
        a.w += __shfl_xor(a.w, off, 64);
        L += __shfl_xor(L, off, 64);
    }
    if (grp == 0) store4<T>(out, qh * D + 4 * c, a.x / L, a.y / L, a.z / L, a.w / L);
}

// Workgroups of one kernel that a CU holds at once, at a given block size and
// dynamic LDS, times the CU count of the current device.  Queried once per
// (kernel, waves, device) and cached; the query itself is host-only.
struct ResidentKey {
    const void *fn;
    int nw, dev;
    size_t lds;
};

static int64_t resident_workgroups(const void *fn, int nw, size_t lds) {
    static std::mutex mu;
    static ResidentKey keys[64];
    static int64_t vals[64];
    static int n = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < n; ++i)
        if (keys[i].fn == fn && keys[i].nw == nw && keys[i].dev == dev && keys[i].lds == lds)
            return vals[i];
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64 * nw, lds) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int64_t r = (int64_t)per_cu * cus;
    if (n < 64) {
        keys[n] = ResidentKey{fn, nw, dev, lds};
        vals[n++] = r;
    }
    return r;
}

// Waves per workgroup of the VALU decode kernel (the matrix-core kernel has
// its own rule at its launch).  8 waves halve the steps each wave walks and double
// the loads a workgroup keeps in flight, which pays when the grid is small,
// but only while every workgroup is still resident at once: a grid that
// spills into a second round of workgroups finishes in two round trips of
// the longest workgroup.  So: 8 waves when the whole grid fits at 8; else 4
// when it fits at 4; else 8 for a grid under 1024 workgroups (fewer rounds
// of shorter workgroups) if 8-wave workgroups fit at all, and 4 beyond.
static int pick_waves(const void *fn8, const void *fn4, int64_t wgs, size_t lds8, size_t lds4) {
    if (fn8 == nullptr) return 4;
    const int64_t r8 = resident_workgroups(fn8, 8, lds8);  // 0 if 8 waves cannot be resident
    if (wgs <= r8) return 8;
    if (wgs <= resident_workgroups(fn4, 4, lds4)) return 4;
    return wgs < 1024 && r8 > 0 ? 8 : 4;
}

template <typename T, int D, int G>
static hipError_t launch_typed(const DecodeLaunch &l, hipStream_t st) {
    DecodeArgs a;
    a.q = (const char *)l.q;
    a.k = (const char *)l.k;
    a.v = (const char *)l.v;
    a.tables = l.tables;
    a.lens = l.lens;
    a.out = l.out;
    const int64_t units = (int64_t)l.S * l.Hq * l.P;
    a.ws_acc = l.PS ? l.ws : nullptr;
    a.ws_ml = l.PS ? l.ws + units * l.D : nullptr;
    a.qk_scale = l.scale * kLog2e;
    a.k_new = (const char *)l.k_new;
    a.v_new = (const char *)l.v_new;
    a.k_w = (char *)l.k_w;
    a.v_w = (char *)l.v_w;
    a.S = l.S;
    a.Hq = l.Hq;
    a.Hkv = l.Hkv;
    a.NB = l.NB;
    a.MBS = l.MBS;
    const int B = l.dense ? kStepTokens : l.B;
    int lb = 0;
    while ((1 << lb) < B) ++lb;
    a.log2B = lb;
    a.max_ctx = l.max_ctx;
    a.PS = l.PS;
    a.P = l.P;
    a.skip = nullptr;
    a.group_start = a.group_shared = nullptr;
    a.skip_out = nullptr;
    a.Gh = l.Hq / l.Hkv;
    a.Pg = 1;
    a.hg = 1;
    a.ips = l.Hkv;
    // Ranking costs the workgroup one dependent round trip; it pays only when
    // the grid is too large to be resident at once, so that order matters.
    a.rank = (l.PS == 0 && l.S > 1 && l.S <= kRankMaxSeqs && (int64_t)l.S * l.Hkv > 512) ? 1 : 0;
    {
        const int64_t span = l.PS ? (l.PS < l.max_ctx ? l.PS : l.max_ctx) : l.max_ctx;
        a.spec_blocks = (int32_t)((span + B - 1) / B);
    }
    const int64_t row = (int64_t)D * sizeof(T);        // one head's row
    const int64_t span = l.dense ? l.pos_stride : B;   // tokens per block / per sequence
    if (l.layout == 0) {  // token-major: [..., tokens, Hkv, D]
        a.tok_bytes = row * l.Hkv;
        a.head_bytes = row;
    } else {              // head-major: [..., Hkv, tokens, D]
        a.tok_bytes = row;
        a.head_bytes = row * span;
    }
    a.blk_bytes = l.dense ? 0 : row * l.Hkv * B;
    a.seq_bytes = l.dense ? row * l.Hkv * l.pos_stride : 0;
    const int64_t wgs = (int64_t)l.S * l.Hkv * l.P;
    dim3 grid((unsigned)wgs, 1, 1);
    auto red_bytes = [](int nw) { return (size_t)nw * G * (D + 2) * 4; };
    auto max2 = [](size_t x, size_t y) { return x > y ? x : y; };
    using Kern = void (*)(DecodeArgs);
    Kern fn;
    int nw;
    size_t lds;
    if constexpr (sizeof(T) == 2 && G >= 2) {  // grouped-query heads: matrix cores
        auto lds_of = [&](int w) {
            return max2((size_t)kTableChunk * 4 + (size_t)w * 2 * kStepTokens * 2 * D, red_bytes(w));
        };
        fn = l.dense ? decode_mma_kernel<T, D, G, kDense>
           : l.B >= kStepTokens ? decode_mma_kernel<T, D, G, kPagedWide>
                                : decode_mma_kernel<T, D, G, kPagedNarrow>;
        // The wave count follows one instantiation for every address mode, so
        // paged and dense launches of one shape split the work identically
        // (and give identical bits).
        // 8 waves only when the whole grid is resident at 8: past that, 4
        // waves ran 10-20% faster on the long-context grouped-query batch at
        // every partition size from 320 to 448 tokens (grids of 600-900
        // workgroups, a third of them without work), where the VALU
        // kernel's rule would take 8.
        const void *ref = (const void *)decode_mma_kernel<T, D, G, kPagedWide>;
        nw = wgs <= resident_workgroups(ref, 8, lds_of(8)) ? 8 : 4;
        lds = lds_of(nw);
    } else {
        auto lds_of = [&](int w) { return max2((size_t)kTableChunk * 4, red_bytes(w)); };
        fn = l.dense ? decode_kernel<T, D, G, kDense>
           : l.B >= kStepTokens ? decode_kernel<T, D, G, kPagedWide>
                                : decode_kernel<T, D, G, kPagedNarrow>;
        const void *ref = (const void *)decode_kernel<T, D, G, kPagedWide>;
        nw = pick_waves(max_waves<T>() >= 8 ? ref : nullptr, ref, wgs, lds_of(8), lds_of(4));
        lds = lds_of(nw);
        // Token-major pools keep a token's kv heads side by side: on grids of
        // at least two rounds of 4-wave workgroups, two adjacent kv heads
        // share an 8-wave workgroup (4 waves each, the same split of the
        // work, so the same bits), and their rows of a token are read
        // together (OPT-13B batch: 85.7 against 88.6 us; 128 x 64: 47.8
        // against 53.5; 128 x 2048: 831 against 859).  On 1.25 rounds (32
        // sequences x 40 heads) it was 3-7% slower, and on head-major pools,
        // where the two heads' rows are 4 KiB apart, 1% slower.
        if (l.layout == 0 && nw == 4 && max_waves<T>() >= 8 && l.Hkv % 2 == 0 &&
            l.n_groups == 0 && wgs >= 2 * resident_workgroups(ref, 4, lds_of(4))) {
            a.hg = 2;
            a.ips = l.Hkv / 2;
            nw = 8;
            lds = lds_of(8);
            grid = dim3((unsigned)((int64_t)l.S * a.ips * l.P), 1, 1);
        }
    }
    (void)hipGetLastError();  // an error left by other code is not this launch's
    if (l.n_groups > 0) {
        // The shared prefixes first: one workgroup per (group, kv head,
        // shared partition), the group's query heads as up to 16 score
        // columns; it also writes skip[] for the launch below.
        if constexpr (sizeof(T) == 2) {
            DecodeArgs g = a;
            g.PS = l.PSg;
            g.rank = 0;
            g.spec_blocks = (int32_t)(((l.PSg < l.max_ctx ? l.PSg : l.max_ctx) + B - 1) / B);
            g.group_start = l.group_start;
            g.group_shared = l.group_shared;
            g.skip_out = l.skip;
            const int64_t sp_max = (int64_t)l.max_shared_blocks * B / l.PSg;
            g.Pg = (int32_t)(sp_max < 1 ? 1 : (sp_max > l.P ? l.P : sp_max));
            const int64_t gwgs = (int64_t)l.n_groups * l.Hkv * g.Pg;
            using Kern = void (*)(DecodeArgs);
            const Kern gfn = l.B >= kStepTokens ? decode_mma_kernel<T, D, 16, kPagedWide, true>
                                                : decode_mma_kernel<T, D, 16, kPagedNarrow, true>;
            auto glds = [&](int w) {
                return max2((size_t)kTableChunk * 4 + (size_t)w * 2 * kStepTokens * 2 * D,
                            (size_t)w * 16 * (D + 2) * 4);
            };
            const void *gref = (const void *)decode_mma_kernel<T, D, 16, kPagedWide, true>;
            const int gnw = gwgs <= resident_workgroups(gref, 8, glds(8)) ? 8 : 4;
            hipLaunchKernelGGL(gfn, dim3((unsigned)gwgs), dim3(64 * gnw), glds(gnw), st, g);
            const hipError_t ge = hipGetLastError();
            if (ge != hipSuccess) return ge;
            a.skip = l.skip;
            a.rank = 0;
        } else {
            return hipErrorInvalidValue;
        }
    }
    hipLaunchKernelGGL(fn, grid, dim3(64 * nw), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || l.PS == 0) return e;
    const int64_t rows = (int64_t)l.S * l.Hq;
    if (l.P <= kMergeRowsP) {
        constexpr int RPW = kMergeThreads / (D / 4);
        hipLaunchKernelGGL((merge_rows_kernel<T, D>), dim3((unsigned)((rows + RPW - 1) / RPW)),
                           dim3(kMergeThreads), 0, st, a.ws_acc, a.ws_ml, l.lens, l.out,
                           (int32_t)rows, l.Hq, l.P, l.PS, l.max_ctx);
    } else if (l.P <= kMergeWaveRegs * (64 / (D / 4))) {
        hipLaunchKernelGGL((merge_wave_kernel<T, D>), dim3((unsigned)rows), dim3(64), 0, st,
                           a.ws_acc, a.ws_ml, l.lens, l.out, l.Hq, l.P, l.PS, l.max_ctx);
    } else {
        hipLaunchKernelGGL((merge_kernel<T, D>), dim3((unsigned)rows), dim3(kMergeThreads), 0, st,
                           a.ws_acc, a.ws_ml, l.lens, l.out, l.Hq, l.P, l.PS, l.max_ctx);
    }
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_g(const DecodeLaunch &l, hipStream_t st) {
    switch (l.Hq / l.Hkv) {
        case 1: return launch_typed<T, D, 1>(l, st);
        case 2: return launch_typed<T, D, 2>(l, st);
        case 3: return launch_typed<T, D, 3>(l, st);
        case 4: return launch_typed<T, D, 4>(l, st);
        case 5: return launch_typed<T, D, 5>(l, st);
        case 6: return launch_typed<T, D, 6>(l, st);
        case 7: return launch_typed<T, D, 7>(l, st);
        case 8: return launch_typed<T, D, 8>(l, st);
    }
    // 9 .. 16 query heads per kv head: 16-bit types only, on the matrix
    // cores, whose score tile has 16 head columns
    if constexpr (sizeof(T) == 2) {
        switch (l.Hq / l.Hkv) {
            case 9: return launch_typed<T, D, 9>(l, st);
            case 10: return launch_typed<T, D, 10>(l, st);
            case 11: return launch_typed<T, D, 11>(l, st);
            case 12: return launch_typed<T, D, 12>(l, st);
            case 13: return launch_typed<T, D, 13>(l, st);
            case 14: return launch_typed<T, D, 14>(l, st);
            case 15: return launch_typed<T, D, 15>(l, st);
            case 16: return launch_typed<T, D, 16>(l, st);
        }
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_d(const DecodeLaunch &l, hipStream_t st) {
    return l.D == 64 ? launch_g<T, 64>(l, st) : launch_g<T, 128>(l, st);
}

int launch_decode(const DecodeLaunch &l, void *stream) {
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    switch (l.dtype) {
        case 0: e = launch_d<float>(l, st); break;
        case 1: e = launch_d<_Float16>(l, st); break;
        default: e = launch_d<__bf16>(l, st); break;
    }
    return (int)e;
}

// ---------------------------------------------------------------- prefill

// Multi-token queries over the paged cache: prompt and chunked-prefill
// attention ([Kwon] §3.4: in the prompt phase every token attends to itself
// and the tokens before it, and the paged kernel reads keys and values
// through the block table).  Sequence s owns query rows qstart[s] ..
// qstart[s+1]-1, the last T of its n cached tokens (their keys and values
// are already in the pool); chunk row r sits at position n - T + r and
// attends to positions 0 .. n - T + r.
//
// One workgroup of 4 waves per (query head, sequence, 128-row tile of its
// chunk); each wave owns two 16-row column tiles, which share every K and
// V^T operand it reads from LDS.  The workgroup walks the keys in LDS tiles
// of 64: the tile's K and V rows go from the pool straight into LDS (16-byte
// LDS DMA per lane, no registers), one tile ahead of the one being computed,
// two stages, one barrier per tile.  Rows are stored unpadded with their
// 16-byte pieces permuted per row (an XOR swizzle) so that the operand reads
// below hit distinct banks.  For each pair of 16-key sub-tiles (32 keys) a
// wave computes its score tiles on matrix cores as S^T = K Q^T (K from LDS as
// the A operand, Q^T held in registers), updates its running softmax per
// query column, and accumulates O^T += V^T P^T on 16x16x32 products whose
// k-slots hold keys 4 kb .. 4 kb + 3 of both sub-tiles: V^T comes from LDS
// through the transposing ds_read_b64_tr_b16 (lane l addresses row l / 4,
// columns d0 + 4 (l % 4), and receives V[4 (l / 16) + j][d0 + l % 16], the
// A-operand layout), and the score tiles' weights, packed, are the B operand
// as they stand.  The weights' sum per query column is one more product, with
// an all-ones A operand, so it is formed from the same rounded weights as the
// output.  The causal mask and the chunk's end are applied only on the pairs
// that need them.  The running max of a query column moves only when a score
// exceeds it by more than 2^8 (weights then stay <= 256, exact in fp16 /
// bf16, and the final division by the running sum is unchanged in exact
// arithmetic), so the accumulator rescale runs in a rare wave-uniform branch
// instead of on every tile.  fp16 and bf16.
struct PrefillArgs {
    const char *q, *k, *v;
    const int32_t *tables, *lens, *qstart;
    void *out;
    float qk_scale;  // scale * log2(e)
    int32_t S, Hq, Hkv, NB, MBS, log2B, max_ctx, max_q, total_rows, tiles;
    int32_t xcd_heads;  // grid x permuted so a kv head's query heads share an XCD
    int64_t tok_bytes, head_bytes, blk_bytes;
};

constexpr int kPrefillWaves = 4;
constexpr int kPrefillCols = 2;  // 16-row column tiles per wave
constexpr int kPrefillKeys = 64;  // keys per LDS tile (one barrier per tile)
constexpr int kPrefillRows = 16 * kPrefillCols * kPrefillWaves;  // query rows per workgroup
static_assert(kPrefillRows == kPrefillTileRows, "the host checks grid z with kPrefillTileRows");

// 16 bytes per lane from global memory straight into LDS: lane i's piece
// lands at LDS byte address lds + 16 i (lds wave-uniform).  M0 carries the
// LDS address; it is an operand of the asm, so the compiler loads it (and
// knows it is clobbered).  The load counts in vmcnt like any other vector
// load; the compiler does not track it, so the caller waits (lds_dma_wait)
// before any wave reads what it wrote.
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
// The same with a wave-uniform 64-bit base in scalar registers and a
// per-lane 32-bit offset (the instruction adds them), which saves the
// per-lane 64-bit address.
__device__ __forceinline__ void lds_dma16_s(const char *base, uint32_t off, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds)
                 : "memory");
}
__device__ __forceinline__ void lds_dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }


template <typename T, int D, int NQ>
__global__ __launch_bounds__(kPrefillWaves * 64, 2) void prefill_kernel(PrefillArgs a) {
    using E = Elem<T>;
    using M = Mma<T>;
    constexpr int KL = D / 32;           // 32-dim slices of the score product
    constexpr int DS = D / 16;           // 16-dim slices of the output
    constexpr int ROWB = D * 2;          // bytes per K / V row
    constexpr int CPR = ROWB / 16;       // 16-byte pieces per row
    constexpr int KT = kPrefillKeys;     // keys per LDS tile: two pairs of 16-key sub-tiles
    constexpr int TILEB = KT * ROWB;     // bytes of K (or V) per tile
    constexpr int RPI = 64 / CPR;        // rows per DMA instruction
    constexpr int NI = KT / RPI / kPrefillWaves;  // DMA instructions per wave per tensor
    static_assert(NI * RPI * kPrefillWaves == KT, "whole DMA instructions per wave");
    constexpr int WROWS = 16 * NQ;       // query rows per wave
    constexpr int GROWS = WROWS * kPrefillWaves;

    __shared__ int32_t s_tab[kTableChunk];
    __shared__ __attribute__((aligned(16))) char s_kv[2][2][TILEB];  // [stage][K, V][tile]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;  // key row of the A operand; query column of the scores
    const int kb = lane >> 4;   // k-block of the operands; 4-key group of the scores
    // Grid (heads, sequences, tiles), dispatched x first: the last tiles of
    // every chunk, which see the most keys, start first.  Consecutive
    // workgroups go to the eight XCDs in turn, so with a multiple of eight
    // heads x = 8 r + x8 runs on XCD x8; when the kv heads are a multiple of
    // eight too, x maps to query head (8 (r / R) + x8) R + r % R (R query
    // heads per kv head), which puts all R heads of a kv head on one XCD,
    // where they read the same keys and values through one L2.
    const int R = a.Hq / a.Hkv;
    const int h = a.xcd_heads ? ((((int)blockIdx.x >> 3) / R) * 8 + ((int)blockIdx.x & 7)) * R +
                                    (((int)blockIdx.x >> 3) % R)
                              : (int)blockIdx.x;
    const int s = blockIdx.y;
    const int tile = a.tiles - 1 - (int)blockIdx.z;
    const int g = h / R;

    // The chunk's rows, clamped so that no access leaves q, out or the table.
    int q0 = a.qstart[s], q1 = a.qstart[s + 1];
    q0 = q0 < 0 ? 0 : (q0 > a.total_rows ? a.total_rows : q0);
    q1 = q1 < q0 ? q0 : (q1 > a.total_rows ? a.total_rows : q1);
    const int n = clamp_len(a.lens[s], a.max_ctx);
    int rows = q1 - q0;  // chunk length
    rows = rows > a.max_q ? a.max_q : rows;
    rows = rows > n ? n : rows;
    const int tr0 = tile * GROWS;
    if (tr0 >= rows) return;  // the whole workgroup idles
    const int r0 = tr0 + WROWS * wave;                         // this wave's first row
    const int rows_w = rows - r0 < 0 ? 0 : (rows - r0 > WROWS ? WROWS : rows - r0);
    const int w_last = rows_w ? n - rows + r0 + rows_w - 1 : -1;  // last key of this wave
    const int nkeys = n - rows + (tr0 + GROWS < rows ? tr0 + GROWS : rows);  // of the WG

    // Column tile c holds rows r0 + 16 c + col.  B operand of S^T = K Q^T:
    // that row's dims 32 i + 8 kb .. + 7 (zero past the chunk).
    vec4 qb[NQ][KL];
    int my_pos[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const int r = r0 + 16 * c + col;
        my_pos[c] = n - rows + r;
        const int64_t qrow = (int64_t)(q0 + r) * a.Hq + h;
#pragma unroll
        for (int i = 0; i < KL; ++i)
            qb[c][i] = r < rows ? load_cached(a.q + (qrow * D + 32 * i + 8 * kb) * 2)
                                : vec4{0u, 0u, 0u, 0u};
    }
    // Scores stay in raw units (q.k) and the scale enters once per weight:
    // p = 2^(s (x - m)) = 2^(fma(s, x, -s m)) with s = |scale| log2 e > 0.  A
    // negative scale is moved onto q, whose sign flip is exact.
    const float sc_abs = fabsf(a.qk_scale);
    if (a.qk_scale < 0.0f) {
#pragma unroll
        for (int c = 0; c < NQ; ++c)
#pragma unroll
            for (int i = 0; i < KL; ++i) qb[c][i] ^= vec4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    }
    // Running max m (raw units) per query column, and the two values derived
    // from it that the loop uses: thr = m + 2^kLazy-in-raw-units (a score
    // above it moves the max) and nms = -s m.  The start value is finite and
    // far below any score, so -s m stays finite.
    constexpr float kRawStart = -1.0e30f;
    const float lazy_raw = kLazy / sc_abs;
    float m[NQ], thr[NQ], nms[NQ];
    float4_t acc[NQ][DS], accl[NQ];
    const vec4 ones = M::ones();
    const int mask_free_rows = n - rows + r0;  // keys up to here are visible to every row
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        m[c] = kRawStart;
        thr[c] = kRawStart + lazy_raw;
        nms[c] = -sc_abs * kRawStart;
        accl[c] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < DS; ++d) acc[c][d] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Loop-invariant LDS offsets of this lane's operand reads (within a
    // 16-row sub-tile): K slice i (row col, piece 4 i + kb) and the
    // transposing V^T read of slice d (row lane / 4, bytes 32 d + 8 (lane % 4)).
    uint32_t koff[KL], voff[DS];
#pragma unroll
    for (int i = 0; i < KL; ++i)
        koff[i] = col * ROWB + (((4 * i + kb) ^ row_swz<D>(col)) << 4);
#pragma unroll
    for (int d = 0; d < DS; ++d)
        voff[d] = (lane >> 2) * ROWB + (((2 * d + ((lane & 3) >> 1)) ^ row_swz<D>(lane >> 2)) << 4) +
                  8 * (lane & 1);

    const int B = 1 << a.log2B;
    const int32_t *trow = a.tables + (int64_t)s * a.MBS;
    const int64_t head0 = (int64_t)g * a.head_bytes;
    // Scalar DMA addressing needs an instruction's rows inside one block; a
    // lane's offset from the instruction's first row then fits 32 bits (RPI
    // rows of at most 128 MiB each) and does not change from tile to tile.
    const bool fast_dma = B >= RPI;
    uint32_t lane_off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = (wave * NI + i) * RPI + lane / CPR;
        lane_off[i] = (uint32_t)(lane / CPR) * (uint32_t)a.tok_bytes +
                      ((uint32_t)((lane % CPR) ^ row_swz<D>(r)) << 4);
    }
    const int nblk = (nkeys + B - 1) >> a.log2B;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)&s_kv[0][0][0];

    for (int cb = 0; cb < nblk; cb += kTableChunk) {
        const int cn = nblk - cb < kTableChunk ? nblk - cb : kTableChunk;
        const int ck0 = cb << a.log2B;
        const int ck1 = (cb + cn) << a.log2B < nkeys ? (cb + cn) << a.log2B : nkeys;
        const int nst = (ck1 - ck0 + KT - 1) / KT;
        const int mask_free = min(mask_free_rows, ck1 - 1);
        __syncthreads();  // the previous chunk's readers are done
        stage_table(trow, cb, cn, a.NB, s_tab, tid, blockDim.x);
        // The q loads complete here, with the first chunk's table entries
        // (their round trips overlap; on later chunks this is a no-op): a
        // wait for q must not fall inside the key loop, where it would also
        // wait for the LDS DMA in flight.
#pragma unroll
        for (int c = 0; c < NQ; ++c)
#pragma unroll
            for (int i = 0; i < KL; ++i) asm volatile("" ::"v"(qb[c][i]));
        __syncthreads();

        // DMA of tile j (keys clamped to the chunk, so rows past its end
        // reload its last key) into stage st: instruction ins of the tile
        // fills rows ins * RPI .. + RPI - 1; lane l the piece at position
        // l % CPR of its row, i.e. global piece (l % CPR) ^ swz(row).
        // When the whole tile lies inside the chunk and an instruction's RPI
        // rows lie in one block (block size >= RPI, rows RPI-aligned), the
        // block id and the block's base are wave-uniform (scalar registers)
        // and a lane adds only its loop-invariant row and piece offset.
        // Otherwise every lane translates its own row.  The table entries
        // are all read before the first DMA: the DMA's asm orders memory, so
        // a read placed after one would wait for it.
        auto issue = [&](int j, int st) {
            const int tt0 = ck0 + KT * j;  // first key of tile j
            if (fast_dma && tt0 + KT <= ck1) {
                int64_t base[NI];
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int t = tt0 + (wave * NI + i) * RPI;  // first row of the instruction
                    const int blk = __builtin_amdgcn_readfirstlane(s_tab[(t - ck0) >> a.log2B]);
                    base[i] = (int64_t)blk * a.blk_bytes + (int64_t)(t & (B - 1)) * a.tok_bytes + head0;
                }
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int ins = wave * NI + i;
                    const uint32_t dk = lds0 + (uint32_t)((st * 2 + 0) * TILEB + ins * 1024);
                    const uint32_t dv = lds0 + (uint32_t)((st * 2 + 1) * TILEB + ins * 1024);
                    lds_dma16_s(a.k + base[i], lane_off[i], __builtin_amdgcn_readfirstlane(dk));
                    lds_dma16_s(a.v + base[i], lane_off[i], __builtin_amdgcn_readfirstlane(dv));
                }
                return;
            }
            int64_t off[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int ins = wave * NI + i;
                const int r = ins * RPI + lane / CPR;
                int t = tt0 + r;
                t = t < ck1 ? t : ck1 - 1;
                off[i] = (int64_t)s_tab[(t - ck0) >> a.log2B] * a.blk_bytes +
                         (int64_t)(t & (B - 1)) * a.tok_bytes + head0 +
                         (((lane % CPR) ^ row_swz<D>(r)) << 4);
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int ins = wave * NI + i;
                const uint32_t dk = lds0 + (uint32_t)((st * 2 + 0) * TILEB + ins * 1024);
                const uint32_t dv = lds0 + (uint32_t)((st * 2 + 1) * TILEB + ins * 1024);
                lds_dma16(a.k + off[i], __builtin_amdgcn_readfirstlane(dk));
                lds_dma16(a.v + off[i], __builtin_amdgcn_readfirstlane(dv));
            }
        };

        // One pair of 16-key sub-tiles (keys key0 .. key0 + 31, rows 16 u ..
        // 16 u + 31 of stage st).
        // K operands (A of S^T = K Q^T) of both 16-key sub-tiles of a pair.
        // The second pair of a tile gets its operands requested under the
        // first pair's softmax and P V (knext), so its score products need
        // not wait for LDS.
        vec4 knext[2][KL];
        auto loadK = [&](int st, int u, vec4 (&kk)[2][KL]) __attribute__((always_inline)) {
            const char *kt = &s_kv[st][0][0] + 16 * u * ROWB;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < KL; ++i)
                    kk[hh][i] = *reinterpret_cast<const vec4 *>(kt + hh * 16 * ROWB + koff[i]);
        };
        auto pair = [&](int st, int u, int key0, bool kready, bool pre) __attribute__((always_inline)) {
            const char *vt = &s_kv[st][1][0] + 16 * u * ROWB;
            const bool masked = key0 + 31 > mask_free;  // wave-uniform
            // K operands of both sub-tiles, requested together (the second
            // sub-tile's rows are in LDS whether or not they are used), or
            // taken from the previous pair's request
            vec4 ka2[2][KL];
            if (kready) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int i = 0; i < KL; ++i) ka2[hh][i] = knext[hh][i];
            } else {
                loadK(st, u, ka2);
            }
            // A operand of O^T += V^T P^T over 32 keys: lane l holds keys
            // 4 kb .. 4 kb + 3 of both sub-tiles (k-slots 8 kb .. 8 kb + 7)
            vec4 va[DS];
#pragma unroll
            for (int d = 0; d < DS; ++d) {
                const short4_t2 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (short4_t2 __attribute__((address_space(3))) *)(vt + voff[d]));
                const short4_t2 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (short4_t2 __attribute__((address_space(3))) *)(vt + 16 * ROWB + voff[d]));
                const vec2 l2 = __builtin_bit_cast(vec2, lo), h2 = __builtin_bit_cast(vec2, hi);
                va[d] = vec4{l2.x, l2.y, h2.x, h2.y};
            }
            // The four score chains (2 sub-tiles x NQ column tiles) advance
            // together, so consecutive products never depend on each other.
            float4_t sc[2][NQ];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int c = 0; c < NQ; ++c) sc[hh][c] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < KL; ++i)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int c = 0; c < NQ; ++c) sc[hh][c] = M::qk(ka2[hh][i], qb[c][i], sc[hh][c]);
            if (pre) loadK(st, u + 2, knext);  // the next pair's K, in flight under this softmax
            // Keys past the wave's last row (all of the second sub-tile when
            // key0 + 16 > w_last) are hidden by the causal mask below, which
            // applies whenever that holds (mask_free <= w_last).
            float x[2][NQ][4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int c = 0; c < NQ; ++c)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) x[hh][c][jj] = sc[hh][c][jj];
            if (masked) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int c = 0; c < NQ; ++c) {
                        // keys key0 + 16 hh + 4 kb + jj with jj > lim are hidden
                        // (causal, or past the chunk's end)
                        const int lim = min(my_pos[c], ck1 - 1) - (key0 + 16 * hh + 4 * kb);
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            x[hh][c][jj] = jj > lim ? -__builtin_inff() : x[hh][c][jj];
                    }
            }
            bool grow = false;
            float mxc[NQ];
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                const float a0 = max3f(x[0][c][0], x[0][c][1], x[0][c][2]);
                const float a1 = max3f(x[0][c][3], x[1][c][0], x[1][c][1]);
                mxc[c] = max3f(max3f(a0, a1, x[1][c][2]), x[1][c][3], x[1][c][3]);
                grow |= mxc[c] > thr[c];
            }
            if (__any(grow)) {
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    float mx = mxc[c];
                    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                    const float mn = fmaxf(m[c], mx);
                    const float alpha = fexp2(fmaf(sc_abs, m[c], -sc_abs * mn));
                    m[c] = mn;
                    thr[c] = mn + lazy_raw;
                    nms[c] = -sc_abs * mn;
                    accl[c] = accl[c] * alpha;
#pragma unroll
                    for (int d = 0; d < DS; ++d) acc[c][d] = acc[c][d] * alpha;
                }
            }
            vec4 pb[NQ], pr[NQ];
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                float p[2][4];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) p[hh][jj] = fexp2(fmaf(sc_abs, x[hh][c][jj], nms[c]));
                const vec2 b0 = M::pack(p[0][0], p[0][1], p[0][2], p[0][3]);
                const vec2 b1 = M::pack(p[1][0], p[1][1], p[1][2], p[1][3]);
                pb[c] = vec4{b0.x, b0.y, b1.x, b1.y};
                if constexpr (M::kSplit) {
                    const vec2 e0 = M::rest(p[0][0], p[0][1], p[0][2], p[0][3], b0);
                    const vec2 e1 = M::rest(p[1][0], p[1][1], p[1][2], p[1][3], b1);
                    pr[c] = vec4{e0.x, e0.y, e1.x, e1.y};
                }
            }
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                // the weights' sum over the 32 keys, as one more output row
                accl[c] = M::pv32(ones, pb[c], accl[c]);
                if constexpr (M::kSplit) accl[c] = M::pv32(ones, pr[c], accl[c]);
            }
#pragma unroll
            for (int d = 0; d < DS; ++d) {
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    acc[c][d] = M::pv32(va[d], pb[c], acc[c][d]);
                    if constexpr (M::kSplit) acc[c][d] = M::pv32(va[d], pr[c], acc[c][d]);
                }
            }
        };

        // Tile j: wait for this thread's DMA of it, barrier (every wave's
        // DMA of tile j has landed, and every wave is done with tile j - 1),
        // start tile j + 1 into the other stage, compute tile j.
        auto step = [&](int st, int j) {
            lds_dma_wait();
            __syncthreads();
            if (j + 1 < nst) issue(j + 1, st ^ 1);
            const int key0 = ck0 + KT * j;
            if (key0 > w_last) return;  // wave-uniform: the whole tile is past this wave's rows
            const bool two = key0 + 32 <= w_last;
            pair(st, 0, key0, false, two);
            if (two) pair(st, 2, key0 + 32, true, false);
        };
        issue(0, 0);
        for (int j = 0; j < nst; j += 2) {
            step(0, j);
            if (j + 1 >= nst) break;
            step(1, j + 1);
        }
    }

    // (q was consumed in the loop; consuming it here too tells the compiler
    // so on every path, and keeps its waits out of the stores below.)
#pragma unroll
    for (int c = 0; c < NQ; ++c)
#pragma unroll
        for (int i = 0; i < KL; ++i) asm volatile("" ::"v"(qb[c][i]));
    // Every lane of a query column holds the column's full weight sum.
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const float l = accl[c][0];
        const int r = r0 + 16 * c + col;
        if (r < rows) {
            const float inv = 1.0f / l;
            const int64_t o = ((int64_t)(q0 + r) * a.Hq + h) * D;
#pragma unroll
            for (int d = 0; d < DS; ++d)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    E::store(a.out, o + 16 * d + 4 * kb + jj, acc[c][d][jj] * inv);
        }
    }
    // The DMA of a tile this wave did not compute (its rows end earlier) may
    // still be in flight: let it land before the workgroup's LDS is released.
    lds_dma_wait();
}

template <typename T>
static hipError_t launch_prefill_t(const PrefillLaunch &l, hipStream_t st) {
    PrefillArgs a;
    a.q = (const char *)l.q;
    a.k = (const char *)l.k;
    a.v = (const char *)l.v;
    a.tables = l.tables;
    a.lens = l.lens;
    a.qstart = l.qstart;
    a.out = l.out;
    a.qk_scale = l.scale * kLog2e;
    a.S = l.S;
    a.Hq = l.Hq;
    a.Hkv = l.Hkv;
    a.NB = l.NB;
    a.MBS = l.MBS;
    int lb = 0;
    while ((1 << lb) < l.B) ++lb;
    a.log2B = lb;
    a.max_ctx = l.max_ctx;
    a.max_q = l.max_q;
    a.total_rows = l.total_rows;
    a.tiles = (l.max_q + kPrefillRows - 1) / kPrefillRows;
    a.xcd_heads = l.Hkv % 8 == 0 && l.Hq > l.Hkv;
    const int64_t row = (int64_t)l.D * sizeof(T);
    if (l.layout == 0) {
        a.tok_bytes = row * l.Hkv;
        a.head_bytes = row;
    } else {
        a.tok_bytes = row;
        a.head_bytes = row * l.B;
    }
    a.blk_bytes = row * l.Hkv * l.B;
    const dim3 grid((unsigned)l.Hq, (unsigned)l.S, (unsigned)a.tiles);
    (void)hipGetLastError();  // an error left by other code is not this launch's
    if (l.D == 64)
        hipLaunchKernelGGL((prefill_kernel<T, 64, kPrefillCols>), grid, dim3(kPrefillWaves * 64), 0,
                           st, a);
    else
        hipLaunchKernelGGL((prefill_kernel<T, 128, kPrefillCols>), grid, dim3(kPrefillWaves * 64),
                           0, st, a);
    return hipGetLastError();
}

int launch_prefill(const PrefillLaunch &l, void *stream) {
    if (l.S == 0 || l.max_q == 0 || l.total_rows == 0) return 0;
    hipStream_t st = (hipStream_t)stream;
    return (int)(l.dtype == 1 ? launch_prefill_t<_Float16>(l, st) : launch_prefill_t<__bf16>(l, st));
}

// ---------------------------------------------------------------- cache_write

// One flat range of 16-byte vectors: token i's K rows, then its V rows, each
// [Hkv, D] in the source.  Vector w of token i belongs to kv head g = w / rv
// and goes to block slot / B, offset slot % B of that head in the pool
// layout given by the strides.  Out-of-range slots are skipped ([Kwon] §3.4
// "Kernel-Level Optimizations", item 1: one fused launch writes every new
// token to the block and slot the scheduler names).
// The new tokens' K and V rows into their slots: work item idx moves one
// 16-byte piece (token i, K or V, kv head g, piece x), grid-strided.
__device__ __forceinline__ void write_rows(const vec4 *__restrict__ k_new,
                                           const vec4 *__restrict__ v_new, char *__restrict__ k_cache,
                                           char *__restrict__ v_cache,
                                           const int32_t *__restrict__ slots, int64_t total, int64_t rv,
                                           int32_t hkv, int32_t log2B, int64_t num_slots,
                                           int64_t blk_bytes, int64_t tok_bytes, int64_t head_bytes) {
    const int64_t per_tensor = (int64_t)hkv * rv;    // vectors of K (or V) per token
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += stride) {
        const int64_t i = idx / (2 * per_tensor);
        int64_t w = idx - i * 2 * per_tensor;
        const bool is_v = w >= per_tensor;
        if (is_v) w -= per_tensor;
        const int32_t slot = slots[i];
        if (slot < 0 || slot >= num_slots) continue;
        const int64_t g = w / rv, x = w - g * rv;
        const int64_t dst = (int64_t)(slot >> log2B) * blk_bytes +
                            (int64_t)(slot & ((1 << log2B) - 1)) * tok_bytes + g * head_bytes +
                            x * 16;
        const vec4 val = is_v ? v_new[i * per_tensor + w] : k_new[i * per_tensor + w];
        *reinterpret_cast<vec4 *>((is_v ? v_cache : k_cache) + dst) = val;
    }
}

__global__ __launch_bounds__(kThreads) void cache_write_kernel(
    const vec4 *__restrict__ k_new, const vec4 *__restrict__ v_new, char *__restrict__ k_cache,
    char *__restrict__ v_cache, const int32_t *__restrict__ slots, int64_t total, int64_t rv,
    int32_t hkv, int32_t log2B, int64_t num_slots, int64_t blk_bytes, int64_t tok_bytes,
    int64_t head_bytes) {
    write_rows(k_new, v_new, k_cache, v_cache, slots, total, rv, hkv, log2B, num_slots, blk_bytes,
               tok_bytes, head_bytes);
}

// Every layer's new rows in one launch: grid y = layer.
__global__ __launch_bounds__(kThreads) void cache_write_layers_kernel(
    CacheWriteLayers w, const int32_t *__restrict__ slots, int64_t total, int64_t rv, int32_t hkv,
    int32_t log2B, int64_t num_slots, int64_t blk_bytes, int64_t tok_bytes, int64_t head_bytes) {
    const int l = blockIdx.y;
    write_rows((const vec4 *)w.k_new[l], (const vec4 *)w.v_new[l], (char *)w.k_cache[l],
               (char *)w.v_cache[l], slots, total, rv, hkv, log2B, num_slots, blk_bytes, tok_bytes,
               head_bytes);
}

// Launch geometry and pool strides shared by the single- and multi-layer
// writes.
struct WriteGeom {
    int64_t rv, total, blk_bytes, tok_bytes, head_bytes, blocks;
    int log2B;
};
static WriteGeom write_geom(int32_t n, int32_t block_size, int32_t hkv, int64_t row_bytes,
                            int32_t layout) {
    WriteGeom g;
    g.rv = row_bytes / 16;  // vectors per head row
    g.total = (int64_t)n * 2 * hkv * g.rv;
    g.log2B = 0;
    while ((1 << g.log2B) < block_size) ++g.log2B;
    g.blk_bytes = row_bytes * hkv * block_size;
    g.tok_bytes = layout == 0 ? row_bytes * hkv : row_bytes;
    g.head_bytes = layout == 0 ? row_bytes : row_bytes * block_size;
    g.blocks = (g.total + kThreads * 4 - 1) / (kThreads * 4);
    if (g.blocks > 65536) g.blocks = 65536;
    if (g.blocks < 1) g.blocks = 1;
    return g;
}

int launch_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       const int32_t *slots, int32_t n, int32_t num_blocks, int32_t block_size,
                       int32_t hkv, int64_t row_bytes, int32_t layout, void *stream) {
    const WriteGeom g = write_geom(n, block_size, hkv, row_bytes, layout);
    (void)hipGetLastError();  // an error left by other code is not this launch's
    hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)g.blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, (const vec4 *)k_new, (const vec4 *)v_new,
                       (char *)k_cache, (char *)v_cache, slots, g.total, g.rv, hkv, g.log2B,
                       (int64_t)num_blocks * block_size, g.blk_bytes, g.tok_bytes, g.head_bytes);
    return (int)hipGetLastError();
}

int launch_cache_write_layers(const CacheWriteLayers &w, const int32_t *slots, int32_t n,
                              int32_t num_blocks, int32_t block_size, int32_t hkv,
                              int64_t row_bytes, int32_t layout, void *stream) {
    const WriteGeom g = write_geom(n, block_size, hkv, row_bytes, layout);
    (void)hipGetLastError();  // an error left by other code is not this launch's
    hipLaunchKernelGGL(cache_write_layers_kernel, dim3((unsigned)g.blocks, (unsigned)w.layers),
                       dim3(kThreads), 0, (hipStream_t)stream, w, slots, g.total, g.rv, hkv,
                       g.log2B, (int64_t)num_blocks * block_size, g.blk_bytes, g.tok_bytes,
                       g.head_bytes);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- block moves

// Whole-block copies for every (src, dst) pair, K and V, for up to
// kMaxLayers layers in one launch ([Kwon] §3.4 "Kernel-Level Optimizations",
// item 3: one fused copy over all layers taking (source, destination)
// pairs; "Scheduling and Preemption": swapping moves the same blocks
// between the GPU pool and a host pool).  A block is one contiguous range in
// either pool layout.  Grid: x = (pair, layer, K|V), y = 16 KiB chunks of
// the block; each thread moves kMoveVecs 16-byte vectors, so the index
// arithmetic is per workgroup and the loads of a thread are independent.
// Source and destination pools may be device memory or device-accessible
// pinned host memory.  Pairs naming a block outside either pool are skipped.
constexpr int kMoveVecs = 4;

__global__ __launch_bounds__(kThreads) void move_blocks_kernel(BlockMove m) {
    const int64_t bv = m.block_bytes / 16;           // vectors per block
    const uint32_t x = blockIdx.x;
    const uint32_t kv = x & 1u;
    const uint32_t pl = x >> 1;                       // pair * layers + layer
    const uint32_t i = pl / (uint32_t)m.layers;
    const uint32_t layer = pl - i * (uint32_t)m.layers;
    const int32_t src = m.pairs[2 * i], dst = m.pairs[2 * i + 1];
    if (src < 0 || src >= m.src_blocks || dst < 0 || dst >= m.dst_blocks) return;
    const vec4 *from = reinterpret_cast<const vec4 *>(kv ? m.src_v[layer] : m.src_k[layer]) +
                       (int64_t)src * bv;
    vec4 *to = reinterpret_cast<vec4 *>(kv ? m.dst_v[layer] : m.dst_k[layer]) + (int64_t)dst * bv;
    const int64_t w0 = (int64_t)blockIdx.y * (kThreads * kMoveVecs) + threadIdx.x;
    vec4 r[kMoveVecs];
#pragma unroll
    for (int u = 0; u < kMoveVecs; ++u) {
        const int64_t w = w0 + u * kThreads;
        if (w < bv) r[u] = from[w];
    }
#pragma unroll
    for (int u = 0; u < kMoveVecs; ++u) {
        const int64_t w = w0 + u * kThreads;
        if (w < bv) to[w] = r[u];
    }
}

int launch_move_blocks(const BlockMove &m, int32_t n, void *stream) {
    const int64_t bv = m.block_bytes / 16;
    const int64_t chunks = (bv + kThreads * kMoveVecs - 1) / (kThreads * kMoveVecs);
    const int64_t gx = (int64_t)n * m.layers * 2;
    (void)hipGetLastError();  // an error left by other code is not this launch's
    hipLaunchKernelGGL(move_blocks_kernel, dim3((unsigned)gx, (unsigned)chunks), dim3(kThreads), 0,
                       (hipStream_t)stream, m);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- static scratch

// The split-K workspace of pa_decode_no_alloc: a fixed device array in place
// of a caller-provided buffer, for callers that cannot allocate.  Every
// device the library runs on holds its own copy at its own address until the
// process ends.  In host code the name is only a stand-in for the symbol:
// the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

int scratch_address(void **ptr) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
        if (e != hipSuccess) return (int)e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return 0;
}

const char *hip_error_name(int err) { return hipGetErrorName((hipError_t)err); }

const char *kernel_build_info() {
    return "gfx950; decode: 4 or 8 wave64 per workgroup (chosen per launch from occupancy), "
           "16-token wave steps, non-temporal K/V loads, LDS block table, longest-first order up "
           "to 256 sequences, G in 1..8 (1..16 for 16-bit types, on matrix cores from G 2), "
           "D in {64,128}, fp32/fp16/bf16, token- or head-major blocks; prefill: matrix cores, "
           "fp16/bf16; cache_write / copy_blocks: 16-byte vectors";
}

}  // namespace pa
