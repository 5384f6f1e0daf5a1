// pa_kernels.hip -- gfx950 (CDNA4) kernels for paged decode attention,
// cache_write and copy_blocks.
//
// Pages cited (by title, then section / equation / figure):
//   [Kwon] "Efficient Memory Management for Large Language Model Serving with
//          PagedAttention" (paper summary page)
//   [Int]  "vLLM Internals: PagedAttention, Continuous Batching, and Where the
//          2-4x Comes From"
//   [Res]  "Paged Attention: Managing the KV Cache Like Virtual Memory"
//
// Decode design (one workgroup of 4 wave64 per (sequence, kv head,
// partition)):
//  * A token row of one kv head is D * e bytes (256 B for fp16/bf16 D=128
//    and fp32 D=64).  LPR = D*e/16 lanes read it with one 16-byte load each,
//    so one wave load instruction covers R = 64/LPR whole rows and every
//    byte fetched is used.  A wave step is 16 consecutive tokens (U = 16/R
//    loads of K and U of V); the four waves take steps round robin and
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
//    four waves through LDS at the end.  This is the one-pass form of the
//    [Kwon] §3.4 two-pass softmax; both equal the defining equation in exact
//    arithmetic.  The reduction order depends only on logical token order,
//    never on where blocks sit, so paged and dense results are bitwise equal
//    and invariant to block placement.
//  * Scheduling: for batches of up to 256 sequences every workgroup ranks the
//    sequences by context length (longest first, ties by index) and takes
//    the sequence whose rank matches its grid position, so the longest
//    sequences start first and the tail of the launch is short.  Which
//    workgroup computes a row never changes its arithmetic.
//  * Split-K: partition p covers tokens [p*PS, (p+1)*PS) and writes its
//    unnormalised partial (acc, m, l) to the workspace; a merge kernel then
//    combines the partitions by the log-sum-exp identity ([Int] "The kernel
//    pays for the indirection": a grid dimension over partitions; [Res]:
//    slices and a merge kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_launch.h"

namespace pa {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef uint32_t vec4 __attribute__((ext_vector_type(4)));  // 16 bytes

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
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
    int32_t S, Hq, Hkv, NB, MBS, log2B, max_ctx, PS, P;
    int32_t rank;       // 1: longest-first sequence order (S <= kRankMaxSeqs)
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

template <typename T, int D, int G, int MODE>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    using E = Elem<T>;
    constexpr int EPL = E::kEPL;
    constexpr int LPR = D / EPL;               // lanes per token row
    constexpr int R = 64 / LPR;                // rows per wave load
    constexpr int U = kStepTokens / R;         // loads per step (K and V each)
    constexpr int RED = kWaves * G * (D + 2);  // cross-wave merge floats
    constexpr int SMEM = RED > kTableChunk ? RED : kTableChunk;
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row must be 128, 256 or 512 bytes");
    static_assert(U * R == kStepTokens, "step shape");

    __shared__ float smem[SMEM];
    __shared__ int32_t s_len[kRankMaxSeqs];
    __shared__ int32_t s_pick;
    int32_t *s_tab = reinterpret_cast<int32_t *>(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int rg = lane / LPR;   // row group
    const int c = lane % LPR;    // 16-byte chunk of the row
    const int h = blockIdx.x % a.Hkv;
    const int part = blockIdx.y;

    int s, n;
    if (a.rank) {
        // Longest-first: rank(t) = #{u : n_u > n_t} + #{u < t : n_u == n_t};
        // this workgroup serves the sequence of rank blockIdx.x / Hkv.
        for (int t = tid; t < a.S; t += kThreads) {
            const int x = a.lens[t];
            s_len[t] = x < 0 ? 0 : (x > a.max_ctx ? a.max_ctx : x);
        }
        __syncthreads();
        const int want = blockIdx.x / a.Hkv;
        for (int t = tid; t < a.S; t += kThreads) {
            const int nt = s_len[t];
            int r = 0;
            for (int u = 0; u < a.S; ++u) {
                const int nu = s_len[u];
                r += (nu > nt) | ((nu == nt) & (u < t));
            }
            if (r == want) s_pick = t;
        }
        __syncthreads();
        s = s_pick;
        n = s_len[s];
    } else {
        s = blockIdx.x / a.Hkv;
        n = a.lens[s];
        n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
    }
    const int tb = a.PS ? part * a.PS : 0;
    const int te = a.PS ? min(n, tb + a.PS) : n;
    const int64_t qrow0 = (int64_t)s * a.Hq + (int64_t)h * G;  // first query head of the group

    if (tb >= te) {
        // Only an empty sequence reaches here with part == 0: its row is zero.
        if (part == 0)
            for (int i = tid; i < G * D; i += kThreads) E::store(a.out, qrow0 * D + i, 0.0f);
        return;
    }

    // q for the G heads of the group: this lane's 16-byte chunk, unscaled.
    vec4 qv[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        qv[g] = load_cached(a.q + ((qrow0 + g) * D + (int64_t)c * EPL) * sizeof(T));

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
    const uint32_t chunk_off = (uint32_t)(c * EPL * (int)sizeof(T));
    uint32_t voff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) voff[u] = (uint32_t)(u * R + rg) * tok_bytes + chunk_off;
    const int B = 1 << a.log2B;
    const int32_t *trow = MODE == kDense ? nullptr : a.tables + (int64_t)s * a.MBS;
    // Base of kv head h (and, dense, of sequence s).
    const int64_t head0 = (int64_t)h * a.head_bytes + (MODE == kDense ? (int64_t)s * a.seq_bytes : 0);
    const char *kh = a.k + head0;
    const char *vh = a.v + head0;

    const int nblk = (te - tb + B - 1) >> a.log2B;
    const int chunk_blocks = MODE == kDense ? nblk : kTableChunk;

    for (int cb = 0; cb < nblk; cb += chunk_blocks) {
        const int cn = min(chunk_blocks, nblk - cb);
        const int ctb = tb + cb * B;                 // first token of this chunk
        const int cte = min(te, ctb + cn * B);       // one past its last token
        if constexpr (MODE != kDense) {
            __syncthreads();  // the previous chunk's readers are done
            const int b0 = (tb >> a.log2B) + cb;
            for (int i = tid; i < cn; i += kThreads) {
                int32_t b = trow[b0 + i];
                s_tab[i] = b < 0 ? 0 : (b >= a.NB ? a.NB - 1 : b);
            }
            __syncthreads();
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

        // Full steps: wave w takes steps w, w + 4, ...  The next step's loads
        // are always issued before the current step is computed, with no
        // conditional loads inside the loop, so exactly one step of loads is
        // outstanding while a step is computed.
        vec4 ka[U], va[U], kb2[U], vb2[U];
        int j = wave;
        if (j < nfull) {
            issue.template operator()<false>(ka, va, j);
            while (j + 2 * kWaves < nfull) {
                issue.template operator()<false>(kb2, vb2, j + kWaves);
                compute.template operator()<false>(ka, va, j);
                issue.template operator()<false>(ka, va, j + 2 * kWaves);
                compute.template operator()<false>(kb2, vb2, j + kWaves);
                j += 2 * kWaves;
            }
            if (j + kWaves < nfull) {
                issue.template operator()<false>(kb2, vb2, j + kWaves);
                compute.template operator()<false>(ka, va, j);
                compute.template operator()<false>(kb2, vb2, j + kWaves);
            } else {
                compute.template operator()<false>(ka, va, j);
            }
        }
        // The partly filled last step goes to the wave whose turn it is.
        if (tail && wave == nfull % kWaves) {
            issue.template operator()<true>(ka, va, nfull);
            compute.template operator()<true>(ka, va, nfull);
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
    // A sequence that fits one partition is finished here; the merge kernel
    // skips it.
    const bool direct = a.PS == 0 || n <= a.PS;
    for (int i = tid; i < G * D; i += kThreads) {
        const int g = i / D, d = i % D;
        float M = kNegBig;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red[(w * G + g) * (D + 2) + D]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float *r = red + (w * G + g) * (D + 2);
            const float cw = fexp2(r[D] - M);
            L = fmaf(r[D + 1], cw, L);
            A = fmaf(r[d], cw, A);
        }
        const int64_t qh = qrow0 + g;
        if (direct) {
            E::store(a.out, qh * D + d, A / L);
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

// Combines the partitions of one (sequence, query head): with M the largest
// partition max, out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
// Sequences that fit one partition were written by the decode kernel.
template <typename T, int D>
__global__ __launch_bounds__(D) void merge_kernel(const float *ws_acc, const float *ws_ml,
                                                  const int32_t *lens, void *out, int32_t Hq,
                                                  int32_t P, int32_t PS, int32_t max_ctx) {
    const int qh = blockIdx.x;  // s * Hq + h
    const int s = qh / Hq;
    const int d = threadIdx.x;
    int n = lens[s];
    n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
    const int np = (n + PS - 1) / PS;
    if (np <= 1) return;
    const float *ml = ws_ml + (int64_t)qh * P * 2;
    const float *ac = ws_acc + (int64_t)qh * P * D;
    float M = kNegBig;
    for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
    float L = 0.0f, A = 0.0f;
    for (int p = 0; p < np; ++p) {
        const float cw = fexp2(ml[2 * p] - M);
        L = fmaf(ml[2 * p + 1], cw, L);
        A = fmaf(ac[(int64_t)p * D + d], cw, A);
    }
    Elem<T>::store(out, (int64_t)qh * D + d, A / L);
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
    a.rank = (l.S > 1 && l.S <= kRankMaxSeqs) ? 1 : 0;
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
    dim3 grid((unsigned)((int64_t)l.S * l.Hkv), (unsigned)l.P, 1);
    if (l.dense)
        hipLaunchKernelGGL((decode_kernel<T, D, G, kDense>), grid, dim3(kThreads), 0, st, a);
    else if (l.B >= kStepTokens)
        hipLaunchKernelGGL((decode_kernel<T, D, G, kPagedWide>), grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((decode_kernel<T, D, G, kPagedNarrow>), grid, dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || l.PS == 0) return e;
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3((unsigned)((int64_t)l.S * l.Hq)), dim3(D), 0, st,
                       a.ws_acc, a.ws_ml, l.lens, l.out, l.Hq, l.P, l.PS, l.max_ctx);
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

// ---------------------------------------------------------------- cache_write

// One flat range of 16-byte vectors: token i's K rows, then its V rows, each
// [Hkv, D] in the source.  Vector w of token i belongs to kv head g = w / rv
// and goes to block slot / B, offset slot % B of that head in the pool
// layout given by the strides.  Out-of-range slots are skipped ([Kwon] §3.4
// "Kernel-Level Optimizations", item 1: one fused launch writes every new
// token to the block and slot the scheduler names).
__global__ __launch_bounds__(kThreads) void cache_write_kernel(
    const vec4 *__restrict__ k_new, const vec4 *__restrict__ v_new, char *__restrict__ k_cache,
    char *__restrict__ v_cache, const int32_t *__restrict__ slots, int64_t total, int64_t rv,
    int32_t hkv, int32_t log2B, int64_t num_slots, int64_t blk_bytes, int64_t tok_bytes,
    int64_t head_bytes) {
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

int launch_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       const int32_t *slots, int32_t n, int32_t num_blocks, int32_t block_size,
                       int32_t hkv, int64_t row_bytes, int32_t layout, void *stream) {
    const int64_t rv = row_bytes / 16;  // vectors per head row
    const int64_t total = (int64_t)n * 2 * hkv * rv;
    int log2B = 0;
    while ((1 << log2B) < block_size) ++log2B;
    const int64_t blk_bytes = row_bytes * hkv * block_size;
    const int64_t tok_bytes = layout == 0 ? row_bytes * hkv : row_bytes;
    const int64_t head_bytes = layout == 0 ? row_bytes : row_bytes * block_size;
    int64_t blocks = (total + kThreads * 4 - 1) / (kThreads * 4);
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, (const vec4 *)k_new, (const vec4 *)v_new,
                       (char *)k_cache, (char *)v_cache, slots, total, rv, hkv, log2B,
                       (int64_t)num_blocks * block_size, blk_bytes, tok_bytes, head_bytes);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------- copy_blocks

// Whole-block copies for every (src, dst) pair, K then V, in one launch
// ([Kwon] §3.4 "Kernel-Level Optimizations", item 3).  A block is one
// contiguous range in either pool layout.  Pairs naming a block outside
// [0, NB) are skipped.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    vec4 *__restrict__ k_cache, vec4 *__restrict__ v_cache, const int32_t *__restrict__ pairs,
    int64_t total, int64_t bv, int32_t num_blocks) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += stride) {
        const int64_t i = idx / (2 * bv);
        const int64_t rem = idx - i * 2 * bv;
        const bool is_v = rem >= bv;
        const int64_t w = is_v ? rem - bv : rem;
        const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
        vec4 *pool = is_v ? v_cache : k_cache;
        pool[(int64_t)dst * bv + w] = pool[(int64_t)src * bv + w];
    }
}

int launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int32_t n,
                       int32_t num_blocks, int64_t block_bytes, void *stream) {
    const int64_t bv = block_bytes / 16;
    const int64_t total = (int64_t)n * 2 * bv;
    int64_t blocks = (total + kThreads * 4 - 1) / (kThreads * 4);
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, (vec4 *)k_cache, (vec4 *)v_cache, pairs, total, bv,
                       num_blocks);
    return (int)hipGetLastError();
}

const char *hip_error_name(int err) { return hipGetErrorName((hipError_t)err); }

const char *kernel_build_info() {
    return "gfx950; decode: 256 threads (4 wave64), 16-token wave steps, non-temporal K/V loads, "
           "LDS block table, longest-first order up to 256 sequences, G in 1..8, D in {64,128}, "
           "fp32/fp16/bf16, token- or head-major blocks; cache_write / copy_blocks: 16-byte vectors";
}

}  // namespace pa
