/*
 * oracle.c -- plain fp64 CPU oracle for paged decode attention and its two
 * companion indexing operations.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no source,
 * header, table or helper with the HIP library and includes nothing from it.
 *
 * Pages cited (title, then the section / equation / figure):
 *   [Kwon]   "Efficient Memory Management for Large Language Model Serving
 *            with PagedAttention" (paper summary page)
 *   [Int]    "vLLM Internals: PagedAttention, Continuous Batching, and Where
 *            the 2-4x Comes From"
 *   [Res]    "Paged Attention: Managing the KV Cache Like Virtual Memory"
 *
 * Everything is deliberately slow and direct: one (sequence, query head)
 * at a time, the sequence's logical blocks gathered into a contiguous fp64
 * buffer, then the textbook max-subtracted two-pass softmax.  OpenMP only
 * spreads independent (sequence, query head) units over host threads; it
 * does not change any arithmetic.
 *
 * Storage dtypes: 0 = fp32, 1 = fp16 (IEEE binary16), 2 = bf16.  Every
 * element is widened to double exactly before any arithmetic.
 *
 * Layouts: 0 = token-major blocks [NB, B, Hkv, D] (dense [S, Smax, Hkv, D]);
 * 1 = head-major blocks [NB, Hkv, B, D] (dense [S, Hkv, Smax, D]), the
 * [blocks, kv heads, 16 tokens, head dim] pool of [Res] "A paged KV cache,
 * in code".
 *
 * Return codes: 0 ok, -1 bad argument, -2 an index (block id, slot, table
 * entry) outside its range.  Nothing is written before the arguments are
 * checked.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* exact widening of the storage formats                               */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Normal: (-1)^s 2^(e-15) (1 + f/1024); subnormal: (-1)^s 2^-14 f/1024. */
double oracle_half_to_double(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);
    return s ? -v : v;
}

/* bf16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static size_t elem_bytes(int dtype) { return dtype == 0 ? 4 : 2; }

static double load(const void *base, size_t i, int dtype) {
    if (dtype == 0) return (double)((const float *)base)[i];
    uint16_t u = ((const uint16_t *)base)[i];
    return dtype == 1 ? oracle_half_to_double(u) : oracle_bf16_to_double(u);
}

/* ------------------------------------------------------------------ */
/* attention over one contiguous sequence                              */

/*
 * [Kwon] §3.4 "PagedAttention Algorithm", the per-token equation:
 *   a_j = exp(q.k_j / sqrt d) / sum_t exp(q.k_t / sqrt d),  o = sum_j a_j v_j.
 * The caller supplies the scale (1/sqrt d in the configurations).  The
 * maximum score is subtracted before exponentiating; that leaves every a_j
 * unchanged in exact arithmetic.  K and V are n x D, row-major, fp64.
 * If n == 0 the output is zero.  If ``a`` is non-null it receives a_0..a_{n-1}.
 */
static void attend(const double *qv, const double *K, const double *V, int n, int D,
                   double scale, double *o, double *a_out, double *x) {
    int t, d;
    for (d = 0; d < D; ++d) o[d] = 0.0;
    if (n <= 0) return;
    double m = -INFINITY;
    for (t = 0; t < n; ++t) {
        double dot = 0.0;
        for (d = 0; d < D; ++d) dot += qv[d] * K[(size_t)t * D + d];
        x[t] = scale * dot;
        if (x[t] > m) m = x[t];
    }
    double Z = 0.0;                         /* first pass: the denominator */
    for (t = 0; t < n; ++t) {
        x[t] = exp(x[t] - m);
        Z += x[t];
    }
    for (t = 0; t < n; ++t) {               /* second pass: the weighted sum */
        double a = x[t] / Z;
        if (a_out) a_out[t] = a;
        for (d = 0; d < D; ++d) o[d] += a * V[(size_t)t * D + d];
    }
}

static int check_shape(int S, int Hq, int Hkv, int D, int dtype) {
    if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return -1;
    if (Hq % Hkv) return -1;
    if (dtype < 0 || dtype > 2) return -1;
    return 0;
}

/* Element index of (block b, offset o, kv head g, dim 0) in a pool. */
static size_t pool_index(int layout, size_t b, size_t o, size_t g, int B, int Hkv, int D) {
    if (layout == 0) return ((b * B + o) * Hkv + g) * D;
    return ((b * Hkv + g) * B + o) * D;
}

/*
 * Gather: sequence s's token t lives at physical block
 * block_tables[s][t / B], offset t % B ([Int] "PagedAttention: page tables,
 * for KV", the resolve() address translation; [Kwon] §3.4 "KV Cache Manager:
 * Block Table Mapping").  Query head h reads kv head h / G, G = Hq / Hkv:
 * contiguous groups of query heads share one kv head ([Res] "Attention over
 * scattered blocks": the 6 query heads sharing one key/value row).
 */
static int gather_seq(const void *cache, const int32_t *row, int n, int B, int NB,
                      int Hkv, int D, int g, int dtype, int layout, double *dst) {
    for (int t = 0; t < n; ++t) {
        int32_t b = row[t / B];
        if (b < 0 || b >= NB) return -2;
        size_t base = pool_index(layout, (size_t)b, (size_t)(t % B), (size_t)g, B, Hkv, D);
        for (int d = 0; d < D; ++d) dst[(size_t)t * D + d] = load(cache, base + d, dtype);
    }
    return 0;
}

/*
 * Paged decode.  out[s][h][:] (fp64, [S, Hq, D]).  ``units``, if non-null,
 * lists n_units (s, h) pairs to compute; otherwise every pair is computed.
 * ``weights``, if non-null, is [S, Hq, wstride] and receives a_t.
 */
int oracle_decode(const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, const int32_t *context_lens, double scale,
                  int S, int Hq, int Hkv, int D, int B, int MBS, int NB, int dtype, int layout,
                  const int32_t *units, int n_units, double *out, double *weights,
                  int wstride, int nthreads) {
    if (check_shape(S, Hq, Hkv, D, dtype) || B <= 0 || MBS <= 0 || NB <= 0) return -1;
    if (layout != 0 && layout != 1) return -1;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return -1;
    for (int s = 0; s < S; ++s) {
        int n = context_lens[s];
        if (n < 0 || n > MBS * B) return -2;
        if (weights && n > wstride) return -1;
        for (int j = 0; j < (n + B - 1) / B; ++j) {
            int32_t b = block_tables[(size_t)s * MBS + j];
            if (b < 0 || b >= NB) return -2;
        }
    }
    int total = units ? n_units : S * Hq;
    for (int u = 0; units && u < n_units; ++u)
        if (units[2 * u] < 0 || units[2 * u] >= S || units[2 * u + 1] < 0 || units[2 * u + 1] >= Hq)
            return -1;
    int G = Hq / Hkv;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
#endif
    for (int u = 0; u < total; ++u) {
        int s = units ? units[2 * u] : u / Hq;
        int h = units ? units[2 * u + 1] : u % Hq;
        int n = context_lens[s];
        int g = h / G;
        size_t nn = n > 0 ? (size_t)n : 1;
        double *K = malloc(nn * D * sizeof(double));
        double *V = malloc(nn * D * sizeof(double));
        double *x = malloc(nn * sizeof(double));
        double *qv = malloc((size_t)D * sizeof(double));
        if (!K || !V || !x || !qv) {
            err = -1;
        } else {
            const int32_t *row = block_tables + (size_t)s * MBS;
            int e1 = gather_seq(k_cache, row, n, B, NB, Hkv, D, g, dtype, layout, K);
            int e2 = gather_seq(v_cache, row, n, B, NB, Hkv, D, g, dtype, layout, V);
            if (e1 || e2) {
                err = -2;
            } else {
                for (int d = 0; d < D; ++d) qv[d] = load(q, ((size_t)s * Hq + h) * D + d, dtype);
                attend(qv, K, V, n, D, scale, out + ((size_t)s * Hq + h) * D,
                       weights ? weights + ((size_t)s * Hq + h) * wstride : NULL, x);
            }
        }
        free(K); free(V); free(x); free(qv);
    }
    return err;
}

/*
 * Dense (contiguous) decode: k, v are [S, Smax, Hkv, D] (layout 0) or
 * [S, Hkv, Smax, D] (layout 1); token t of sequence s is row (s, t).  Same
 * attention as above, no table ([Res] "Attention over scattered blocks":
 * the contiguous cache addressed directly).
 */
int oracle_decode_dense(const void *q, const void *k, const void *v,
                        const int32_t *context_lens, double scale, int S, int Hq, int Hkv,
                        int D, int Smax, int dtype, int layout, const int32_t *units,
                        int n_units, double *out, int nthreads) {
    if (check_shape(S, Hq, Hkv, D, dtype) || Smax <= 0) return -1;
    if (layout != 0 && layout != 1) return -1;
    if (!q || !k || !v || !context_lens || !out) return -1;
    for (int s = 0; s < S; ++s)
        if (context_lens[s] < 0 || context_lens[s] > Smax) return -2;
    int total = units ? n_units : S * Hq;
    for (int u = 0; units && u < n_units; ++u)
        if (units[2 * u] < 0 || units[2 * u] >= S || units[2 * u + 1] < 0 || units[2 * u + 1] >= Hq)
            return -1;
    int G = Hq / Hkv;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
#endif
    for (int u = 0; u < total; ++u) {
        int s = units ? units[2 * u] : u / Hq;
        int h = units ? units[2 * u + 1] : u % Hq;
        int n = context_lens[s];
        int g = h / G;
        size_t nn = n > 0 ? (size_t)n : 1;
        double *K = malloc(nn * D * sizeof(double));
        double *V = malloc(nn * D * sizeof(double));
        double *x = malloc(nn * sizeof(double));
        double *qv = malloc((size_t)D * sizeof(double));
        if (!K || !V || !x || !qv) {
            err = -1;
        } else {
            for (int t = 0; t < n; ++t) {
                size_t base = layout == 0 ? (((size_t)s * Smax + t) * Hkv + g) * D
                                          : (((size_t)s * Hkv + g) * Smax + t) * D;
                for (int d = 0; d < D; ++d) {
                    K[(size_t)t * D + d] = load(k, base + d, dtype);
                    V[(size_t)t * D + d] = load(v, base + d, dtype);
                }
            }
            for (int d = 0; d < D; ++d) qv[d] = load(q, ((size_t)s * Hq + h) * D + d, dtype);
            attend(qv, K, V, n, D, scale, out + ((size_t)s * Hq + h) * D, NULL, x);
        }
        free(K); free(V); free(x); free(qv);
    }
    return err;
}

/*
 * Context split into partitions of P tokens, each reduced on its own, then
 * combined.  The pages name the split and a merge step ([Int] "The kernel
 * pays for the indirection": a grid dimension over partitions; [Res]
 * "Attention over scattered blocks": slices and a merge kernel) without
 * printing the merge; this is the log-sum-exp identity:
 *   per partition p:  m_p = max x,  l_p = sum exp(x - m_p),
 *                     A_p = sum exp(x - m_p) v
 *   M = max_p m_p,  out = sum_p A_p exp(m_p - M) / sum_p l_p exp(m_p - M).
 * Partitions holding no token are skipped.  fp64 throughout.
 */
int oracle_decode_split(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, const int32_t *context_lens,
                        double scale, int S, int Hq, int Hkv, int D, int B, int MBS, int NB,
                        int dtype, int layout, int P, double *out, int nthreads) {
    if (check_shape(S, Hq, Hkv, D, dtype) || B <= 0 || MBS <= 0 || NB <= 0 || P <= 0) return -1;
    if (layout != 0 && layout != 1) return -1;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return -1;
    for (int s = 0; s < S; ++s)
        if (context_lens[s] < 0 || context_lens[s] > MBS * B) return -2;
    int G = Hq / Hkv;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
#endif
    for (int u = 0; u < S * Hq; ++u) {
        int s = u / Hq, h = u % Hq, g = h / G;
        int n = context_lens[s];
        size_t nn = n > 0 ? (size_t)n : 1;
        double *K = malloc(nn * D * sizeof(double));
        double *V = malloc(nn * D * sizeof(double));
        double *qv = malloc((size_t)D * sizeof(double));
        double *acc = calloc((size_t)D, sizeof(double));
        double *A = malloc((size_t)D * sizeof(double));
        double *o = out + ((size_t)s * Hq + h) * D;
        if (!K || !V || !qv || !acc || !A) {
            err = -1;
            goto done;
        }
        const int32_t *row = block_tables + (size_t)s * MBS;
        if (gather_seq(k_cache, row, n, B, NB, Hkv, D, g, dtype, layout, K) ||
            gather_seq(v_cache, row, n, B, NB, Hkv, D, g, dtype, layout, V)) {
            err = -2;
            goto done;
        }
        for (int d = 0; d < D; ++d) qv[d] = load(q, ((size_t)s * Hq + h) * D + d, dtype);
        int nparts = (n + P - 1) / P;
        double M = -INFINITY, L = 0.0;
        for (int p = 0; p < nparts; ++p) {
            int t0 = p * P, t1 = (p + 1) * P < n ? (p + 1) * P : n;
            double mp = -INFINITY;
            for (int t = t0; t < t1; ++t) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += qv[d] * K[(size_t)t * D + d];
                if (scale * dot > mp) mp = scale * dot;
            }
            double lp = 0.0;
            for (int d = 0; d < D; ++d) A[d] = 0.0;
            for (int t = t0; t < t1; ++t) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += qv[d] * K[(size_t)t * D + d];
                double w = exp(scale * dot - mp);
                lp += w;
                for (int d = 0; d < D; ++d) A[d] += w * V[(size_t)t * D + d];
            }
            /* fold partition p into the running (M, L, acc) */
            double Mn = mp > M ? mp : M;
            double ca = (M == -INFINITY) ? 0.0 : exp(M - Mn);
            double cp = exp(mp - Mn);
            L = L * ca + lp * cp;
            for (int d = 0; d < D; ++d) acc[d] = acc[d] * ca + A[d] * cp;
            M = Mn;
        }
        for (int d = 0; d < D; ++d) o[d] = nparts ? acc[d] / L : 0.0;
    done:
        free(K); free(V); free(qv); free(acc); free(A);
    }
    return err;
}

/*
 * cache_write: for each new token i in order, if slot_mapping[i] >= 0, its
 * K and V rows ([Hkv, D] each) are copied byte for byte into block
 * slot / B, offset slot % B ([Kwon] §3.4 "Kernel-Level Optimizations", item
 * 1: the write goes to the physical block and slot the scheduler names;
 * [Res] "A paged KV cache, in code": the slot mapping).  A negative slot is
 * padding and is skipped.  Slots >= NB * B are an error (nothing written).
 * Each kv head's [D] row is placed at (block, offset, head) of the layout.
 */
int oracle_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       const int32_t *slot_mapping, int N, int NB, int B, int Hkv, int D,
                       int dtype, int layout) {
    if (N < 0 || NB <= 0 || B <= 0 || Hkv <= 0 || D <= 0 || dtype < 0 || dtype > 2) return -1;
    if (layout != 0 && layout != 1) return -1;
    if (N > 0 && (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)) return -1;
    for (int i = 0; i < N; ++i)
        if (slot_mapping[i] >= (int64_t)NB * B) return -2;
    size_t e = elem_bytes(dtype), row = (size_t)D * e;
    for (int i = 0; i < N; ++i) {
        int32_t slot = slot_mapping[i];
        if (slot < 0) continue;
        for (int g = 0; g < Hkv; ++g) {
            size_t dst = pool_index(layout, (size_t)(slot / B), (size_t)(slot % B), (size_t)g,
                                    B, Hkv, D) * e;
            size_t src = ((size_t)i * Hkv + g) * row;
            memcpy((char *)k_cache + dst, (const char *)k_new + src, row);
            memcpy((char *)v_cache + dst, (const char *)v_new + src, row);
        }
    }
    return 0;
}

/*
 * copy_blocks: for each (src, dst) pair in order, the whole K block and the
 * whole V block ([B, Hkv, D] each) are copied byte for byte ([Kwon] §3.4
 * "Memory Sharing ...": copy-on-write copies the entire contents of the old
 * block; "Kernel-Level Optimizations", item 3: a list of (source,
 * destination) pairs).
 */
int oracle_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int n_pairs,
                       int NB, int B, int Hkv, int D, int dtype) {
    if (n_pairs < 0 || NB <= 0 || B <= 0 || Hkv <= 0 || D <= 0 || dtype < 0 || dtype > 2) return -1;
    if (n_pairs > 0 && (!k_cache || !v_cache || !pairs)) return -1;
    for (int i = 0; i < 2 * n_pairs; ++i)
        if (pairs[i] < 0 || pairs[i] >= NB) return -2;
    size_t blk = (size_t)B * Hkv * D * elem_bytes(dtype);
    for (int i = 0; i < n_pairs; ++i) {
        size_t src = (size_t)pairs[2 * i] * blk, dst = (size_t)pairs[2 * i + 1] * blk;
        memmove((char *)k_cache + dst, (const char *)k_cache + src, blk);
        memmove((char *)v_cache + dst, (const char *)v_cache + src, blk);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* multi-token queries: a chunk of new tokens per sequence             */

/* Prefill / chunked prefill over the paged cache ([Kwon] §3.4: the prompt
 * phase computes attention for all prompt tokens at once, each token
 * attending to itself and the tokens before it; the paged kernel reads keys
 * and values through the block table).  Sequence s owns query rows
 * query_start[s] .. query_start[s+1]-1 (T_s rows), the LAST T_s of its
 * context_lens[s] cached tokens, whose keys and values are already in the
 * pool.  Row r of the chunk sits at position pos = n - T_s + r and attends
 * to cached tokens 0 .. pos (causal), with the same softmax as decode.
 * q, out: [total_rows, Hq, D]; out is fp64. */
int oracle_prefill(const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *block_tables, const int32_t *context_lens,
                   const int32_t *query_start, double scale, int S, int Hq, int Hkv, int D,
                   int B, int MBS, int NB, int total_rows, int dtype, int layout,
                   double *out, int nthreads) {
    if (check_shape(S, Hq, Hkv, D, dtype) || B <= 0 || MBS <= 0 || NB <= 0) return -1;
    if ((layout != 0 && layout != 1) || total_rows < 0) return -1;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
        return -1;
    if (query_start[0] != 0 || query_start[S] != total_rows) return -1;
    for (int s = 0; s < S; ++s) {
        int rows = query_start[s + 1] - query_start[s];
        int len = context_lens[s];
        if (rows < 0 || len < rows || len > MBS * B) return -1;
        for (int j = 0; j < (len + B - 1) / B; ++j) {
            int32_t id = block_tables[(size_t)s * MBS + j];
            if (id < 0 || id >= NB) return -2;
        }
    }
    const int group = Hq / Hkv;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(min : status)
#endif
    for (int unit = 0; unit < S * Hq; ++unit) {
        const int seq = unit / Hq, head = unit % Hq;
        const int kv = head / group;
        const int len = context_lens[seq];
        const int first = query_start[seq], rows = query_start[seq + 1] - first;
        if (rows == 0) continue;
        double *Kc = malloc((size_t)len * D * sizeof(double));
        double *Vc = malloc((size_t)len * D * sizeof(double));
        double *scratch = malloc((size_t)len * sizeof(double));
        double *qrow = malloc((size_t)D * sizeof(double));
        if (!Kc || !Vc || !scratch || !qrow) {
            status = -1;
        } else {
            const int32_t *trow = block_tables + (size_t)seq * MBS;
            if (gather_seq(k_cache, trow, len, B, NB, Hkv, D, kv, dtype, layout, Kc) ||
                gather_seq(v_cache, trow, len, B, NB, Hkv, D, kv, dtype, layout, Vc)) {
                status = -2;
            } else {
                for (int r = 0; r < rows; ++r) {
                    const size_t at = ((size_t)(first + r) * Hq + head) * D;
                    const int pos = len - rows + r;   /* this row's position */
                    for (int d = 0; d < D; ++d) qrow[d] = load(q, at + d, dtype);
                    attend(qrow, Kc, Vc, pos + 1, D, scale, out + at, NULL, scratch);
                }
            }
        }
        free(Kc); free(Vc); free(scratch); free(qrow);
    }
    return status;
}
