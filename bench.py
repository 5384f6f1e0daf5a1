"""Benchmark: paged decode attention at the OPT-13B layer shape on one MI355X.

One step = the decode iteration's hot path over one batch, in one launch
(pa_decode_append): each sequence's newest token is stored in its slot and
the whole batch attends (64 sequences, 40/40 heads, head_dim 128, fp16,
16-token blocks, lognormal context lengths, blocks scattered by a seeded
permutation).  The same step as two launches (pa_cache_write, then
pa_decode) is timed too and reported beside it.  The
batch's copy-on-write list is empty at this shape (no forks), so no
copy_blocks launch is part of the step; copy_blocks is timed on its own on
the parallel-sampling workload and reported beside the step.

value = attended KV tokens / s (sum of context lengths per step / step time).
Inputs are resident in HBM before the timed region; R replicas of the KV
pool are cycled so that no step finds its K/V in the 256 MB last-level cache.

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_opt13b_f16_counters.json")
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_pa_amd", "csrc", "pa_kernels.hip")


# How the committed profile summaries are made (run from the repository root;
# OUT is any scratch directory for the raw rocprofv3 output).
PROFILE_COMMANDS = [
    "rocprofv3 --kernel-trace --stats -f csv -d OUT/prof_trace -o trace -- "
    "python3 bench.py --steps 30 --warmup 5 --no-extras",
    "rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/prof_fetch -o fetch -- "
    "python3 bench.py --counters-run --steps 5 > OUT/prof_fetch.log",
    "rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/prof_write -o write -- "
    "python3 bench.py --counters-run --steps 5 > OUT/prof_write.log",
    "python3 bench.py --summarize-profiles OUT/prof_trace OUT/prof_fetch OUT/prof_write profiles",
]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The decode kernels' source: everything in pa_kernels.hip before its prefill
# section (element types, decode kernels, merge, launcher).
DECODE_SECTION_END = b"// ---------------------------------------------------------------- prefill"


def kernel_hash() -> str:
    """Hash of the decode kernels' source, which the committed counter
    summary was taken with: changes to other kernels in the same file (prefill,
    cache_write, copies) leave it, and the traffic figure, valid."""
    with open(KERNEL_SRC, "rb") as f:
        src = f.read()
    i = src.find(DECODE_SECTION_END)
    if i < 0:
        raise RuntimeError(f"{KERNEL_SRC}: prefill section marker not found")
    return hashlib.sha256(src[:i]).hexdigest()[:16]


def decode_bytes(lens, hq, hkv, d, e, block):
    """Algorithmic bytes of one decode launch: valid K and V rows, q and out,
    the block-table entries used, the context lengths."""
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(lens.sum()) * hkv * d * 2 * e
    qo = 2 * len(lens) * hq * d * e
    table = 4 * int(((lens + block - 1) // block).sum())
    return kv + qo + table + 4 * len(lens)


def unique_decode_bytes(tables, lens, hq, hkv, d, e, block):
    """Algorithmic bytes of one decode launch counting each physical block
    once: a block shared by several sequences (copy-on-write sharing) is
    stored once in HBM, so its valid rows are read from HBM at most once;
    its valid rows are the most any sharer uses.  q, out, table and lengths
    as in decode_bytes."""
    tables = np.asarray(tables)
    lens = np.asarray(lens, dtype=np.int64)
    rows = {}
    for s, n in enumerate(lens):
        for j in range(int(-(-n // block))):
            b = int(tables[s, j])
            rows[b] = max(rows.get(b, 0), int(min(block, n - j * block)))
    kv = sum(rows.values()) * hkv * d * 2 * e
    qo = 2 * len(lens) * hq * d * e
    table = 4 * int(((lens + block - 1) // block).sum())
    return kv + qo + table + 4 * len(lens)


def time_events(fn, iters, stream):
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for i in range(iters):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e-3 for a, b in evs]


def replicas_for(nbytes, floor=2, target=1 << 30, cap=64):
    """Copies of a working set so that consecutive launches never find their
    data in the 256 MB last-level cache: at least ``floor``, enough to pass
    ``target`` bytes in all."""
    return int(min(cap, max(floor, -(-target // max(1, nbytes)))))


def paged_dense_ratio(points, rounds=15, warm=3):
    """Config 3: paged vs dense decode on identical values, in both layouts
    (token-major: the pool is the dense buffer cut into blocks; head-major:
    both transposed to [.., Hkv, tokens, D]).  paged_us / dense_us: R
    launches over R replicas captured in a HIP graph, replayed between one
    event pair (median over rounds), which measures the GPU also where a
    launch is shorter than the host's per-call cost.  eager_*: the same R
    launches issued from Python (host-bound for the small points)."""
    import torch

    import paged_kv_cache_pa_amd as pa
    import workloads as W

    res = {}
    st = torch.cuda.current_stream()
    for batch, ctx in points:
        d = W.config3_device(batch, ctx)
        out = torch.empty_like(d["q"])
        nbytes = batch * ctx * 40 * 128 * 2 * 2
        R = replicas_for(nbytes)
        for layout in ("NHD", "HND"):
            if layout == "HND":  # same values, head-major
                for key in ("k_cache", "v_cache", "k_dense", "v_dense"):
                    d[key] = d[key].transpose(1, 2).contiguous()
            pk = [(d["k_cache"], d["v_cache"])] + [(d["k_cache"].clone(), d["v_cache"].clone())
                                                   for _ in range(R - 1)]
            dk = [(d["k_dense"], d["v_dense"])] + [(d["k_dense"].clone(), d["v_dense"].clone())
                                                   for _ in range(R - 1)]

            def paged(i):
                k, v = pk[i % R]
                pa.pa_decode(d["q"], k, v, d["block_tables"], d["context_lens"], d["scale"], out,
                             max_context_len=ctx, layout=layout)

            def dense(i):
                k, v = dk[i % R]
                pa.pa_decode_dense(d["q"], k, v, d["context_lens"], d["scale"], out,
                                   max_context_len=ctx, layout=layout)

            for i in range(warm * R):
                paged(i)
                dense(i)
            tp, td = [], []
            for _ in range(rounds):
                tp.append(time_group(paged, R, st))
                td.append(time_group(dense, R, st))
            ep, ed = float(np.median(tp)), float(np.median(td))
            mp = time_graph(paged, R, rounds, st)
            md = time_graph(dense, R, rounds, st)
            res[f"{layout} {batch}x{ctx}"] = {
                "paged_us": round(mp * 1e6, 2), "dense_us": round(md * 1e6, 2),
                "ratio": round(mp / md, 4), "paged_GB_s": round(nbytes / mp / 1e9, 1),
                "replicas": R, "eager_paged_us": round(ep * 1e6, 2),
                "eager_dense_us": round(ed * 1e6, 2)}
            del pk, dk
        del d, out
        torch.cuda.empty_cache()
    return res


SETTLE_SCALE = 1.0  # --settle: 0 times each leg from a cold start (counter passes)


def settle(run_once, seconds):
    """Repeat run_once() (GPU work, synchronized after each call) for
    ``seconds`` of wall time before a leg is timed, so that the GPU runs at
    the clock it holds under sustained load: started cold, prefill read 524 /
    648 TFLOP/s where the same launches read 587-592 / 729-740 after 0.1 s
    or more of work."""
    import torch

    run_once()  # at least once: the first launches also page in code and data
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds * SETTLE_SCALE:
        run_once()
        torch.cuda.synchronize()


def time_group(fn, n, stream):
    """Average seconds per call of n back-to-back calls between one event pair."""
    import torch

    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) * 1e-3 / n


def time_graph(fn, n, rounds, stream, min_calls=16):
    """Median seconds per call of fn(0) .. fn(m-1) (m = n rounded up to at
    least ``min_calls``; callers cycle their n replicas by i % n) captured
    once into a HIP graph and replayed ``rounds`` times, each replay between
    one event pair on ``stream``.  A short launch costs the host more (Python
    binding and runtime, ~12 us) than the GPU; a replay launches all m
    kernels without host work in between, so this measures the GPU, and m
    calls per event pair keep the events' own cost out of a short call's
    time."""
    import torch

    m = n * -(-min_calls // n)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(n):  # first calls outside the capture
            fn(i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(m):
            fn(i)
    torch.cuda.synchronize()
    settle(g.replay, 0.05)
    ts = []
    for _ in range(rounds):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3 / m)
    del g
    return float(np.median(ts))


def copy_blocks_rate(rounds=15):
    """pa_copy_blocks on the parallel-sampling workload (80 block pairs), over
    pool replicas so the copied blocks are not served from cache."""
    import torch

    import paged_kv_cache_pa_amd as pa
    import workloads as W

    sc = W.config4(poison=False)
    p = sc.paged
    k0 = torch.from_numpy(p.k_cache).cuda()
    v0 = torch.from_numpy(p.v_cache).cuda()
    R = replicas_for(2 * k0.numel() * k0.element_size())
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
    pairs = torch.from_numpy(p.block_pairs).cuda()
    st = torch.cuda.current_stream()

    def f(i):
        k, v = pools[i % R]
        pa.pa_copy_blocks(k, v, pairs)

    for i in range(R):
        f(i)
    te = float(np.median([time_group(f, R, st) for _ in range(rounds)]))
    t = time_graph(f, R, rounds, st)
    n = p.block_pairs.shape[0]
    nbytes = 2 * 2 * n * 16 * 40 * 128 * 2 + 8 * n
    return {"pairs": int(n), "us": round(t * 1e6, 2), "GB_s": round(nbytes / t / 1e9, 1),
            "replicas": R, "timing": "HIP graph of at least 16 launches over the R replicas, replayed",
            "eager_us": round(te * 1e6, 2)}


def stream_lib():
    """The benchmark's bandwidth reference kernels (libpa_stream.so, built
    beside libpa.so from csrc/stream_ref.hip; not part of the library)."""
    import ctypes

    from paged_kv_cache_pa_amd.build import STREAM_LIB_PATH

    if not os.path.exists(STREAM_LIB_PATH):
        raise RuntimeError(f"{STREAM_LIB_PATH} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(STREAM_LIB_PATH)
    P, SZ, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.pa_ref_stream_read.argtypes = [P, SZ, I, I, ctypes.c_uint32, P, P]
    L.pa_ref_stream_copy.argtypes = [P, P, SZ, I, P]
    L.pa_ref_stream_read.restype = I
    L.pa_ref_stream_copy.restype = I
    L.pa_ref_threads.restype = I
    return L


# (access order, workgroups) of the read reference: 0 = a contiguous chunk per
# workgroup, 1 = grid-stride
STREAM_READ_SHAPES = [(0, w) for w in (256, 1024, 4096, 8192, 16384)] + \
    [(1, w) for w in (256, 512, 1024, 2048, 4096)]
STREAM_COPY_GRIDS = (1024, 4096, 8192, 16384)


def stream_reference(nbytes, replicas=4, rounds=10):
    """What a kernel that only moves the bytes reaches on this GPU: a plain
    streaming read of ``nbytes`` (the decode launch's algorithmic bytes) and a
    plain copy of ``nbytes`` / 2 each way, with the decode kernels' 16-byte
    non-temporal loads.  ``replicas`` buffers are cycled so that no launch
    finds its data in the last-level cache.  Every access order and grid
    size in STREAM_READ_SHAPES / STREAM_COPY_GRIDS is timed (4R back-to-back
    launches between one event pair, median over rounds); the best is the
    reference."""
    import ctypes

    import torch

    L = stream_lib()
    st = torch.cuda.current_stream()
    sth = ctypes.c_void_p(st.cuda_stream)
    n = -(-nbytes // 16) * 16
    bufs = [torch.empty(n // 8, dtype=torch.int64, device="cuda").random_() for _ in range(replicas)]
    sink = torch.zeros(L.pa_ref_threads() * 4, dtype=torch.int32, device="cuda")
    key = int(np.random.default_rng(7).integers(1, 2**32 - 1))
    half = -(-(n // 2) // 16) * 16
    dsts = [torch.empty(half // 8, dtype=torch.int64, device="cuda") for _ in range(replicas)]

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: hipError {rc}")

    def timed(f, moved):
        settle(lambda: [f(i) for i in range(4 * replicas)], 0.05)
        t = float(np.median([time_group(f, 4 * replicas, st) for _ in range(rounds)]))
        return round(moved / t / 1e9, 1)

    read, copy = {}, {}
    for order, wg in STREAM_READ_SHAPES:
        def f_read(i, wg=wg, order=order):
            check(L.pa_ref_stream_read(ctypes.c_void_p(bufs[i % replicas].data_ptr()), n, wg,
                                       order, key, ctypes.c_void_p(sink.data_ptr()), sth),
                  "stream read")

        read[("chunk " if order == 0 else "stride ") + str(wg)] = timed(f_read, n)
    for wg in STREAM_COPY_GRIDS:
        def f_copy(i, wg=wg):
            check(L.pa_ref_stream_copy(ctypes.c_void_p(dsts[i % replicas].data_ptr()),
                                       ctypes.c_void_p(bufs[i % replicas].data_ptr()), half, wg,
                                       sth), "stream copy")

        copy[wg] = timed(f_copy, 2 * half)
    del bufs, dsts
    torch.cuda.empty_cache()
    return {"read_GB_s": max(read.values()), "copy_GB_s": max(copy.values()),
            "read_bytes": n, "copy_bytes_moved": 2 * half, "replicas": replicas,
            "read_by_workgroups": read, "copy_by_workgroups": copy,
            "what": "plain streaming read / copy kernels (csrc/stream_ref.hip): 16-byte "
                    "non-temporal loads, a contiguous chunk per workgroup (512 threads) or "
                    "grid-stride (256 threads); best access order and grid size"}


def copy_layers_rate(rounds=10, layers=40):
    """pa_copy_blocks_layers: the 80 copy-on-write pairs of the
    parallel-sampling workload applied to every one of OPT-13B's 40 layers in
    one launch.  The pairs' blocks are renumbered into a compact pool per layer
    (2 x 160 blocks x 160 KiB x 40 layers = 2 GiB, past the last-level cache)."""
    import torch

    import paged_kv_cache_pa_amd as pa
    import workloads as W

    pairs = W.config4(poison=False).paged.block_pairs
    ids, inv = np.unique(pairs, return_inverse=True)
    compact = inv.reshape(pairs.shape).astype(np.int32)
    nb, B, H, D = len(ids), 16, 40, 128
    ks = [torch.empty((nb, H, B, D), dtype=torch.float16, device="cuda") for _ in range(layers)]
    vs = [torch.empty_like(k) for k in ks]
    for t in ks + vs:
        t.normal_()
    bp = torch.from_numpy(compact).cuda()
    st = torch.cuda.current_stream()

    def f(i):
        pa.pa_copy_blocks_layers(ks, vs, bp, layout="HND")

    f(0)
    t = float(np.median([time_group(f, 1, st) for _ in range(rounds)]))
    n = compact.shape[0]
    nbytes = 2 * 2 * n * layers * B * H * D * 2 + 8 * n
    del ks, vs
    torch.cuda.empty_cache()
    return {"pairs": int(n), "layers": layers, "us": round(t * 1e6, 1),
            "GB_s": round(nbytes / t / 1e9, 1), "launches": -(-layers // 64)}


def write_layers_rate(rounds=10, layers=40, tokens=64):
    """pa_cache_write_layers: one decode iteration's new rows (64 sequences)
    for all 40 layers of OPT-13B in one launch, against 40 pa_cache_write
    launches; both timed as HIP-graph replays (GPU time).  Pools of 256
    blocks per layer (head-major), distinct random slots."""
    import torch

    import paged_kv_cache_pa_amd as pa

    nb, B, H, D = 256, 16, 40, 128
    g = torch.Generator(device="cuda").manual_seed(808)
    ks = [torch.empty((nb, H, B, D), dtype=torch.float16, device="cuda") for _ in range(layers)]
    vs = [torch.empty_like(k) for k in ks]
    kn = [torch.randn((tokens, H, D), generator=g, device="cuda").half() for _ in range(layers)]
    vn = [torch.randn((tokens, H, D), generator=g, device="cuda").half() for _ in range(layers)]
    slots = torch.from_numpy(np.random.default_rng(9).permutation(nb * B)[:tokens]
                             .astype(np.int32)).cuda()
    st = torch.cuda.current_stream()

    def one(i):
        pa.pa_cache_write_layers(kn, vn, ks, vs, slots, layout="HND")

    def per_layer(i):
        for layer in range(layers):
            pa.pa_cache_write(kn[layer], vn[layer], ks[layer], vs[layer], slots, layout="HND")

    t1 = time_graph(one, 1, rounds, st)
    tn = time_graph(per_layer, 1, rounds, st)
    nbytes = 2 * 2 * tokens * H * D * 2 * layers + 4 * tokens
    del ks, vs, kn, vn
    torch.cuda.empty_cache()
    return {"tokens": tokens, "layers": layers, "one_launch_us": round(t1 * 1e6, 1),
            "one_launch_GB_s": round(nbytes / t1 / 1e9, 1),
            "per_layer_launches_us": round(tn * 1e6, 1)}


def swap_rate(rounds=5, mib=64):
    """Swapping between HBM and pinned host memory at block sizes 16 / 64 /
    256 tokens (OPT-13B layer geometry, 40 heads x 128 dims fp16): one
    pa_swap_blocks launch for all blocks, against one asynchronous copy per
    K / V block (torch copy_, a hipMemcpyAsync each) for the same blocks.
    ``mib`` MiB of K+V move each way."""
    import torch

    import paged_kv_cache_pa_amd as pa

    res = {}
    rng = np.random.default_rng(7)
    st = torch.cuda.current_stream()
    for B in (16, 64, 256):
        blk = B * 40 * 128 * 2
        n = max(1, (mib << 20) // (2 * blk))
        gk = torch.randn((2 * n, 40, B, 128), dtype=torch.float16, device="cuda")
        gv = torch.randn_like(gk)
        hk = torch.empty((n, 40, B, 128), dtype=torch.float16, pin_memory=True)
        hv = torch.empty_like(hk, pin_memory=True)
        g_ids = rng.permutation(2 * n)[:n]
        out_pairs = torch.from_numpy(np.stack([g_ids, np.arange(n)], 1).astype(np.int32)).cuda()
        in_pairs = torch.from_numpy(np.stack([np.arange(n), g_ids], 1).astype(np.int32)).cuda()

        def k_out(i):
            pa.pa_swap_blocks([hk], [hv], [gk], [gv], out_pairs, layout="HND")

        def k_in(i):
            pa.pa_swap_blocks([gk], [gv], [hk], [hv], in_pairs, layout="HND")

        def c_out(i):
            for j, g in enumerate(g_ids):
                hk[j].copy_(gk[g], non_blocking=True)
                hv[j].copy_(gv[g], non_blocking=True)

        def c_in(i):
            for j, g in enumerate(g_ids):
                gk[g].copy_(hk[j], non_blocking=True)
                gv[g].copy_(hv[j], non_blocking=True)

        row = {"blocks": int(n), "block_KiB": blk // 1024}
        nbytes = 2 * n * blk
        for name, fn in (("kernel_out", k_out), ("kernel_in", k_in), ("per_block_out", c_out),
                         ("per_block_in", c_in)):
            fn(0)
            t = float(np.median([time_group(fn, 1, st) for _ in range(rounds)]))
            row[name + "_GB_s"] = round(nbytes / t / 1e9, 1)
        res[f"B{B}"] = row
        del gk, gv, hk, hv
        torch.cuda.empty_cache()
    return res


def block_manager_rate(steps=400):
    """Host cost of the block manager for one decode iteration of the
    OPT-13B-shape batch: reserve one slot for each of the 64 sequences, then
    export the block tables and lengths pa_decode reads.  Host-only; median
    microseconds per iteration, through the Python binding and as the bare
    C calls on preallocated buffers."""
    import ctypes
    import time as _t

    import workloads as W
    from paged_kv_cache_pa_amd.block_manager import BlockManager

    lens, _ = W.config2_lens()
    B, mbs = 16, 256
    nb = int(sum(-(-int(n) // B) for n in lens)) + 64 * (2 * steps // B + 2)
    bm = BlockManager(nb, 0, B)
    seqs = [bm.new_seq() for _ in lens]
    bm.reserve(seqs, [int(n) for n in lens])
    ones = [1] * len(seqs)
    py = []
    for _ in range(steps):
        t0 = _t.perf_counter()
        bm.reserve(seqs, ones)
        bm.tables(seqs, mbs)
        py.append(_t.perf_counter() - t0)
    L = bm._L
    S = len(seqs)
    s_arr = (ctypes.c_int32 * S)(*seqs)
    k_arr = (ctypes.c_int32 * S)(*ones)
    slots = (ctypes.c_int32 * S)()
    pairs = (ctypes.c_int32 * (2 * S))()
    tables = (ctypes.c_int32 * (S * mbs))()
    cl = (ctypes.c_int32 * S)()
    npairs = ctypes.c_int32()
    native = []
    for _ in range(steps):
        t0 = _t.perf_counter()
        rc = L.pa_bm_reserve(bm._h, s_arr, k_arr, S, slots, S, pairs, S, ctypes.byref(npairs))
        rc |= L.pa_bm_tables(bm._h, s_arr, S, tables, mbs, cl)
        native.append(_t.perf_counter() - t0)
        if rc:
            raise RuntimeError(f"block manager call failed: {rc}")
    bm.close()
    return {"seqs": S, "binding_us": round(float(np.median(py)) * 1e6, 1),
            "native_us": round(float(np.median(native)) * 1e6, 2),
            "what": "median per decode iteration: reserve(64 x 1 token) + tables export"}


def _dev_pool(a, layout):
    import torch

    a = np.ascontiguousarray(np.swapaxes(a, 1, 2)) if layout == "HND" else a
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _dev(a):
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


PREFILL_POINTS = (
    # (label, dtype, seqs, context, chunk, Hq, Hkv)
    ("OPT-13B prompt 8 x 1024", "f16", 8, 1024, 1024, 40, 40),
    ("GQA chunk 512 after 3584 (4 seqs)", "bf16", 4, 4096, 512, 32, 8),
)


def prefill_flops(ctx, chunk, seqs, hq, d):
    """Multiply-adds of the causal product, 2 flops each, for QK^T and PV:
    each chunk row at position p sees p + 1 keys."""
    pos = np.arange(ctx - chunk, ctx, dtype=np.int64)
    return int(4 * d * hq * seqs * int((pos + 1).sum()))


def prefill_rate(rounds=10, d=128):
    """pa_prefill on the points above (head-major pools, block size 16, two
    pool replicas): median over ``rounds`` groups of 8 back-to-back launches
    of the time per launch, and achieved TFLOP/s against the dense 16-bit
    matrix-core peak."""
    import torch

    import paged_kv_cache_pa_amd as pa

    res = {}
    st = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(707)
    for label, dt, S, ctx, chunk, hq, hkv in PREFILL_POINTS:
        tdt = torch.float16 if dt == "f16" else torch.bfloat16
        B = 16
        nbs = ctx // B
        nb = S * nbs
        R = 2
        pools = [(torch.randn((nb, hkv, B, d), generator=g, device="cuda").to(tdt),
                  torch.randn((nb, hkv, B, d), generator=g, device="cuda").to(tdt))
                 for _ in range(R)]
        table = torch.from_numpy(np.random.default_rng(7).permutation(nb).reshape(S, nbs)
                                 .astype(np.int32)).cuda()
        cl = torch.full((S,), ctx, dtype=torch.int32, device="cuda")
        qs = torch.arange(0, (S + 1) * chunk, chunk, dtype=torch.int32, device="cuda")
        q = torch.randn((S * chunk, hq, d), generator=g, device="cuda").to(tdt)
        out = torch.empty_like(q)

        def f(i):
            k, v = pools[i % R]
            pa.pa_prefill(q, k, v, table, cl, qs, 1.0 / np.sqrt(d), out, max_query_len=chunk,
                          max_context_len=ctx, layout="HND")

        settle(lambda: [f(i) for i in range(4 * R)], 0.25)
        # 4 R launches back to back per event pair (the replicas cycled), so
        # the events' own cost and the gaps between groups stay small
        t = float(np.median([time_group(f, 4 * R, st) for _ in range(rounds)]))
        fl = prefill_flops(ctx, chunk, S, hq, d)
        res[label] = {"us": round(t * 1e6, 1), "TFLOP_s": round(fl / t / 1e12, 1),
                      "frac_of_2500": round(fl / t / 2.5e15, 4), "flops": fl}
        del pools
        torch.cuda.empty_cache()
    return res


def config_rates(rounds=10, only=None):
    """pa_decode on the other workloads, head-major pools over replicas,
    timed as HIP-graph replays (the GPU's time, also for short launches):
    the tiny fp32 batch, the parallel-sampling beams (96 sequences sharing
    prompt blocks; bytes counted per sequence as the kernel reads them) and
    the grouped-query long-context batch with 512-token split-K (decode and
    merge launches together).  ``only``: time just the workloads whose label
    starts with it."""
    import torch

    import paged_kv_cache_pa_amd as pa
    import workloads as W

    st = torch.cuda.current_stream()
    res = {}
    for label, make, ps in (("tiny fp32 (4 seqs, 8/8 heads, D 64)", lambda: W.config1(poison=False), 0),
                            ("beams fp16 (96 seqs, 40/40 heads)", lambda: W.config4(poison=False).paged, 0),
                            ("GQA bf16 (8 seqs to 16384, 12/2 heads, split 512)", W.config5, 512)):
        if only is not None and not label.startswith(only):
            continue
        p = make()
        S, Hq, D = p.q.shape
        k0, v0 = _dev_pool(p.k_cache, "HND"), _dev_pool(p.v_cache, "HND")
        R = replicas_for(2 * k0.numel() * k0.element_size())
        pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
        q, bt, cl = _dev(p.q), _dev(p.block_tables), _dev(p.context_lens)
        out = torch.empty_like(q)
        mcl = int(p.context_lens.max())
        params = pa.DecodeParams(S, Hq, p.num_kv_heads, D, p.block_size, p.max_blocks_per_seq,
                                 p.num_blocks, mcl, ps, {"f32": 0, "f16": 1, "bf16": 2}[p.dtype],
                                 pa.LAYOUTS["HND"])
        ws = torch.empty(max(1, pa.pa_decode_workspace_size(params) // 4), dtype=torch.float32,
                         device="cuda")

        def f(i):
            k, v = pools[i % R]
            pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=mcl, partition_size=ps,
                         workspace=ws, layout="HND")

        for i in range(2 * R):
            f(i)
        t = time_graph(f, R, rounds, st)
        b = decode_bytes(p.context_lens, Hq, p.num_kv_heads, D, W.ELEM_BYTES[p.dtype], p.block_size)
        u = unique_decode_bytes(p.block_tables, p.context_lens, Hq, p.num_kv_heads, D,
                                W.ELEM_BYTES[p.dtype], p.block_size)
        r = {"us": round(t * 1e6, 2), "kv_tokens_per_s": round(float(p.context_lens.sum()) / t, 1),
             "replicas": R}
        if u == b:
            r.update({"algorithmic_bytes": b, "GB_s": round(b / t / 1e9, 1),
                      "frac_of_8000": round(b / t / 8e12, 4)})
        else:  # blocks shared between sequences: HBM holds (and must read) each once
            r.update({"unique_bytes": u, "GB_s": round(u / t / 1e9, 1),
                      "frac_of_8000": round(u / t / 8e12, 4),
                      "logical_bytes": b, "logical_GB_s": round(b / t / 1e9, 1),
                      "bytes": "GB_s and frac_of_8000 on unique bytes (each physical block "
                               "once); logical = every sequence's rows as it reads them"})
        res[label] = r
        del pools, k0, v0
        torch.cuda.empty_cache()
    # The beams again through pa_decode_shared: each prompt's 32 shared blocks
    # read once per group of 6 beams (split 256: the prompt is partitions 0
    # and 1), and pa_decode with the same split for comparison.
    label = "beams fp16, shared-prefix decode (16 groups x 6 beams, split 256)"
    if only is None or label.startswith(only):
        sc = W.config4(poison=False)
        p = sc.paged
        S, Hq, D = p.q.shape
        gs, gsh = W.config4_groups(sc)
        k0, v0 = _dev_pool(p.k_cache, "HND"), _dev_pool(p.v_cache, "HND")
        R = replicas_for(2 * k0.numel() * k0.element_size())
        pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
        q, bt, cl = _dev(p.q), _dev(p.block_tables), _dev(p.context_lens)
        gs_d, gsh_d = _dev(gs), _dev(gsh)
        out = torch.empty_like(q)
        mcl = int(p.context_lens.max())
        ps = 256
        params = pa.DecodeParams(S, Hq, p.num_kv_heads, D, p.block_size, p.max_blocks_per_seq,
                                 p.num_blocks, mcl, ps, 1, pa.LAYOUTS["HND"])
        ws = torch.empty(max(1, pa.pa_decode_shared_workspace_size(params) // 4),
                         dtype=torch.float32, device="cuda")

        def fs(i):
            k, v = pools[i % R]
            pa.pa_decode_shared(q, k, v, bt, cl, gs_d, gsh_d, p.scale, out,
                                max_shared_blocks=int(gsh.max()), max_context_len=mcl,
                                partition_size=ps, workspace=ws, layout="HND")

        def fp(i):
            k, v = pools[i % R]
            pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=mcl, partition_size=ps,
                         workspace=ws, layout="HND")

        for i in range(2 * R):
            fs(i)
            fp(i)
        t = time_graph(fs, R, rounds, st)
        t_plain = time_graph(fp, R, rounds, st)
        b = decode_bytes(p.context_lens, Hq, p.num_kv_heads, D, W.ELEM_BYTES[p.dtype], p.block_size)
        u = unique_decode_bytes(p.block_tables, p.context_lens, Hq, p.num_kv_heads, D,
                                W.ELEM_BYTES[p.dtype], p.block_size)
        res[label] = {"us": round(t * 1e6, 2),
                      "kv_tokens_per_s": round(float(p.context_lens.sum()) / t, 1),
                      "replicas": R, "unique_bytes": u, "GB_s": round(u / t / 1e9, 1),
                      "frac_of_8000": round(u / t / 8e12, 4), "logical_bytes": b,
                      "pa_decode_same_split_us": round(t_plain * 1e6, 2),
                      "launches": "grouped prefix pass + per-sequence pass + merge",
                      "bytes": "GB_s and frac_of_8000 on unique bytes (each physical block once)"}
        del pools, k0, v0
        torch.cuda.empty_cache()
    return res


BLOCK_SWEEP_SIZES = (1, 2, 4, 8, 16, 32, 64, 128, 256)


def block_sweep(rounds=10, seqs=16, ctx=4096, hq=12, hkv=2, d=128, partition=256):
    """Decode time against block size, blocks in order and scattered, against
    the contiguous twin, on the shape of [Res] "Attention over scattered
    blocks" (16 sequences x 4096 cached tokens, 12 query / 2 kv heads, head
    dim 128, fp16: 64 MiB of K and V per step; head-major pools).  The
    identical values sit in every layout: the dense [S, Hkv, ctx, D] buffer
    is cut into blocks of B tokens, which are placed in order or by a seeded
    permutation.  Split into partitions of ``partition`` tokens so the
    16 x 2 (sequence, kv head) pairs fill the GPU.  One JSON line per point;
    times are per launch over rotating replicas (decode + merge)."""
    import torch

    import paged_kv_cache_pa_amd as pa

    st = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(606)
    per = seqs * hkv * ctx * d * 2 * 2  # K + V bytes
    R = replicas_for(per)
    dense = [(torch.randn((seqs, hkv, ctx, d), generator=g, device="cuda").half(),
              torch.randn((seqs, hkv, ctx, d), generator=g, device="cuda").half())
             for _ in range(R)]
    q = torch.randn((seqs, hq, d), generator=g, device="cuda").half()
    cl = torch.full((seqs,), ctx, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    scale = 1.0 / np.sqrt(d)
    nbytes = decode_bytes(np.full(seqs, ctx), hq, hkv, d, 2, 16) - 4 * seqs * ctx // 16

    def timed(f):
        for i in range(2 * R):
            f(i)
        return float(np.median([time_group(f, R, st) for _ in range(rounds)]))

    def f_dense(i):
        k, v = dense[i % R]
        pa.pa_decode_dense(q, k, v, cl, scale, out, max_context_len=ctx,
                           partition_size=partition, layout="HND")

    t_dense = timed(f_dense)
    print(json.dumps({"config": "block sweep", "block_size": None, "placement": "contiguous",
                      "us": round(t_dense * 1e6, 2), "GB_s": round(nbytes / t_dense / 1e9, 1),
                      "replicas": R}), flush=True)
    rng = np.random.default_rng(606)
    for B in BLOCK_SWEEP_SIZES:
        nb_seq = ctx // B
        nb = seqs * nb_seq
        for placement in ("in order", "scattered"):
            ids = np.arange(nb) if placement == "in order" else rng.permutation(nb)
            # block j of sequence s holds tokens [j B, (j + 1) B) of the dense buffer
            table = ids.reshape(seqs, nb_seq).astype(np.int32)
            bt = torch.from_numpy(table).cuda()
            inv = torch.from_numpy(np.argsort(ids)).cuda()  # pool slot -> (s, j) in order
            pools = []
            for k, v in dense:
                def blocks(x):
                    x = x.view(seqs, hkv, nb_seq, B, d).permute(0, 2, 1, 3, 4)
                    return x.reshape(nb, hkv, B, d)[inv].contiguous()
                pools.append((blocks(k), blocks(v)))

            def f_paged(i):
                k, v = pools[i % R]
                pa.pa_decode(q, k, v, bt, cl, scale, out, max_context_len=ctx,
                             partition_size=partition, layout="HND")

            t = timed(f_paged)
            print(json.dumps({"config": "block sweep", "block_size": B, "placement": placement,
                              "us": round(t * 1e6, 2), "vs_contiguous": round(t / t_dense, 3),
                              "GB_s": round(nbytes / t / 1e9, 1), "replicas": R}), flush=True)
            del pools
            torch.cuda.empty_cache()


def sweep(rounds=10):
    """Every configuration's kernels, timed as HIP-graph replays over rotating
    replicas (one JSON object per line; not the benchmark's contract line)."""
    import torch

    import paged_kv_cache_pa_amd as pa
    import workloads as W

    st = torch.cuda.current_stream()

    def emit(**kw):
        print(json.dumps(kw), flush=True)

    def time_decode(p, layout, ps, label, nbytes=None):
        S, Hq, D = p.q.shape
        e = W.ELEM_BYTES[p.dtype]
        k0, v0 = _dev_pool(p.k_cache, layout), _dev_pool(p.v_cache, layout)
        R = replicas_for(2 * k0.numel() * k0.element_size())
        pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
        q, bt, cl = _dev(p.q), _dev(p.block_tables), _dev(p.context_lens)
        out = torch.empty_like(q)
        mcl = int(p.context_lens.max())
        params = pa.DecodeParams(S, Hq, p.num_kv_heads, D, p.block_size, p.max_blocks_per_seq,
                                 p.num_blocks, mcl, ps, {"f32": 0, "f16": 1, "bf16": 2}[p.dtype],
                                 pa.LAYOUTS[layout])
        need = pa.pa_decode_workspace_size(params)
        ws = torch.empty(max(1, need // 4), dtype=torch.float32, device="cuda")

        def f(i):
            k, v = pools[i % R]
            pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=mcl, partition_size=ps,
                         workspace=ws, layout=layout)

        for i in range(2 * R):
            f(i)
        t = time_graph(f, R, rounds, st)
        b = nbytes or decode_bytes(p.context_lens, Hq, p.num_kv_heads, D, e, p.block_size)
        emit(config=label, kernel="pa_decode", layout=layout, partition=ps, us=round(t * 1e6, 2),
             algorithmic_bytes=b, GB_s=round(b / t / 1e9, 1), frac=round(b / t / 8e12, 4),
             kv_tokens_per_s=round(float(p.context_lens.sum()) / t, 1), replicas=R)
        del pools
        torch.cuda.empty_cache()

    def time_write(p, layout, label):
        k0, v0 = _dev_pool(p.k_cache, layout), _dev_pool(p.v_cache, layout)
        R = replicas_for(2 * k0.numel() * k0.element_size())
        pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
        kn, vn, sm = _dev(p.k_new), _dev(p.v_new), _dev(p.slot_mapping)

        def f(i):
            k, v = pools[i % R]
            pa.pa_cache_write(kn, vn, k, v, sm, layout=layout)

        for i in range(R):
            f(i)
        t = time_graph(f, R, rounds, st)
        N = p.slot_mapping.shape[0]
        b = 2 * 2 * N * p.num_kv_heads * p.head_dim * W.ELEM_BYTES[p.dtype] + 4 * N
        emit(config=label, kernel="pa_cache_write", layout=layout, tokens=N, us=round(t * 1e6, 2),
             algorithmic_bytes=b, GB_s=round(b / t / 1e9, 1))
        del pools
        torch.cuda.empty_cache()

    def time_copy(p, label):
        k0, v0 = _dev(p.k_cache), _dev(p.v_cache)
        R = replicas_for(2 * k0.numel() * k0.element_size())
        pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
        pairs = _dev(p.block_pairs)

        def f(i):
            k, v = pools[i % R]
            pa.pa_copy_blocks(k, v, pairs)

        for i in range(R):
            f(i)
        t = time_graph(f, R, rounds, st)
        n = p.block_pairs.shape[0]
        b = 2 * 2 * n * p.block_size * p.num_kv_heads * p.head_dim * W.ELEM_BYTES[p.dtype] + 8 * n
        emit(config=label, kernel="pa_copy_blocks", pairs=n, us=round(t * 1e6, 2),
             algorithmic_bytes=b, GB_s=round(b / t / 1e9, 1))
        del pools
        torch.cuda.empty_cache()

    c1 = W.config1(poison=False)
    for lay in ("NHD", "HND"):
        time_write(c1, lay, "c1")
        time_decode(c1, lay, 0, "c1")
    c2 = W.config2()
    for lay in ("HND", "NHD"):
        for ps in (0, 512):
            time_decode(c2, lay, ps, "c2")
    sc = W.config4(poison=False)
    time_copy(sc.paged, "c4")
    for lay in ("HND", "NHD"):
        time_write(sc.paged, lay, "c4")
        time_decode(sc.paged, lay, 0, "c4")
    c5 = W.config5()
    for lay in ("HND", "NHD"):
        for ps in (512, 256, 0):
            time_decode(c5, lay, ps, "c5 mixed")
    for n in W.CONFIG5_LENS:
        time_decode(W.config5(uniform_len=n), "HND", 512, f"c5 uniform {n}")
    for point, r in paged_dense_ratio(W.CONFIG3_POINTS, rounds=rounds).items():
        emit(config="c3 " + point, kernel="pa_decode vs pa_decode_dense", **r)


def cpu_baseline(p, budget_s=12.0, max_runs=200):
    """The fp64 oracle on the host cores, on the same batch: the whole batch,
    repeated for about ``budget_s`` seconds (at least 3 runs); median."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    times = []
    t_start = time.time()
    while len(times) < 3 or ((time.time() - t_start) < budget_s and len(times) < max_runs):
        t0 = time.perf_counter()
        oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale,
                      p.dtype, nthreads=threads)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    toks = int(p.context_lens.sum())
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(toks / t, 1), "unit": "KV tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole batch ({toks} KV tokens x 40 heads), fp64, {len(times)} runs, "
                      f"median {t:.3f} s; host {model or platform.processor()}"}


def counters_run(args):
    """A short run for rocprofv3 --pmc passes: a few decode launches of the
    benchmark workload, then pa_copy_blocks over a pool of known size, whose
    FETCH_SIZE / WRITE_SIZE calibrate the counters (bytes read = bytes
    written = half the pool, K and V)."""
    import torch

    import paged_kv_cache_pa_amd as pa
    import workloads as W

    p = W.config2(poison=False)
    S, Hq, D = p.q.shape
    NB, B, Hkv, _ = p.k_cache.shape
    dev = torch.device("cuda:0")
    lay = args.layout
    pool = (lambda a: np.ascontiguousarray(np.swapaxes(a, 1, 2))) if lay == "HND" else (lambda a: a)
    k = torch.from_numpy(pool(p.k_cache)).to(dev)
    v = torch.from_numpy(pool(p.v_cache)).to(dev)
    q = torch.from_numpy(p.q).to(dev)
    out = torch.empty_like(q)
    bt = torch.from_numpy(p.block_tables).to(dev)
    cl = torch.from_numpy(p.context_lens).to(dev)
    rng = np.random.default_rng(2020)
    k_new = torch.from_numpy(W.randn(rng, (S, Hkv, D), "f16")).to(dev)
    v_new = torch.from_numpy(W.randn(rng, (S, Hkv, D), "f16")).to(dev)
    for _ in range(args.steps):
        pa.pa_decode_append(q, k_new, v_new, k, v, bt, cl, p.scale, out,
                            max_context_len=int(p.context_lens.max()), layout=lay)
    torch.cuda.synchronize()
    nbc = 4096  # calibration pool: 4096 blocks of 160 KiB per tensor
    kc = torch.zeros((nbc, 16, 40, 128), dtype=torch.float16, device=dev)
    vc = torch.zeros_like(kc)
    half = nbc // 2
    pairs = torch.tensor([[i, half + i] for i in range(half)], dtype=torch.int32, device=dev)
    for _ in range(3):
        pa.pa_copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    blk = 16 * 40 * 128 * 2
    print(json.dumps({"decode_launches": args.steps,
                      "decode_algorithmic_bytes": decode_bytes(p.context_lens, Hq, Hkv, D, 2, B)
                      + 2 * S * Hkv * D * 2,
                      "copy_launches": 3, "copy_read_bytes": 2 * half * blk,
                      "copy_write_bytes": 2 * half * blk, "kernel_sha256_16": kernel_hash()}),
          flush=True)


DECODE_KERNEL_PREFIX = "_ZN2pa13decode_kernelIDF16_Li128ELi1ELi1E"  # fp16, D 128, G 1, paged B>=16
COPY_KERNEL_PREFIX = "pa::move_blocks_kernel"


def _rows(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def summarize_profiles(trace_dir, fetch_dir, write_dir, out_dir, commands):
    """Turn rocprofv3 CSV output into the committed summaries: the kernel
    trace statistics (markdown) and the calibrated HBM traffic per decode
    launch (json, read back by the benchmark)."""
    import re

    stats = _rows(_find(trace_dir, "_kernel_stats.csv"))
    fetch = _rows(_find(fetch_dir, "_counter_collection.csv"))
    write = _rows(_find(write_dir, "_counter_collection.csv"))
    meta = None
    log = os.path.join(os.path.dirname(fetch_dir.rstrip("/")), os.path.basename(fetch_dir.rstrip("/")) + ".log")
    with open(log) as f:
        for ln in f:
            if ln.startswith("{") and "kernel_sha256_16" in ln:
                meta = json.loads(ln)
    if meta is None:
        raise RuntimeError(f"no counters-run record in {log}")

    def per_dispatch(rows, prefix):
        v = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].startswith(prefix)]
        return float(np.mean(v)), len(v)

    f_dec, nf = per_dispatch(fetch, DECODE_KERNEL_PREFIX)
    w_dec, nw = per_dispatch(write, DECODE_KERNEL_PREFIX)
    f_cpy, _ = per_dispatch(fetch, COPY_KERNEL_PREFIX)
    w_cpy, _ = per_dispatch(write, COPY_KERNEL_PREFIX)
    kib = 1024.0
    f_scale = meta["copy_read_bytes"] / (f_cpy * kib)
    w_scale = meta["copy_write_bytes"] / (w_cpy * kib)
    hbm = f_dec * kib * f_scale + w_dec * kib * w_scale
    counters = {
        "workload": "OPT-13B-shape decode, fp16, 64 seqs, 40/40 heads, D 128, B 16, head-major pool",
        "kernel": DECODE_KERNEL_PREFIX + "...",
        "kernel_sha256_16": meta["kernel_sha256_16"],
        "fetch_kib_per_dispatch": round(f_dec, 3), "write_kib_per_dispatch": round(w_dec, 3),
        "dispatches": [nf, nw],
        "calibration": {"kernel": "pa::move_blocks_kernel (pa_copy_blocks, a plain block copy)",
                        "read_bytes": meta["copy_read_bytes"], "write_bytes": meta["copy_write_bytes"],
                        "fetch_kib": round(f_cpy, 3), "write_kib": round(w_cpy, 3),
                        "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5)},
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_bytes_per_launch": meta["decode_algorithmic_bytes"],
        "traffic_over_algorithmic": round(hbm / meta["decode_algorithmic_bytes"], 4),
        "commands": commands[1:],
    }
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "decode_opt13b_f16_counters.json"), "w") as f:
        json.dump(counters, f, indent=1)
    lines = ["# Kernel trace: OPT-13B-shape decode step (fp16, head-major pool; "
             "pa_decode_append: newest token stored, then attention, one launch)", "",
             "Command (from the repository root, on one MI355X; OUT is a scratch directory for the raw output):", "", "```",
             commands[0], "```", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"]
        short = re.sub(r"\(.*", "", name)[:70]
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    dec = [r for r in stats if r["Name"].startswith(DECODE_KERNEL_PREFIX)][0]
    avg = float(dec["AverageNs"]) * 1e-9
    lines += ["", "Algorithmic bytes = K/V rows read + queries read + outputs written + the "
              "newest K/V rows read and stored.",
              "", f"Decode kernel: {meta['decode_algorithmic_bytes']} algorithmic bytes per launch / "
              f"{avg * 1e6:.2f} us = {meta['decode_algorithmic_bytes'] / avg / 1e9:.0f} GB/s "
              f"({meta['decode_algorithmic_bytes'] / avg / 8e12 * 100:.1f}% of 8 TB/s).",
              f"HBM traffic per launch from the counter passes: {hbm / 1e6:.1f} MB "
              f"({hbm / meta['decode_algorithmic_bytes']:.4f} x algorithmic); see "
              "decode_opt13b_f16_counters.json.", ""]
    with open(os.path.join(out_dir, "decode_opt13b_f16_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(counters, indent=1))


def traffic_from_counters(launch_bytes):
    """HBM bytes per decode launch from the committed rocprofv3 counter runs,
    or None if the kernel source changed since they were taken."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_sha256_16") != kernel_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 500 untimed steps (~43 ms): after 20 the timed region read ~1.5% slower
    # than after 500 or 2000, the GPU still settling into sustained load
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--settle", type=float, default=1.0,
                    help="scale of the time each leg runs before it is timed (0: none; for "
                         "counter passes, which profile every launch)")
    ap.add_argument("--partition", type=int, default=0,
                    help="split-K partition size for pa_decode (0 = none)")
    ap.add_argument("--replicas", type=int, default=4,
                    help="KV pool replicas cycled by consecutive steps (>= 2 defeats the LLC)")
    ap.add_argument("--layout", choices=("NHD", "HND"), default="HND",
                    help="KV pool layout: token-major or head-major blocks")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense ratio, copy_blocks and CPU legs (for profiling runs)")
    ap.add_argument("--counters-run", action="store_true",
                    help="short run for rocprofv3 --pmc passes (decode launches + calibration copy)")
    ap.add_argument("--prefill", action="store_true",
                    help="time pa_prefill (chunked prompt attention) only; one JSON line")
    ap.add_argument("--gqa", action="store_true",
                    help="time pa_decode on the grouped-query long-context batch only (split 512, "
                         "decode + merge); one JSON line")
    ap.add_argument("--beams", action="store_true",
                    help="time pa_decode and pa_decode_shared on the beams batch only; one JSON line")
    ap.add_argument("--block-sweep", action="store_true",
                    help="decode time against block size (1..256), in order / scattered / "
                         "contiguous, on a 16 x 4096-token GQA batch; one JSON line per point")
    ap.add_argument("--sweep", action="store_true",
                    help="time every configuration's kernels (JSON lines, not the contract line)")
    ap.add_argument("--summarize-profiles", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "OUT_DIR"),
                    help="write profile summaries from rocprofv3 CSV output (no GPU needed)")
    args = ap.parse_args()
    global SETTLE_SCALE
    SETTLE_SCALE = max(0.0, args.settle)
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, commands=PROFILE_COMMANDS)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decode path has no "
              "cross-GPU step at this scope.", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_pa_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pa.lib()  # fail loudly if the HIP library is missing
    if args.counters_run:
        counters_run(args)
        return
    if args.sweep:
        sweep()
        return
    if args.block_sweep:
        block_sweep()
        return
    if args.prefill:
        print(json.dumps(prefill_rate()), flush=True)
        return
    if args.gqa:
        print(json.dumps(config_rates(only="GQA")), flush=True)
        return
    if args.beams:
        print(json.dumps(config_rates(only="beams")), flush=True)
        return
    dev = torch.device("cuda:0")
    t_gen = time.time()
    p = W.config2(poison=False)
    S, Hq, D = p.q.shape
    NB, B, Hkv, _ = p.k_cache.shape
    lens = p.context_lens
    log(f"config2 generated in {time.time() - t_gen:.1f} s: S={S} sum_n={int(lens.sum())} NB={NB}")
    rng = np.random.default_rng(2020)
    k_new = torch.from_numpy(W.randn(rng, (S, Hkv, D), "f16")).to(dev)
    v_new = torch.from_numpy(W.randn(rng, (S, Hkv, D), "f16")).to(dev)
    slots = torch.from_numpy(np.array([W.slots_of(p.block_tables[s], [lens[s] - 1], B)[0]
                                       for s in range(S)], np.int32)).to(dev)
    q = torch.from_numpy(p.q).to(dev)
    bt = torch.from_numpy(p.block_tables).to(dev)
    cl = torch.from_numpy(lens).to(dev)
    if args.layout == "HND":  # same values, head-major blocks [NB, Hkv, B, D]
        kc0 = torch.from_numpy(np.ascontiguousarray(np.swapaxes(p.k_cache, 1, 2))).to(dev)
        vc0 = torch.from_numpy(np.ascontiguousarray(np.swapaxes(p.v_cache, 1, 2))).to(dev)
    else:
        kc0 = torch.from_numpy(p.k_cache).to(dev)
        vc0 = torch.from_numpy(p.v_cache).to(dev)
    R = max(1, args.replicas)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(R - 1)]
    out = torch.empty_like(q)
    mcl = int(lens.max())
    ws_bytes = pa.pa_decode_workspace_size(pa.DecodeParams(S, Hq, Hkv, D, B, p.max_blocks_per_seq,
                                                           NB, mcl, args.partition, 1,
                                                           pa.LAYOUTS[args.layout]))
    ws = torch.empty(max(1, ws_bytes // 4), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def run(count, timed):
        """count steps back to back; step i is one pa_decode_append launch on
        pool replica i % R (each sequence's new token written to its slot,
        then attention over the batch).  With timed, one HIP event pair on the
        launch stream brackets all of them: nothing but the launches runs
        between the events, so (e1 - e0) / count is the average launch time.
        Returns the event pair."""
        e0 = e1 = None
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        for i in range(count):
            k, v = pools[i % R]
            pa.pa_decode_append(q, k_new, v_new, k, v, bt, cl, p.scale, out,
                                max_context_len=mcl, partition_size=args.partition,
                                workspace=ws, layout=args.layout)
        if timed:
            e1.record(stream)
        return e0, e1

    def run_two_launch(count):
        """The same step as two launches (pa_cache_write, then pa_decode):
        wall seconds per step."""
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(count):
            k, v = pools[i % R]
            pa.pa_cache_write(k_new, v_new, k, v, slots, layout=args.layout)
            pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=mcl,
                         partition_size=args.partition, workspace=ws, layout=args.layout)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / count

    run(args.warmup, False)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    t0 = time.perf_counter()
    e0, e1 = run(args.steps, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_avg = e0.elapsed_time(e1) * 1e-3 / args.steps
    log(f"timed {args.steps} steps: {wall / args.steps * 1e3:.4f} ms/step, "
        f"decode avg {dec_avg * 1e6:.2f} us per launch")
    # (left out of --no-extras runs, so that a kernel trace of one holds only
    # the fused launches)
    two_launch = None if args.no_extras else run_two_launch(max(args.steps, 10))
    # Spread: the timed region repeated after the measurement (not part of
    # value), one event pair per repeat.
    spread = None
    if not args.no_extras:
        per = []
        for _ in range(10):
            a0, a1 = run(args.steps, True)
            torch.cuda.synchronize()
            per.append(a0.elapsed_time(a1) * 1e3 / args.steps)
        spread = {"repeats": len(per), "steps_each": args.steps,
                  "launch_us_median": round(float(np.median(per)), 3),
                  "launch_us_p10": round(float(np.percentile(per, 10)), 3),
                  "launch_us_p90": round(float(np.percentile(per, 90)), 3),
                  "what": "the timed region repeated after the measurement; average launch "
                          "time of each repeat (HIP events on the launch stream)"}

    # The same step on a pool in the other layout (token-major when the
    # measured one is head-major), timed the same way: reported beside the
    # line, not part of value.
    other_layout = None
    if not args.no_extras:
        lay2 = "NHD" if args.layout == "HND" else "HND"
        if lay2 == "HND":
            kc2 = torch.from_numpy(np.ascontiguousarray(np.swapaxes(p.k_cache, 1, 2))).to(dev)
            vc2 = torch.from_numpy(np.ascontiguousarray(np.swapaxes(p.v_cache, 1, 2))).to(dev)
        else:
            kc2 = torch.from_numpy(p.k_cache).to(dev)
            vc2 = torch.from_numpy(p.v_cache).to(dev)
        pools2 = [(kc2, vc2)] + [(kc2.clone(), vc2.clone()) for _ in range(R - 1)]

        def run2(count):
            for i in range(count):
                k, v = pools2[i % R]
                pa.pa_decode_append(q, k_new, v_new, k, v, bt, cl, p.scale, out,
                                    max_context_len=mcl, partition_size=args.partition,
                                    workspace=ws, layout=lay2)

        run2(args.warmup)
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        run2(args.steps)
        b1.record(stream)
        torch.cuda.synchronize()
        us2 = b0.elapsed_time(b1) * 1e3 / args.steps
        del pools2, kc2, vc2
        torch.cuda.empty_cache()
        other_layout = {"layout": lay2, "kv_layout": "[NB, B, Hkv, D]" if lay2 == "NHD" else "[NB, Hkv, B, D]",
                        "avg_launch_us": round(us2, 3)}
        log(f"other layout {lay2}: {us2:.2f} us per launch")

    toks = int(lens.sum())
    value = toks * args.steps / wall
    # attention's reads plus the newest rows written into their slots
    launch_bytes = decode_bytes(lens, Hq, Hkv, D, 2, B) + 2 * S * Hkv * D * 2
    achieved = launch_bytes / dec_avg / 1e9
    traffic = traffic_from_counters(launch_bytes)
    result = {
        "metric": "paged decode attention: KV tokens/s + achieved HBM GB/s (% of peak), OPT-13B shape",
        "value": round(value, 1),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "OPT-13B-shape single-layer decode step (each sequence's new token "
                        "written to its slot + paged decode, one launch), fp16",
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
            "block_size": B, "sum_context_lens": toks, "max_context_len": mcl,
            "num_blocks": NB, "partition_size": args.partition, "kv_pool_replicas": R,
            "kv_layout": "[NB, Hkv, B, D]" if args.layout == "HND" else "[NB, B, Hkv, D]",
            "seed": 202,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_kernel<_Float16,128,1,kPagedWide>" + (" + merge_kernel" if args.partition else ""),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": launch_bytes,
            "avg_launch_us": round(dec_avg * 1e6, 3),
            "timing": "one HIP event pair around all timed launches (back to back) on the launch stream",
        },
        "two_launch_ms_per_step": None if two_launch is None else round(two_launch * 1e3, 5),
        "launch_spread": spread,
    }
    if other_layout is not None:
        gbs2 = launch_bytes / (other_layout["avg_launch_us"] * 1e-6) / 1e9
        other_layout["GB_s"] = round(gbs2, 1)
        other_layout["frac_of_8000"] = round(gbs2 / HBM_PEAK_GBS, 4)
        other_layout["what"] = ("the same decode step (same values, same algorithmic bytes) on a pool "
                                "in the other block layout, one HIP event pair around the launches")
        result["other_layout"] = other_layout
    if not args.no_extras:
        try:
            ref = stream_reference(launch_bytes)
            result["stream_reference"] = ref
            result["roofline"]["stream_read_GB_s"] = ref["read_GB_s"]
            result["roofline"]["frac_of_stream_read"] = round(achieved / ref["read_GB_s"], 4)
        except Exception as e:  # report, do not lose the main line
            result["stream_reference"] = {"error": repr(e)}
        log("stream reference done")
        try:
            result["other_workloads"] = config_rates()
        except Exception as e:  # report, do not lose the main line
            result["other_workloads"] = {"error": repr(e)}
        log("other workloads done")
        try:
            result["paged_vs_dense"] = paged_dense_ratio(W.CONFIG3_POINTS)
        except Exception as e:  # report, do not hide the main result
            result["paged_vs_dense"] = {"error": repr(e)}
        log("paged/dense done")
        try:
            result["copy_blocks"] = copy_blocks_rate()
        except Exception as e:
            result["copy_blocks"] = {"error": repr(e)}
        log("copy_blocks done")
        for key, fn in (("copy_blocks_layers", copy_layers_rate),
                        ("cache_write_layers", write_layers_rate), ("swap", swap_rate),
                        ("block_manager", block_manager_rate), ("prefill", prefill_rate)):
            try:
                result[key] = fn()
            except Exception as e:
                result[key] = {"error": repr(e)}
            log(f"{key} done")
        result["cpu_baseline"] = cpu_baseline(p)
        log("cpu baseline done")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
