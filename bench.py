"""Benchmark: paged decode attention at the OPT-13B layer shape on one MI355X.

One step = the decode iteration's hot path over one batch: pa_cache_write
of each sequence's newest token into its slot, then pa_decode over the whole
batch (64 sequences, 40/40 heads, head_dim 128, fp16, 16-token blocks,
lognormal context lengths, blocks scattered by a seeded permutation).  The
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def decode_bytes(lens, hq, hkv, d, e, block):
    """Algorithmic bytes of one decode launch: valid K and V rows, q and out,
    the block-table entries used, the context lengths."""
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(lens.sum()) * hkv * d * 2 * e
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


def paged_dense_ratio(points, iters=20, warm=5):
    """Config 3: paged vs dense decode on identical values, interleaved round
    by round, in both layouts (token-major: the pool is the dense buffer cut
    into blocks; head-major: both transposed to [.., Hkv, tokens, D])."""
    import torch

    import paged_kv_cache_pa_amd as pa
    import workloads as W

    res = {}
    st = torch.cuda.current_stream()
    for batch, ctx in points:
        d = W.config3_device(batch, ctx)
        out = torch.empty_like(d["q"])
        for layout in ("NHD", "HND"):
            if layout == "HND":  # same values, head-major
                for key in ("k_cache", "v_cache", "k_dense", "v_dense"):
                    d[key] = d[key].transpose(1, 2).contiguous()

            def paged(i):
                pa.pa_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                             d["context_lens"], d["scale"], out, max_context_len=ctx,
                             layout=layout)

            def dense(i):
                pa.pa_decode_dense(d["q"], d["k_dense"], d["v_dense"], d["context_lens"],
                                   d["scale"], out, max_context_len=ctx, layout=layout)

            for _ in range(warm):
                paged(0)
                dense(0)
            tp, td = [], []
            for _ in range(iters):
                tp += time_events(paged, 1, st)
                td += time_events(dense, 1, st)
            mp, md = float(np.median(tp)), float(np.median(td))
            nbytes = batch * ctx * 40 * 128 * 2 * 2
            res[f"{layout} {batch}x{ctx}"] = {
                "paged_us": round(mp * 1e6, 2), "dense_us": round(md * 1e6, 2),
                "ratio": round(mp / md, 4), "paged_GB_s": round(nbytes / mp / 1e9, 1)}
        del d, out
        torch.cuda.empty_cache()
    return res


def copy_blocks_rate(iters=20):
    """pa_copy_blocks on the parallel-sampling workload (80 block pairs)."""
    import torch

    import paged_kv_cache_pa_amd as pa
    import workloads as W

    sc = W.config4(poison=False)
    p = sc.paged
    k = torch.from_numpy(p.k_cache).cuda()
    v = torch.from_numpy(p.v_cache).cuda()
    pairs = torch.from_numpy(p.block_pairs).cuda()
    st = torch.cuda.current_stream()
    for _ in range(3):
        pa.pa_copy_blocks(k, v, pairs)
    t = float(np.median(time_events(lambda i: pa.pa_copy_blocks(k, v, pairs), iters, st)))
    nbytes = 2 * 2 * p.block_pairs.shape[0] * 16 * 40 * 128 * 2 + 8 * p.block_pairs.shape[0]
    return {"pairs": int(p.block_pairs.shape[0]), "us": round(t * 1e6, 2),
            "GB_s": round(nbytes / t / 1e9, 1)}


def cpu_baseline(p, budget_s=10.0, max_runs=40):
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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--partition", type=int, default=0,
                    help="split-K partition size for pa_decode (0 = none)")
    ap.add_argument("--replicas", type=int, default=2)
    ap.add_argument("--layout", choices=("NHD", "HND"), default="HND",
                    help="KV pool layout: token-major or head-major blocks")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense ratio, copy_blocks and CPU legs (for profiling runs)")
    args = ap.parse_args()
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
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    def step(i, timed=False):
        k, v = pools[i % R]
        pa.pa_cache_write(k_new, v_new, k, v, slots, layout=args.layout)
        if timed:
            ev[i][0].record(stream)
        pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=mcl,
                     partition_size=args.partition, workspace=ws, layout=args.layout)
        if timed:
            ev[i][1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, timed=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec = [a.elapsed_time(b) * 1e-3 for a, b in ev]
    dec_avg = float(np.mean(dec))
    log(f"timed {args.steps} steps: {wall / args.steps * 1e3:.4f} ms/step, "
        f"decode avg {dec_avg * 1e6:.2f} us (min {min(dec) * 1e6:.2f})")

    toks = int(lens.sum())
    value = toks * args.steps / wall
    launch_bytes = decode_bytes(lens, Hq, Hkv, D, 2, B)
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
            "workload": "OPT-13B-shape single-layer decode step (cache_write of each sequence's "
                        "new token + paged decode), fp16",
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
        },
    }
    if not args.no_extras:
        try:
            result["paged_vs_dense"] = paged_dense_ratio([(8, 256), (32, 1024), (128, 2048)])
        except Exception as e:  # report, do not hide the main result
            result["paged_vs_dense"] = {"error": repr(e)}
        log("paged/dense done")
        try:
            result["copy_blocks"] = copy_blocks_rate()
        except Exception as e:
            result["copy_blocks"] = {"error": repr(e)}
        log("copy_blocks done")
        result["cpu_baseline"] = cpu_baseline(p)
        log("cpu baseline done")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
