"""Split-K decode: partitions of the context as a grid dimension, each
leaving an unnormalised partial in the workspace, and a merge by the
log-sum-exp identity ([Int] "The kernel pays for the indirection"; [Res]
"Attention over scattered blocks": slices and a merge).  Against the fp64
oracle on the cases that exercise the merge's paths (more partitions than
one pass stages, head groups of 1 to 16, head dim 64 and 128, fp32 / fp16 /
bf16), with a NaN-filled workspace, one workspace reused across calls of
different shapes, and paged against dense."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import empty_out, f64, to_host, upload
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(p, ps, ws, layout="NHD", dense=False):
    import torch

    import paged_kv_cache_pa_amd as pa

    q, k, v, bt, cl = upload(p, layout)
    out = empty_out(p)
    mcl = int(p.context_lens.max(initial=0))
    pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=mcl, partition_size=ps,
                 workspace=ws, layout=layout)
    torch.cuda.synchronize()
    return to_host(out, p.dtype)


def ref(p):
    return oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale,
                         p.dtype)


def check(p, got, what):
    if p.dtype == "f32":
        r = ref(p)
        rel = np.abs(f64(got, "f32") - r).max(axis=-1) / np.maximum(np.abs(r).max(axis=-1), 1e-300)
        assert rel.max() <= 1e-5, (what, rel.max())
    else:
        assert_fp_close(f64(got, p.dtype), ref(p), p.dtype, what)


CASES = [
    # (label, generator, partition)
    ("grouped-query bf16, 8 seqs to 16384 tokens (32 partitions)", lambda: W.config5(), 512),
    ("fp16 G 4, ragged with an empty and a 1-token sequence", lambda: W.random_paged(
        901, "f16", [1, 300, 77, 0, 1000, 513], 8, 2, 128), 64),
    ("fp16 MHA 40 heads, 70 partitions (past the merge's register pass)", lambda: W.random_paged(
        902, "f16", [16 * 70, 16 * 65 + 3, 5], 40, 40, 128), 16),
    ("fp32 G 8 on the VALU kernel, head dim 64", lambda: W.random_paged(
        903, "f32", [640, 17, 333], 16, 2, 64), 64),
    ("bf16 G 16", lambda: W.random_paged(
        904, "bf16", [2000, 1500, 31], 32, 2, 128), 128),
    ("fp16 G 7, head dim 64", lambda: W.random_paged(905, "f16", [900, 450], 14, 2, 64), 32),
]


@pytest.mark.parametrize("label,make,ps", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_split_cases(label, make, ps, layout):
    import torch

    import paged_kv_cache_pa_amd as pa

    p = make()
    print(label, layout, flush=True)
    S, Hq, D = p.q.shape
    params = pa.DecodeParams(S, Hq, p.num_kv_heads, D, p.block_size, p.max_blocks_per_seq,
                             p.num_blocks, int(p.context_lens.max()), ps,
                             {"f32": 0, "f16": 1, "bf16": 2}[p.dtype], pa.LAYOUTS[layout])
    need = pa.pa_decode_workspace_size(params)
    assert need > 0
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    got = run(p, ps, ws, layout)
    check(p, got, label)
    again = run(p, ps, ws, layout)
    assert same_bits(again, got), f"{label}: second call differs"


def test_one_workspace_across_shapes():
    """One buffer serves calls of different shapes one after another: a later
    call's partials land where an earlier one's were."""
    import torch

    ws = torch.zeros(4 << 20, dtype=torch.float32, device="cuda")
    made = [(label, make(), ps) for label, make, ps in CASES]
    order = [0, 1, 2, 3, 4, 5, 2, 0, 5, 1]
    first = {}
    for i in order:
        label, p, ps = made[i]
        got = run(p, ps, ws)
        if i in first:
            assert same_bits(got, first[i]), f"{label}: differs on reuse"
        else:
            check(p, got, label)
            first[i] = got


def test_split_equals_dense_split():
    """The paged and dense split-K launches share the merge: same bits."""
    import torch

    import paged_kv_cache_pa_amd as pa
    from gpu_util import in_layout, to_dev

    p = W.random_with_dense(906, "bf16", [3000, 1200, 17, 0, 2048], 12, 2, 128)
    ws = torch.zeros(1 << 20, dtype=torch.float32, device="cuda")
    got = run(p, 256, ws)
    out = empty_out(p)
    pa.pa_decode_dense(to_dev(p.q, "bf16"), to_dev(p.k_dense, "bf16"), to_dev(p.v_dense, "bf16"),
                       to_dev(p.context_lens), p.scale, out, max_context_len=3000,
                       partition_size=256, workspace=ws)
    torch.cuda.synchronize()
    assert same_bits(to_host(out, "bf16"), got)
    check(p, got, "ragged bf16 G 6")


# Partition counts at the edges of the merge forms: up to 8 partitions one
# thread per row chunk (merge_rows_kernel), then one wave per row up to 32
# (head dim 128) or 64 (head dim 64) partitions, then a 256-thread
# workgroup per row.  The longest sequence has exactly P partitions; the
# others end inside the first, the middle and the last of them.
MERGE_EDGES = [
    # (label, dtype, D, P)
    ("8 partitions, head dim 128", "f16", 128, 8),
    ("9 partitions, head dim 128", "bf16", 128, 9),
    ("32 partitions, head dim 128", "f16", 128, 32),
    ("33 partitions, head dim 128", "bf16", 128, 33),
    ("64 partitions, head dim 64", "f16", 64, 64),
    ("65 partitions, head dim 64", "bf16", 64, 65),
]


@pytest.mark.parametrize("label,dtype,d,P", MERGE_EDGES, ids=[m[0] for m in MERGE_EDGES])
def test_merge_form_edges(label, dtype, d, P):
    import torch

    import paged_kv_cache_pa_amd as pa

    ps = 16
    lens = [P * ps, P * ps - 5, 9, (P // 2) * ps + 1, 0, ps + 1]
    p = W.random_paged(907 + P, dtype, lens, 8, 2, d)
    print(label, flush=True)
    S, Hq, D = p.q.shape
    params = pa.DecodeParams(S, Hq, p.num_kv_heads, D, p.block_size, p.max_blocks_per_seq,
                             p.num_blocks, int(p.context_lens.max()), ps,
                             {"f32": 0, "f16": 1, "bf16": 2}[dtype], pa.LAYOUTS["HND"])
    ws = torch.full((pa.pa_decode_workspace_size(params) // 4,), float("nan"),
                    dtype=torch.float32, device="cuda")
    got = run(p, ps, ws, "HND")
    check(p, got, label)
    assert (f64(got, dtype)[4] == 0).all(), "the empty sequence's rows are zero"
