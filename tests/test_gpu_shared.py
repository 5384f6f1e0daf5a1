"""pa_decode_shared (sequences in groups that share leading blocks: each
shared block read once per group) against the fp64 oracle's decode, which
knows nothing of sharing, and against pa_decode.  Tolerance as decode
(|err| <= 2e-3 + 1e-2 |ref| for fp16 / bf16).

Cases: config 4 (16 prompts x 6 beams sharing a 512-token prompt, after
its copy-on-write and new-token writes) at partition sizes that share 0, 1,
2 and 4 partitions; synthetic groups with members shorter than the shared
prefix, empty members, single-sequence groups, a group too wide for one
16-column tile (computed unshared), grouped-query heads, head dim 64 and
block size 8 (steps spanning blocks), both pool layouts; a workspace full
of NaN; repeated calls (same bits); no groups (same bits as pa_decode).
Each sequence's count of partitions taken by the grouped pass is read back
from the workspace, and the shared partitions are shown to be read through
the group's first sequence: with the other members' shared table entries
pointed at a NaN block the result is unchanged."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import empty_out, f64, in_layout, run_decode, to_dev, to_host, upload
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu
LAYOUTS = ["NHD", "HND"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def poisoned_table(p, gs, sp, ps, nan_block):
    """The table with every member but the first of each group pointed at a
    NaN block for its shared partitions (sp per sequence): the result stays
    exact only if those partitions are read once, through the group's first
    sequence (as pa_decode_shared states)."""
    t = p.block_tables.copy()
    for i in range(len(gs) - 1):
        for s in range(gs[i] + 1, gs[i + 1]):
            nb = int(sp[s]) * ps // p.block_size
            if nb > 0:
                t[s, :nb] = nan_block
    return t


def unused_block(p):
    used = set(int(b) for b in p.block_tables.ravel() if b >= 0)
    return next(b for b in range(p.k_cache.shape[0]) if b not in used)


def run_shared(p, gstart, gshared, layout, ps, tensors=None, max_shared=None, skips=None,
               table=None):
    """pa_decode_shared with a NaN-filled workspace; returns the host output
    (and appends to ``skips`` each sequence's count of partitions the
    grouped pass computed, read back from the workspace)."""
    import torch

    import paged_kv_cache_pa_amd as pa

    q, k, v, bt, cl = tensors if tensors is not None else upload(p, layout)
    if table is not None:  # in place of the block table
        bt = to_dev(table)
    S, Hq, D = p.q.shape
    mcl = int(p.context_lens.max())
    P = -(-mcl // ps) if mcl > ps else 1
    words = S * Hq * P * (D + 2) + S + 64
    ws = torch.full((words,), float("nan"), dtype=torch.float32, device=q.device)
    out = empty_out(p)
    pa.pa_decode_shared(q, k, v, bt, cl, to_dev(gstart), to_dev(gshared), p.scale, out,
                        max_shared_blocks=int(gshared.max()) if max_shared is None else max_shared,
                        max_context_len=mcl, partition_size=ps, workspace=ws, layout=layout)
    torch.cuda.synchronize()
    if skips is not None:
        off = (S * Hq * P * (D + 2) * 4 if P > 1 else 0) + 15 & ~15
        skips.append(ws.view(torch.int32)[off // 4: off // 4 + S].cpu().numpy().copy())
    return to_host(out, p.dtype)


@pytest.fixture(scope="module")
def beams():
    """Config 4 after its copy-on-write and new-token writes (host state from
    the oracle's copy and write, which the parity tests pin bitwise)."""
    sc = W.config4()
    p = sc.paged
    kc, vc = oracle.copy_blocks(p.k_cache, p.v_cache, p.block_pairs, "f16")
    kc, vc = oracle.cache_write(p.k_new, p.v_new, kc, vc, p.slot_mapping, "f16")
    pw = W.Paged("f16", p.q, kc, vc, p.block_tables, p.context_lens, p.scale, 16)
    ref = oracle.decode(p.q, kc, vc, p.block_tables, p.context_lens, p.scale, "f16")
    return pw, ref, W.config4_groups(sc)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_config4_beams(beams, layout):
    pw, ref, (gs, gsh) = beams
    t = upload(pw, layout)
    # 512-token prompt: 1, 2 and 4 shared partitions; 1024 covers each whole
    # context in one partition that the prompt does not fill (nothing shared)
    for ps, shared_parts in ((512, 1), (256, 2), (128, 4), (1024, 0)):
        print(f"config4 {layout} partition {ps}", flush=True)
        skips = []
        got = run_shared(pw, gs, gsh, layout, ps, tensors=t, skips=skips)
        assert_fp_close(f64(got, "f16"), ref, "f16", f"config4 shared {layout} partition {ps}")
        # every beam's prompt partitions came from its group's pass, read
        # through the group's first beam
        assert (skips[0] == shared_parts).all(), (ps, skips[0])
        table = poisoned_table(pw, gs, skips[0], ps, unused_block(pw))
        got = run_shared(pw, gs, gsh, layout, ps, tensors=t, table=table)
        assert_fp_close(f64(got, "f16"), ref, "f16", f"config4 shared {layout} partition {ps}, "
                                                     "the other beams' prompt entries poisoned")
    plain = run_decode(pw, partition_size=512, tensors=t, layout=layout)
    assert_fp_close(f64(run_shared(pw, gs, gsh, layout, 512, tensors=t), "f16"), f64(plain, "f16"),
                    "f16", "shared vs pa_decode")


# (shared blocks, member lengths) per group, in batch order
MHA_GROUPS = [
    (8, [130, 140, 200, 129, 250, 135]),     # parallel samples of a 128-token prompt
    (0, [77]),                               # alone
    (5, [40, 0, 200]),                       # one member inside the prefix, one empty
    (4, [64, 65, 66, 90, 100, 70, 80, 81, 82, 83, 84, 85, 86, 87, 88, 120]),  # 16 members
    (3, [48]),                               # alone, with a "shared" prefix
    (6, [96, 96]),                           # the whole context shared
]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype,d,B", [("f16", 128, 16), ("bf16", 64, 8), ("f16", 64, 32)])
def test_synthetic_groups_mha(dtype, d, B, layout):
    groups = [(sb * 16 // B, ms) for sb, ms in MHA_GROUPS]  # the same shared tokens
    p, gs, gsh = W.random_shared(91, dtype, groups, 4, 4, d, block_size=B)
    ref = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dtype)
    t = upload(p, layout)
    for ps in (32, 64, 128):
        if ps % B:
            continue
        print(f"mha {dtype} d{d} B{B} {layout} partition {ps}", flush=True)
        skips = []
        got = run_shared(p, gs, gsh, layout, ps, tensors=t, skips=skips)
        assert_fp_close(f64(got, dtype), ref, dtype, f"shared mha {dtype} {layout} ps {ps}")
        # expected: whole partitions in each group's shared tokens, for
        # groups of 2+ members; 0 for single members and the empty one
        want = []
        for sb, ms in groups:
            sp = sb * B // ps if len(ms) >= 2 else 0
            want += [sp if n > 0 else 0 for n in ms]
        assert (skips[0] == np.array(want)).all(), (ps, skips[0], want)
        got = run_shared(p, gs, gsh, layout, ps, tensors=t,
                         table=poisoned_table(p, gs, want, ps, unused_block(p)))
        assert_fp_close(f64(got, dtype), ref, dtype, f"shared mha {dtype} {layout} ps {ps} poisoned")
        assert (f64(got, dtype)[8] == 0).all(), "the empty member's row is zero"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_synthetic_groups_gqa(layout):
    """2 query heads per kv head: 8 members fill the 16 columns; 9 do not
    (that group is computed unshared)."""
    groups = [(6, [100 + 7 * i for i in range(8)]), (6, [97 + 5 * i for i in range(9)]),
              (2, [33, 200]), (0, [15, 16])]
    p, gs, gsh = W.random_shared(92, "bf16", groups, 8, 4, 128)
    ref = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "bf16")
    t = upload(p, layout)
    for ps in (32, 96):
        print(f"gqa {layout} partition {ps}", flush=True)
        skips = []
        got = run_shared(p, gs, gsh, layout, ps, tensors=t, skips=skips)
        assert_fp_close(f64(got, "bf16"), ref, "bf16", f"shared gqa {layout} ps {ps}")
        sp = 6 * 16 // ps
        want = [sp] * 8 + [0] * 9 + [2 * 16 // ps] * 2 + [0] * 2
        assert (skips[0] == np.array(want)).all(), (ps, skips[0], want)
        got = run_shared(p, gs, gsh, layout, ps, tensors=t,
                         table=poisoned_table(p, gs, want, ps, unused_block(p)))
        assert_fp_close(f64(got, "bf16"), ref, "bf16", f"shared gqa {layout} ps {ps} poisoned")


def test_deterministic_and_no_groups():
    """Repeated calls give the same bits; with no groups the call is pa_decode
    with the same split (same bits); a max_shared_blocks below a group's
    shared count shares less (still exact within tolerance)."""
    import torch

    import paged_kv_cache_pa_amd as pa

    p, gs, gsh = W.random_shared(93, "f16", [(8, [140, 150, 160, 170]), (4, [70, 90])], 4, 4, 128)
    ref = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "f16")
    t = upload(p, "HND")
    a = run_shared(p, gs, gsh, "HND", 32, tensors=t)
    b = run_shared(p, gs, gsh, "HND", 32, tensors=t)
    assert same_bits(a, b)
    assert_fp_close(f64(a, "f16"), ref, "f16", "shared")
    low = run_shared(p, gs, gsh, "HND", 32, tensors=t, max_shared=2)
    assert_fp_close(f64(low, "f16"), ref, "f16", "shared, lower bound")
    q, k, v, bt, cl = t
    out = empty_out(p)
    pa.pa_decode_shared(q, k, v, bt, cl, to_dev(gs[:1]), to_dev(gsh[:0]), p.scale, out,
                        max_shared_blocks=0, max_context_len=int(p.context_lens.max()),
                        partition_size=32, layout="HND")
    torch.cuda.synchronize()
    plain = run_decode(p, partition_size=32, tensors=t, layout="HND")
    assert same_bits(to_host(out, "f16"), plain)


def test_back_to_back_calls_and_graph_replays():
    """Calls issued back to back on one stream with one shared workspace (no
    synchronisation between them) each see only their own partials, on the
    default stream and on another one; and the call (grouped pass, usual
    pass, merge) captured in a HIP graph replays, after eager NaN poisoning
    of its output and workspace, with the eager call's bits and the
    oracle's values every time."""
    import torch

    import paged_kv_cache_pa_amd as pa

    p, gs, gsh = W.random_shared(94, "f16", [(8, [140, 150, 160, 170]), (4, [70, 90]), (0, [33])],
                                 4, 4, 128)
    rng = np.random.default_rng(95)
    q2 = W.randn(rng, p.q.shape, "f16")
    ref1 = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "f16")
    ref2 = oracle.decode(q2, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "f16")
    q, k, v, bt, cl = upload(p, "HND")
    qb = to_dev(q2, "f16")
    gs_d, gsh_d = to_dev(gs), to_dev(gsh)
    mcl = int(p.context_lens.max())
    ps = 32
    S, Hq, D = p.q.shape
    P = -(-mcl // ps)
    ws = torch.full((S * Hq * P * (D + 2) + S + 64,), float("nan"), dtype=torch.float32,
                    device=q.device)

    def call(qq, out, stream=None):
        pa.pa_decode_shared(qq, k, v, bt, cl, gs_d, gsh_d, p.scale, out,
                            max_shared_blocks=int(gsh.max()), max_context_len=mcl,
                            partition_size=ps, workspace=ws, layout="HND", stream=stream)

    torch.cuda.synchronize()   # the inputs are ready for any stream
    first = None
    for stream in (None, torch.cuda.Stream()):
        with torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(
                torch.cuda.current_stream()):
            outs = [empty_out(p) for _ in range(4)]
            for i, o in enumerate(outs):   # q, q2, q, q2 back to back
                call(q if i % 2 == 0 else qb, o)
        torch.cuda.synchronize()
        got = [to_host(o, "f16") for o in outs]
        assert_fp_close(f64(got[0], "f16"), ref1, "f16", "back to back, first")
        assert_fp_close(f64(got[1], "f16"), ref2, "f16", "back to back, second")
        assert same_bits(got[0], got[2]) and same_bits(got[1], got[3]), "back to back: repeat differs"
        if first is None:
            first = got[0]
        assert same_bits(got[0], first), "default stream vs another stream"

    out = empty_out(p)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(q, out)          # one eager call on the capture stream first
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(q, out)
    torch.cuda.synchronize()
    for replay in range(4):
        out.fill_(float("nan"))
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = to_host(out, "f16")
        assert same_bits(got, first), f"replay {replay} differs from the eager call"
        assert_fp_close(f64(got, "f16"), ref1, "f16", f"replay {replay}")
