"""The benchmark's own arithmetic (CPU): algorithmic bytes and flops against
hand counts, the headline workload's byte count, and the one-GPU guard."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_decode_bytes_hand_count():
    # 2 sequences of 1 and 17 tokens, 4 query / 2 kv heads, D 8, 2-byte
    # elements, 16-token blocks:
    #   K and V rows   18 tokens x 2 heads x 8 x 2 B x 2 = 1152
    #   q and out      2 x 2 seqs x 4 heads x 8 x 2 B  =  256
    #   table entries  (1 + 2 blocks) x 4 B              =   12
    #   lengths        2 x 4 B                           =    8
    assert bench.decode_bytes([1, 17], 4, 2, 8, 2, 16) == 1152 + 256 + 12 + 8
    assert bench.decode_bytes([0], 1, 1, 8, 4, 16) == 2 * 8 * 4 + 4   # q, out, one length


def test_headline_bytes():
    """The OPT-13B-shape batch: 26260 tokens x 40 heads x 128 x 2 B x 2 of
    K and V, q and out, 1670 table entries, 64 lengths; the appended rows
    add their stores."""
    lens, _ = W.config2_lens()
    assert int(lens.sum()) == 26260
    blocks = int(((lens + 15) // 16).sum())
    assert blocks == 1670
    kv = 26260 * 40 * 128 * 2 * 2
    qo = 2 * 64 * 40 * 128 * 2
    want = kv + qo + 4 * blocks + 4 * 64
    assert bench.decode_bytes(lens, 40, 40, 128, 2, 16) == want == 539122456
    assert want + 2 * 64 * 40 * 128 * 2 == 540433176


def test_prefill_flops_hand_count():
    # one sequence, 4 cached tokens, the last 2 are the chunk: rows at
    # positions 2 and 3 see 3 and 4 keys; 2 products x 2 flops x D x Hq each
    assert bench.prefill_flops(4, 2, 1, 1, 8) == 4 * 8 * (3 + 4)
    # a full causal prompt of n rows: n (n + 1) / 2 (query, key) pairs
    n, hq, d, s = 1024, 40, 128, 8
    assert bench.prefill_flops(n, n, s, hq, d) == 4 * d * hq * s * n * (n + 1) // 2
    assert bench.prefill_flops(n, n, s, hq, d) == 85983232000


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_replicas_leave_the_last_level_cache():
    assert bench.replicas_for(540_000_000) == 2            # 2 x 540 MB > 256 MB
    assert bench.replicas_for(87_000_000) * 87_000_000 >= 1 << 30
    assert bench.replicas_for(1) == 64                     # capped
    assert np.all([bench.replicas_for(b) >= 2 for b in (1, 10**6, 10**9, 10**10)])


def test_unique_bytes_hand_count():
    # 2 sequences sharing block 0 (16 full rows); sequence 0 also holds
    # block 1 with 3 rows, sequence 1 block 2 with 5 rows; 1 kv head, D 8,
    # 2-byte elements: unique K/V rows 16 + 3 + 5 = 24, logical 19 + 21 = 40
    tables = np.array([[0, 1], [0, 2]], np.int32)
    lens = [19, 21]
    rest = 2 * 2 * 1 * 8 * 2 + 4 * 4 + 4 * 2          # q/out, 4 table entries, 2 lengths
    assert bench.unique_decode_bytes(tables, lens, 1, 1, 8, 2, 16) == 24 * 8 * 2 * 2 + rest
    assert bench.decode_bytes(lens, 1, 1, 8, 2, 16) == 40 * 8 * 2 * 2 + rest
    # a block shared with different fill: its most-used rows count once
    tables = np.array([[4], [4]], np.int32)
    assert bench.unique_decode_bytes(tables, [7, 12], 1, 1, 8, 2, 16) == \
        12 * 8 * 2 * 2 + 2 * 2 * 8 * 2 + 4 * 2 + 4 * 2


def test_beams_unique_bytes():
    """Parallel sampling: each group's 512-token prompt (32 full blocks) is
    stored once and read by its 6 beams; after the copy-on-write split every
    beam owns its stem block and suffix.  So the unique K/V rows are the
    logical ones minus 5 x 512 per group."""
    p = W.config4(poison=False).paged
    e, row = 2, 40 * 128 * 2 * 2
    logical = bench.decode_bytes(p.context_lens, 40, 40, 128, e, 16)
    unique = bench.unique_decode_bytes(p.block_tables, p.context_lens, 40, 40, 128, e, 16)
    assert logical - unique == 16 * 5 * 512 * row
