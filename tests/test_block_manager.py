"""Host KV block manager: the plain-Python model (oracle/block_manager.py)
pinned to the tables the pages print, and the library's C++ manager
(include/pa_block_manager.h) checked against that model operation by
operation.  CPU only: the manager never touches the GPU.

Pins (each applies to both implementations):
  * [Kwon] Figure 6 slots, [Int] flowchart state, [Int] copy-on-write trace,
    [Res] four-sample tables, [Res] two-prompt interleaving, [Kwon] Figure 9
    beam update (tests/golden/);
  * replay: every emitted copy pair and slot is applied to a token-labelled
    pool, and every live sequence must read back exactly its own history
    (its parent's tokens up to the fork, then its own);
  * all-or-nothing: a refused call leaves every observable unchanged.
"""
from __future__ import annotations

import json
import os
import random

import pytest

from oracle.block_manager import BMError, OracleBlockManager

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


class LibManager:
    """The C++ manager behind the oracle's interface (lists in, lists out)."""

    def __init__(self, num_gpu_blocks, num_cpu_blocks, block_size, gpu_free_order=None):
        from paged_kv_cache_pa_amd import PaError
        from paged_kv_cache_pa_amd.block_manager import BlockManager

        self._E = PaError
        try:
            self.m = BlockManager(num_gpu_blocks, num_cpu_blocks, block_size, gpu_free_order)
        except PaError as e:
            raise BMError(e.name) from None
        except ValueError:  # the binding refuses an order of the wrong length itself
            raise BMError("PA_ERR_SHAPE") from None
        self.block_size = block_size

    def _call(self, f, *a):
        try:
            return f(*a)
        except self._E as e:
            raise BMError(e.name) from None

    def new_seq(self):
        return self._call(self.m.new_seq)

    def fork(self, p):
        return self._call(self.m.fork, p)

    def free_group(self, seqs):
        return self._call(self.m.free, seqs)

    def reserve(self, seqs, k):
        slots, pairs = self._call(self.m.reserve, seqs, k)
        return slots.tolist(), [tuple(p) for p in pairs.tolist()]

    def tables(self, seqs, mbs):
        bt, cl = self._call(self.m.tables, seqs, mbs)
        return bt.tolist(), cl.tolist()

    def swap_out(self, seqs):
        return [tuple(p) for p in self._call(self.m.swap_out, seqs).tolist()]

    def swap_in(self, seqs):
        return [tuple(p) for p in self._call(self.m.swap_in, seqs).tolist()]

    def num_free(self):
        return self.m.num_free()

    def free_list(self, side):
        return self.m.free_list(side == "cpu")

    def seq_info(self, h):
        return self._call(self.m.seq_info, h)

    def block_table(self, h):
        return self._call(self.m.block_table, h)

    def ref(self, side, b):
        return self.m.ref_count(b, side == "cpu")


class OracleAdapter(OracleBlockManager):
    def ref(self, side, b):
        return self.refs[side][b]


def lib_available():
    try:
        from paged_kv_cache_pa_amd import lib

        lib()
        return True
    except Exception:
        return False


IMPLS = ["oracle", pytest.param("lib", marks=pytest.mark.skipif(
    not lib_available(), reason="libpa.so not built"))]


def make(impl, *a, **kw):
    return (OracleAdapter if impl == "oracle" else LibManager)(*a, **kw)


def order_from(first, n):
    """A free order that hands out `first` and then the rest ascending."""
    return list(first) + [b for b in range(n) if b not in first]


# --------------------------------------------------------------- golden pins
@pytest.mark.parametrize("impl", IMPLS)
def test_fig6_slots(impl):
    g = golden("fig6_block_table.json")
    m = make(impl, g["num_blocks"], 0, g["block_size"], order_from(g["block_table"], g["num_blocks"]))
    s = m.new_seq()
    slots = m.reserve([s], [7])[0] + m.reserve([s], [1])[0] + m.reserve([s], [1])[0]
    assert slots == g["slots"]
    assert m.block_table(s) == g["block_table"]
    assert m.seq_info(s)[0] == g["context_len"]
    B, n = g["block_size"], g["context_len"]
    filled = [min(B, n - i * B) for i in range(len(g["block_table"]))]
    assert filled == g["filled"]


@pytest.mark.parametrize("impl", IMPLS)
def test_internals_flowchart(impl):
    g = golden("internals_flowchart.json")
    nb = g["num_blocks"]
    m = make(impl, nb, 0, g["block_size"], order_from([7, 1, 3, 9], nb))
    a = m.new_seq()
    m.reserve([a], [32])
    b = m.fork(a)
    m.reserve([a, b], [4, 11])
    rows, lens = m.tables([a, b], 3)
    assert rows == g["tables"] and lens == g["context_lens"]
    for blk, r in g["ref_counts"].items():
        assert m.ref("gpu", int(blk)) == r
    assert sorted(m.free_list("gpu")) == g["free"]


@pytest.mark.parametrize("impl", IMPLS)
def test_internals_cow_trace(impl):
    g = golden("internals_cow_trace.json")
    nb = g["num_blocks"]
    m = make(impl, nb, 0, g["block_size"], order_from([7, 1, 3], nb))
    a1 = m.new_seq()
    m.reserve([a1], [g["context_len_before"]])
    assert m.block_table(a1) == g["shared_table"]
    a2 = m.fork(a1)
    s1, p1 = m.reserve([a1], [1])
    s2, p2 = m.reserve([a2], [1])
    assert [list(p) for p in p1 + p2] == g["copy_pairs"]
    assert s1 == [g["write_slots"]["A1"]] and s2 == [g["write_slots"]["A2"]]
    assert m.block_table(a1) == g["tables_after"]["A1"]
    assert m.block_table(a2) == g["tables_after"]["A2"]
    assert m.ref("gpu", 7) == 2 and m.ref("gpu", 1) == 1 and m.ref("gpu", 3) == 1


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("batched", [False, True])
def test_res_four_samples(impl, batched):
    g = golden("share_py_tables.json")
    m = make(impl, 64, 0, g["block_size"])
    first = m.new_seq()
    m.reserve([first], [g["prompt_len"]])
    assert m.block_table(first) == g["prompt_blocks"]
    seqs = [first] + [m.fork(first) for _ in range(g["samples"] - 1)]
    pairs = []
    for _ in range(g["final_context_len"] - g["prompt_len"]):
        if batched:
            pairs += m.reserve(seqs, [1] * len(seqs))[1]
        else:
            for s in seqs:
                pairs += m.reserve([s], [1])[1]
    assert [m.block_table(s) for s in seqs] == g["tables"]
    assert [list(p) for p in pairs] == g["copy_pairs"] and len(pairs) == g["copies"]
    assert 64 - m.num_free()[0] == g["blocks_in_use"]
    B = g["block_size"]
    unshared = g["samples"] * -(-g["final_context_len"] // B)
    assert unshared == g["blocks_without_sharing"]


@pytest.mark.parametrize("impl", IMPLS)
def test_res_two_prompts(impl):
    g = golden("res_two_prompts.json")
    m = make(impl, g["num_blocks"], 0, g["block_size"])
    seqs = [m.new_seq() for _ in g["prompt_lens"]]
    for t in range(g["turns"]):
        for s, p in zip(seqs, g["prompt_lens"]):
            m.reserve([s], [p if t == 0 else 1])
    assert [m.block_table(s) for s in seqs] == g["tables"]
    assert [m.seq_info(s)[0] for s in seqs] == g["context_lens"]
    assert m.num_free()[0] == g["free_blocks"]


@pytest.mark.parametrize("impl", IMPLS)
def test_kwon_fig9_beam_update(impl):
    g = golden("kwon_fig9_beams.json")
    B = g["block_size"]
    m = make(impl, g["num_blocks"], 0, B)
    root = m.new_seq()
    m.reserve([root], [B])                  # block 0
    c3 = m.fork(root)
    for s in (root, c3, root, c3):          # blocks 1, 2, 3, 4
        m.reserve([s], [B])
    c1, c2 = m.fork(root), m.fork(root)
    cands = [root, c1, c2, c3]
    m.reserve(cands, [B] * 4)               # blocks 5, 6, 7, 8
    assert [m.block_table(c) for c in cands] == g["before"]
    new = [m.fork(cands[p]) for p in g["parents"]]
    m.reserve(new, [B] * 4)                 # blocks 9..12
    before_free = set(m.free_list("gpu"))
    m.free_group(cands)
    assert [m.block_table(c) for c in new] == g["after"]
    assert sorted(set(m.free_list("gpu")) - before_free) == g["freed"]


# ------------------------------------------------------------ replay checker
class Replay:
    """Token-labelled pools.  Applies the manager's outputs the way the
    device entry points would and tracks what each sequence should read."""

    def __init__(self, m):
        self.m, self.B = m, m.block_size
        self.mem = {"gpu": {}, "cpu": {}}
        self.hist = {}
        self.label = 0

    def new_seq(self):
        h = self.m.new_seq()
        self.hist[h] = []
        return h

    def fork(self, p):
        h = self.m.fork(p)
        self.hist[h] = list(self.hist[p])
        return h

    def _copy_block(self, src_side, src, dst_side, dst):
        for o in range(self.B):
            v = self.mem[src_side].get(src * self.B + o)
            self.mem[dst_side][dst * self.B + o] = v

    def reserve(self, seqs, ks):
        slots, pairs = self.m.reserve(seqs, ks)
        for src, dst in pairs:              # pa_copy_blocks first
            self._copy_block("gpu", src, "gpu", dst)
        it = iter(slots)                    # then pa_cache_write
        for s, k in zip(seqs, ks):
            for _ in range(k):
                self.label += 1
                self.mem["gpu"][next(it)] = self.label
                self.hist[s].append(self.label)
        assert next(it, None) is None
        return slots, pairs

    def free(self, seqs):
        self.m.free_group(seqs)
        for s in seqs:
            del self.hist[s]

    def swap_out(self, seqs):
        pairs = self.m.swap_out(seqs)
        for g, c in pairs:
            self._copy_block("gpu", g, "cpu", c)
        return pairs

    def swap_in(self, seqs):
        pairs = self.m.swap_in(seqs)
        for c, g in pairs:
            self._copy_block("cpu", c, "gpu", g)
        return pairs

    def check(self):
        for h, want in self.hist.items():
            n, nb, where = self.m.seq_info(h)
            assert n == len(want) and nb == -(-n // self.B)
            side = "cpu" if where else "gpu"
            t = self.m.block_table(h)
            got = [self.mem[side].get(t[i // self.B] * self.B + i % self.B) for i in range(n)]
            assert got == want, f"sequence {h} reads back another history"
        # reference counts equal the table entries naming each block; the
        # free stacks hold exactly the unreferenced blocks
        for side in ("gpu", "cpu"):
            named = {}
            for h in self.hist:
                if (self.m.seq_info(h)[2] == 1) == (side == "cpu"):
                    for b in self.m.block_table(h):
                        named[b] = named.get(b, 0) + 1
            free = self.m.free_list(side)
            assert len(set(free)) == len(free)
            assert not (set(free) & set(named))
            for b, r in named.items():
                assert self.m.ref(side, b) == r


def random_ops(rp, rng, steps, swap=True):
    """Random fork / reserve / free / swap traffic; refused calls allowed."""
    live = [rp.new_seq()]
    refused = 0
    for _ in range(steps):
        on_gpu = [s for s in live if rp.m.seq_info(s)[2] == 0]
        swapped = [s for s in live if rp.m.seq_info(s)[2] == 1]
        op = rng.random()
        try:
            if op < 0.08 or not live:
                live.append(rp.new_seq())
            elif op < 0.25 and on_gpu:
                live.append(rp.fork(rng.choice(on_gpu)))
            elif op < 0.75 and on_gpu:
                batch = rng.sample(on_gpu, rng.randint(1, len(on_gpu)))
                ks = [rng.choice([0, 1, 1, 1, 2, rp.B, 2 * rp.B + 1]) for _ in batch]
                rp.reserve(batch, ks)
            elif op < 0.85 and live:
                grp = rng.sample(live, rng.randint(1, min(3, len(live))))
                rp.free(grp)
                live = [s for s in live if s not in grp]
            elif swap and op < 0.93 and on_gpu:
                rp.swap_out(rng.sample(on_gpu, rng.randint(1, min(3, len(on_gpu)))))
            elif swap and swapped:
                rp.swap_in(rng.sample(swapped, rng.randint(1, len(swapped))))
        except BMError as e:
            assert e.status == "PA_ERR_NO_BLOCKS"
            refused += 1
        rp.check()
    return refused


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("nb,ncpu,B,seed", [(12, 6, 4, 1), (40, 40, 16, 2), (9, 0, 1, 3),
                                            (64, 16, 2, 4), (24, 24, 8, 5)])
def test_replay_every_sequence_reads_its_history(impl, nb, ncpu, B, seed):
    rp = Replay(make(impl, nb, ncpu, B))
    refused = random_ops(rp, random.Random(seed), 400, swap=ncpu > 0)
    assert refused > 0  # the pools are small enough that exhaustion happens


def snapshot(m, handles):
    g, c = m.num_free()
    state = {"free": (g, c, m.free_list("gpu"), m.free_list("cpu"))}
    for h in handles:
        try:
            state[h] = (m.seq_info(h), m.block_table(h))
        except BMError:
            state[h] = None
    return state


@pytest.mark.parametrize("impl", IMPLS)
def test_refused_calls_change_nothing(impl):
    m = make(impl, 10, 3, 4)
    a = m.new_seq()
    m.reserve([a], [9])                  # 3 blocks
    b = m.fork(a)
    c = m.fork(a)                        # last block shared 3 ways, 1 slot used
    before = snapshot(m, [a, b, c])
    # copies for a and b (c writes in place) + 3 new blocks each would need 2 + 9 > 7
    with pytest.raises(BMError) as e:
        m.reserve([a, b, c], [12, 12, 12])
    assert e.value.status == "PA_ERR_NO_BLOCKS"
    assert snapshot(m, [a, b, c]) == before
    # swapping a group that names more distinct blocks than the host pool holds
    m2 = make(impl, 10, 2, 4)
    x = m2.new_seq()
    m2.reserve([x], [9])
    before = snapshot(m2, [x])
    with pytest.raises(BMError) as e:
        m2.swap_out([x])
    assert e.value.status == "PA_ERR_NO_BLOCKS"
    assert snapshot(m2, [x]) == before


@pytest.mark.parametrize("impl", IMPLS)
def test_refusals(impl):
    m = make(impl, 8, 4, 4)
    a = m.new_seq()
    m.reserve([a], [5])
    cases = [
        (lambda: m.reserve([a, a], [1, 1]), "PA_ERR_STATE"),
        (lambda: m.reserve([a + 7], [1]), "PA_ERR_STATE"),
        (lambda: m.reserve([a], [-1]), "PA_ERR_SHAPE"),
        (lambda: m.fork(a + 7), "PA_ERR_STATE"),
        (lambda: m.free_group([a, a]), "PA_ERR_STATE"),
        (lambda: m.swap_in([a]), "PA_ERR_STATE"),
        (lambda: m.tables([a], 1), "PA_ERR_SHAPE"),
    ]
    for f, status in cases:
        with pytest.raises(BMError) as e:
            f()
        assert e.value.status == status
    m.swap_out([a])
    for f in (lambda: m.reserve([a], [1]), lambda: m.fork(a), lambda: m.tables([a], 4),
              lambda: m.swap_out([a])):
        with pytest.raises(BMError) as e:
            f()
        assert e.value.status == "PA_ERR_STATE"
    m.swap_in([a])
    assert m.seq_info(a) == (5, 2, 0)
    for bad in ([0, 0, 1, 2, 3, 4, 5, 6], [0, 1, 2], [0, 1, 2, 3, 4, 5, 6, 8]):
        with pytest.raises(BMError) as e:
            make(impl, 8, 0, 4, bad)
        assert e.value.status == "PA_ERR_SHAPE"
    for args in ((0, 0, 4), (8, -1, 4), (8, 0, 3), (8, 0, 512)):
        with pytest.raises(BMError) as e:
            make(impl, *args)
        assert e.value.status == "PA_ERR_SHAPE"


@pytest.mark.parametrize("impl", IMPLS)
def test_swap_keeps_sharing_inside_the_group(impl):
    """Two forks sharing a prompt swap out as one group: each shared block
    gets one host block (the group's references move together), and swap-in
    gives every sequence back its tokens."""
    rp = Replay(make(impl, 16, 16, 4))
    p = rp.new_seq()
    rp.reserve([p], [10])                 # blocks 0, 1, 2 (2 half full)
    q = rp.fork(p)
    rp.reserve([p, q], [1, 3])            # p copies 2 -> 3; q fills 2 in place, takes 4
    other = rp.fork(q)                    # a sequence outside the group
    rp.check()
    pairs = rp.swap_out([p, q])
    assert [g for g, _ in pairs] == [0, 1, 3, 2, 4]  # each distinct block once
    assert rp.m.ref("gpu", 0) == 1 and rp.m.ref("cpu", pairs[0][1]) == 2
    rp.check()
    rp.reserve([other], [5])
    back = rp.swap_in([p, q])
    assert len(back) == 5
    rp.check()


def test_lib_matches_oracle_operation_by_operation():
    if not lib_available():
        pytest.skip("libpa.so not built")
    for seed, (nb, ncpu, B) in enumerate([(16, 8, 4), (33, 11, 1), (64, 64, 16), (20, 5, 2)]):
        ms = [OracleAdapter(nb, ncpu, B), LibManager(nb, ncpu, B)]
        rngs = [random.Random(seed), random.Random(seed)]
        logs = [[], []]
        for m, rng, log in zip(ms, rngs, logs):
            rp = Replay(m)
            orig = rp.m

            class Logged:
                block_size = B

                def __getattr__(self, name):
                    f = getattr(orig, name)

                    def g(*a):
                        try:
                            r = f(*a)
                        except BMError as e:
                            log.append((name, a, e.status))
                            raise
                        log.append((name, a, r))
                        return r
                    return g

            rp.m = Logged()
            random_ops(rp, rng, 600, swap=ncpu > 0)
        assert len(logs[0]) == len(logs[1])
        for x, y in zip(*logs):
            assert x == y
