"""Plain-Python model of the KV block manager.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the tests compare
the library's C++ block manager with this model operation by operation.

Written from the pages' description, not from the library's code:

* [Kwon] "Efficient Memory Management for Large Language Model Serving with
  PagedAttention", section 3.4 "Memory Sharing": fork copies the parent's
  block table and adds one reference to each block; append writes into the
  last block when it has room, takes a new block when it is full, and copies
  a shared last block first (copy-on-write: take a block, copy, repoint, drop
  one reference from the old block); free drops one reference per table
  entry and returns blocks that reach zero to the free list.  "Scheduling
  and Preemption": a sequence group is evicted all or nothing; swapping moves
  its blocks to a CPU block allocator and back.
* [Int] "vLLM Internals ...", "PagedAttention: page tables, for KV": the
  allocator pops the free list and pushes released blocks back on it;
  "Ref counts and copy-on-write": the append rule, and the last sharer to
  write finds count 1 and writes in place.
* [Res] "Paged Attention: Managing the KV Cache Like Virtual Memory",
  "A paged KV cache, in code": reserve room for new tokens before the
  forward pass, copying a shared partly filled last block first.

Reading: the free list is a stack whose top is handed out next; a new pool's
stack hands out blocks in a given order (ascending ids by default, which
reproduces every table [Res] prints).  A call that cannot complete changes
nothing: this model applies the call to a deep copy of its state and keeps
the copy only if every step succeeded.

Parity is pinned by tests/test_block_manager.py: the tables, slots and
counts printed on the pages (tests/golden/), and a replay of every emitted
copy and slot write on a token-labelled pool that must give each sequence
back exactly its own token history.
"""
from __future__ import annotations

import copy


class BMError(Exception):
    """A refused call; ``status`` is the pa_status name."""

    def __init__(self, status: str):
        super().__init__(status)
        self.status = status


class OracleBlockManager:
    def __init__(self, num_gpu_blocks, num_cpu_blocks, block_size, gpu_free_order=None):
        if num_gpu_blocks < 1 or num_cpu_blocks < 0:
            raise BMError("PA_ERR_SHAPE")
        if block_size < 1 or block_size > 256 or block_size & (block_size - 1):
            raise BMError("PA_ERR_SHAPE")
        order = list(range(num_gpu_blocks)) if gpu_free_order is None else list(gpu_free_order)
        if sorted(order) != list(range(num_gpu_blocks)):
            raise BMError("PA_ERR_SHAPE")
        self.block_size = block_size
        # stacks: the LAST element is handed out next
        self.free = {"gpu": order[::-1], "cpu": list(range(num_cpu_blocks))[::-1]}
        self.refs = {"gpu": [0] * num_gpu_blocks, "cpu": [0] * num_cpu_blocks}
        self.seqs = {}          # handle -> {"table": [...], "n": int, "side": "gpu"|"cpu"}
        self.spare = []         # freed handles, most recent last
        self.count = 0          # handles ever issued

    # -- helpers -----------------------------------------------------------
    def _alloc(self, side):
        if not self.free[side]:
            raise BMError("PA_ERR_NO_BLOCKS")
        b = self.free[side].pop()
        self.refs[side][b] = 1
        return b

    def _release(self, side, b):
        self.refs[side][b] -= 1
        if self.refs[side][b] == 0:
            self.free[side].append(b)

    def _handle(self):
        if self.spare:
            return self.spare.pop()
        self.count += 1
        return self.count - 1

    def _group(self, seqs, side):
        if len(set(seqs)) != len(seqs):
            raise BMError("PA_ERR_STATE")
        for h in seqs:
            if h not in self.seqs:
                raise BMError("PA_ERR_STATE")
            if side is not None and self.seqs[h]["side"] != side:
                raise BMError("PA_ERR_STATE")

    def _atomic(self, fn):
        saved = copy.deepcopy(self.__dict__)
        try:
            return fn()
        except BMError:
            self.__dict__.clear()
            self.__dict__.update(saved)
            raise

    # -- the operations ----------------------------------------------------
    def new_seq(self):
        h = self._handle()
        self.seqs[h] = {"table": [], "n": 0, "side": "gpu"}
        return h

    def fork(self, parent):
        self._group([parent], "gpu")
        p = self.seqs[parent]
        h = self._handle()
        self.seqs[h] = {"table": list(p["table"]), "n": p["n"], "side": "gpu"}
        for b in p["table"]:
            self.refs["gpu"][b] += 1
        return h

    def free_group(self, seqs):
        self._group(seqs, None)
        for h in seqs:
            s = self.seqs.pop(h)
            for b in s["table"]:
                self._release(s["side"], b)
            self.spare.append(h)

    def reserve(self, seqs, num_new):
        """Returns (slot_mapping, block_pairs)."""
        self._group(seqs, "gpu")
        if any(k < 0 for k in num_new):
            raise BMError("PA_ERR_SHAPE")

        def run():
            B = self.block_size
            slots, pairs = [], []
            for h, k in zip(seqs, num_new):
                if k == 0:
                    continue
                s = self.seqs[h]
                if s["n"] % B != 0 and self.refs["gpu"][s["table"][-1]] > 1:
                    old = s["table"][-1]
                    new = self._alloc("gpu")
                    pairs.append((old, new))
                    self._release("gpu", old)
                    s["table"][-1] = new
                while len(s["table"]) * B < s["n"] + k:
                    s["table"].append(self._alloc("gpu"))
                for t in range(s["n"], s["n"] + k):
                    slots.append(s["table"][t // B] * B + t % B)
                s["n"] += k
            return slots, pairs

        return self._atomic(run)

    def tables(self, seqs, max_blocks_per_seq):
        """Returns (block_tables rows padded with -1, context_lens)."""
        rows, lens = [], []
        for h in seqs:
            if h not in self.seqs or self.seqs[h]["side"] != "gpu":
                raise BMError("PA_ERR_STATE")
            t = self.seqs[h]["table"]
            if len(t) > max_blocks_per_seq:
                raise BMError("PA_ERR_SHAPE")
            rows.append(t + [-1] * (max_blocks_per_seq - len(t)))
            lens.append(self.seqs[h]["n"])
        return rows, lens

    def _move(self, seqs, src, dst):
        self._group(seqs, src)

        def run():
            mapping, uses = {}, {}
            for h in seqs:                       # distinct blocks, first appearance
                for b in self.seqs[h]["table"]:
                    if b not in mapping:
                        mapping[b] = None
                        uses[b] = 0
                    uses[b] += 1
            if len(mapping) > len(self.free[dst]):
                raise BMError("PA_ERR_NO_BLOCKS")
            pairs = []
            for b in mapping:                    # dict keeps insertion order
                c = self._alloc(dst)
                self.refs[dst][c] = uses[b]
                mapping[b] = c
                pairs.append((b, c))
                for _ in range(uses[b]):
                    self._release(src, b)
            for h in seqs:
                s = self.seqs[h]
                s["table"] = [mapping[b] for b in s["table"]]
                s["side"] = dst
            return pairs

        return self._atomic(run)

    def swap_out(self, seqs):
        return self._move(seqs, "gpu", "cpu")

    def swap_in(self, seqs):
        return self._move(seqs, "cpu", "gpu")

    # -- observation -------------------------------------------------------
    def num_free(self):
        return len(self.free["gpu"]), len(self.free["cpu"])

    def free_list(self, side):
        """Next-to-be-handed-out first."""
        return self.free[side][::-1]

    def seq_info(self, h):
        if h not in self.seqs:
            raise BMError("PA_ERR_STATE")
        s = self.seqs[h]
        return s["n"], len(s["table"]), 0 if s["side"] == "gpu" else 1

    def block_table(self, h):
        if h not in self.seqs:
            raise BMError("PA_ERR_STATE")
        return list(self.seqs[h]["table"])
