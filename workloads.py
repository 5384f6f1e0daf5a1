"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and decides where blocks sit in the
pool.  It holds none of the method's arithmetic (no attention, no softmax, no
cache_write or copy_blocks step): both the fp64 oracle (``oracle/``) and the
HIP library are fed from here, and nothing here is shared with either beyond
the arrays it returns.

Recipe (stated once, used everywhere):

* ``numpy.random.default_rng(seed)`` (PCG64).  Values are drawn in fp32 from
  N(0, 1) and cast to the storage dtype with round-to-nearest-even (torch's
  CPU cast).  bf16 arrays are held as ``uint16`` bit patterns.
* Physical placement: a seeded permutation of the pool is consumed in
  (sequence, logical block) order, so consecutive logical blocks land at
  unrelated physical ids ("blocks can be stored anywhere", Efficient Memory
  Management ... with PagedAttention, §3.4 "PagedAttention Algorithm").
* Unused block-table entries are -1.  In ``poison=True`` mode every slot that
  no valid token occupies (the tail of a last block, unassigned blocks) holds
  NaN, so that any read past ``context_lens`` shows up in the output.

Layouts (the library's):
  q, out          [S, Hq, D]
  k_cache/v_cache [NB, B, Hkv, D]   (one block = B rows of the dense layout)
  block_tables    [S, MBS] int32
  context_lens    [S] int32
  dense k/v       [S, Smax, Hkv, D]
  k_new/v_new     [N, Hkv, D], slot_mapping [N] int32 (slot = block*B + offset)
  block_pairs     [n, 2] int32 (src, dst)
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
_NAN_BITS = {"f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round an fp32 array to the storage dtype (RNE); bf16 -> uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)  # numpy's cast is round-to-nearest-even
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(x).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a storage array to float64 (used by tests only)."""
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def nan_fill(shape, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, _NAN_BITS[dtype], dtype=np.uint16).view(
        np.float16 if dtype == "f16" else np.uint16)


def randn(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return to_storage(rng.standard_normal(size=shape, dtype=np.float32), dtype)


@dataclasses.dataclass
class Paged:
    """One decode batch over a paged pool."""

    dtype: str
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    scale: float
    block_size: int
    partition_size: int = 0
    # optional companion work that precedes the decode
    k_new: Optional[np.ndarray] = None
    v_new: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None
    block_pairs: Optional[np.ndarray] = None
    # dense twin of the same values, [S, Smax, Hkv, D] (config 3)
    k_dense: Optional[np.ndarray] = None
    v_dense: Optional[np.ndarray] = None
    name: str = ""

    @property
    def num_seqs(self):
        return self.q.shape[0]

    @property
    def num_q_heads(self):
        return self.q.shape[1]

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]

    @property
    def num_kv_heads(self):
        return self.k_cache.shape[2]

    @property
    def max_blocks_per_seq(self):
        return self.block_tables.shape[1]

    def kv_bytes(self) -> int:
        """Bytes of valid K and V the decode must read (both tensors)."""
        e = ELEM_BYTES[self.dtype]
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * e


# --------------------------------------------------------------------------
# building blocks


def place(rng, lens, block_size, num_blocks, mbs=None):
    """Assign physical ids from a seeded permutation in (seq, logical) order."""
    nblk = [(int(n) + block_size - 1) // block_size for n in lens]
    need = sum(nblk)
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks < {need} needed")
    mbs = mbs if mbs is not None else max(1, max(nblk) if nblk else 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((len(lens), mbs), -1, dtype=np.int32)
    pos = 0
    for s, nb in enumerate(nblk):
        table[s, :nb] = perm[pos:pos + nb]
        pos += nb
    return table


def valid_slots(table, lens, num_blocks, block_size, skip_last=None):
    """[NB, B] bool: True where a valid token of some sequence sits."""
    mask = np.zeros((num_blocks, block_size), dtype=bool)
    for s, n in enumerate(lens):
        n = int(n) - (0 if skip_last is None else int(skip_last[s]))
        if n <= 0:
            continue
        nb = (n + block_size - 1) // block_size
        mask[table[s, :nb - 1]] = True
        mask[table[s, nb - 1], :n - (nb - 1) * block_size] = True
    return mask


def fill_pool(rng, table, lens, num_blocks, block_size, hkv, d, dtype, poison, skip_last=None):
    """Random K and V for the whole pool; with ``poison`` every slot that holds
    no valid token is then set to NaN.

    ``skip_last[s] = m`` treats the last ``m`` valid tokens of sequence s as
    not yet written (they arrive later through cache_write)."""
    shape = (num_blocks, block_size, hkv, d)
    k = randn(rng, shape, dtype)
    v = randn(rng, shape, dtype)
    if poison:
        bad = ~valid_slots(table, lens, num_blocks, block_size, skip_last)
        k[bad] = nan_fill((1, hkv, d), dtype)
        v[bad] = nan_fill((1, hkv, d), dtype)
    return k, v


def slots_of(table_row, positions, block_size):
    positions = np.asarray(positions, dtype=np.int64)
    return (table_row[positions // block_size].astype(np.int64) * block_size
            + positions % block_size).astype(np.int32)


# --------------------------------------------------------------------------
# the five workloads


def config1(seed=101, poison=True) -> Paged:
    """Tiny fp32 batch: 4 seqs, 8/8 heads, D 64, B 16, n ~ U{1..100}, pool 64.

    Tokens 0..n-2 are in the pool; token n-1 of each sequence arrives as
    k_new/v_new with its slot in slot_mapping, to be written before decode."""
    rng = np.random.default_rng(seed)
    S, H, D, B, NB = 4, 8, 64, 16, 64
    lens = rng.integers(1, 101, size=S).astype(np.int32)
    table = place(rng, lens, B, NB, mbs=7)
    k, v = fill_pool(rng, table, lens, NB, B, H, D, "f32", poison, skip_last=[1] * S)
    q = randn(rng, (S, H, D), "f32")
    k_new = randn(rng, (S, H, D), "f32")
    v_new = randn(rng, (S, H, D), "f32")
    slot = np.array([slots_of(table[s], [lens[s] - 1], B)[0] for s in range(S)], dtype=np.int32)
    return Paged("f32", q, k, v, table, lens, 1.0 / math.sqrt(D), B, 0,
                 k_new=k_new, v_new=v_new, slot_mapping=slot, name="c1-tiny-f32")


def lognormal_lengths(rng, mean, count, sigma=1.0, lo=1, hi=1024):
    mu = math.log(mean) - sigma * sigma / 2.0
    x = rng.lognormal(mu, sigma, size=count)
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def config2_lens(seed=202, S=64):
    rng = np.random.default_rng(seed)
    p = lognormal_lengths(rng, 220.0, S)
    g = lognormal_lengths(rng, 204.0, S)
    return (p + g).astype(np.int32), rng


def config2(seed=202, poison=False, S=64) -> Paged:
    """OPT-13B-shaped layer, fp16: 64 seqs, 40/40 heads, D 128, B 16.

    n = prompt + generated, each lognormal (means 220 and 204, sigma 1,
    rounded, clipped to [1, 1024]); pool sized to fit, blocks permuted."""
    lens, rng = config2_lens(seed, S)
    H, D, B, MBS = 40, 128, 16, 128
    NB = int(sum((int(n) + B - 1) // B for n in lens))
    table = place(rng, lens, B, NB, mbs=MBS)
    k, v = fill_pool(rng, table, lens, NB, B, H, D, "f16", poison)
    q = randn(rng, (S, H, D), "f16")
    return Paged("f16", q, k, v, table, lens, 1.0 / math.sqrt(D), B, 0, name="c2-opt13b-f16")


def config3(batch, ctx, seed=303, with_dense=True) -> Paged:
    """Contiguous-vs-paged sweep point, fp16, 40/40 heads, D 128.

    The dense [S, n, 40, 128] buffers are cut into 16-token blocks; block i of
    the flattened (seq, block) order is stored at pool id pi(i), so the paged
    pool holds exactly the dense values, scattered."""
    rng = np.random.default_rng(seed + 7919 * batch + ctx)
    H, D, B = 40, 128, 16
    assert ctx % B == 0
    k_dense = randn(rng, (batch, ctx, H, D), "f16")
    v_dense = randn(rng, (batch, ctx, H, D), "f16")
    nb_seq = ctx // B
    NB = batch * nb_seq
    perm = rng.permutation(NB).astype(np.int32)
    table = perm.reshape(batch, nb_seq).copy()
    k = np.empty((NB, B, H, D), dtype=np.float16)
    v = np.empty((NB, B, H, D), dtype=np.float16)
    k[perm] = k_dense.reshape(NB, B, H, D)
    v[perm] = v_dense.reshape(NB, B, H, D)
    q = randn(rng, (batch, H, D), "f16")
    lens = np.full(batch, ctx, dtype=np.int32)
    return Paged("f16", q, k, v, table, lens, 1.0 / math.sqrt(D), B, 0,
                 k_dense=k_dense if with_dense else None,
                 v_dense=v_dense if with_dense else None,
                 name=f"c3-sweep-f16-b{batch}-n{ctx}")


CONFIG3_POINTS = [(b, n) for b in (8, 32, 128) for n in (64, 256, 1024, 2048)]


@dataclasses.dataclass
class BeamScenario:
    """Config 4: 16 prompts x 6 beams sharing a 512-token prompt.

    Before decode: ``block_pairs`` (copy-on-write of each group's shared,
    partly filled stem block for 5 of its 6 beams; the sixth writes in place),
    then ``slot_mapping``/``k_new``/``v_new`` (every beam's private suffix)."""

    paged: Paged            # k_cache/v_cache hold the state BEFORE copy and write
    groups: int
    beams: int
    prompt_len: int
    stem: np.ndarray        # t0 per group
    suffix: np.ndarray      # s_b per beam
    prompt_blocks: np.ndarray   # [groups, 32]
    stem_block: np.ndarray      # [groups]
    blocks_in_use: int


def config4(seed=404, poison=True, groups=16, beams=6, prompt_len=512, NB=2048) -> BeamScenario:
    rng = np.random.default_rng(seed)
    H, D, B = 40, 128, 16
    dt = "f16"
    P = prompt_len // B
    stem = rng.integers(1, B, size=groups)                 # t0 in [1, 15]
    suffix = rng.integers(1, 201, size=groups * beams)     # s_b in [1, 200]
    free = list(rng.permutation(NB).astype(np.int32))[::-1]  # pop() from the end

    def alloc():
        return free.pop()

    S = groups * beams
    lens = np.zeros(S, dtype=np.int32)
    for gi in range(groups):
        for bi in range(beams):
            lens[gi * beams + bi] = prompt_len + stem[gi] + suffix[gi * beams + bi]
    MBS = int((lens.max() + B - 1) // B)
    table = np.full((S, MBS), -1, dtype=np.int32)
    prompt_blocks = np.zeros((groups, P), dtype=np.int32)
    stem_block = np.zeros(groups, dtype=np.int32)
    for gi in range(groups):
        for j in range(P):
            prompt_blocks[gi, j] = alloc()
        stem_block[gi] = alloc()
    shape = (NB, B, H, D)
    k = nan_fill(shape, dt) if poison else randn(rng, shape, dt)
    v = nan_fill(shape, dt) if poison else randn(rng, shape, dt)
    for gi in range(groups):
        k[prompt_blocks[gi]] = randn(rng, (P, B, H, D), dt)
        v[prompt_blocks[gi]] = randn(rng, (P, B, H, D), dt)
        k[stem_block[gi], :stem[gi]] = randn(rng, (stem[gi], H, D), dt)
        v[stem_block[gi], :stem[gi]] = randn(rng, (stem[gi], H, D), dt)
    pairs = []
    slots = []
    for gi in range(groups):
        t0 = int(stem[gi])
        for bi in range(beams):
            s = gi * beams + bi
            table[s, :P] = prompt_blocks[gi]
            if bi < beams - 1:       # copy-on-write: refcount > 1 at its first write
                dst = alloc()
                pairs.append((int(stem_block[gi]), int(dst)))
                table[s, P] = dst
            else:                    # the last writer is the sole owner: in place
                table[s, P] = stem_block[gi]
            n = int(lens[s])
            for j in range(P + 1, (n + B - 1) // B):
                table[s, j] = alloc()
            slots.append(slots_of(table[s], np.arange(prompt_len + t0, n), B))
    slot_mapping = np.concatenate(slots).astype(np.int32)
    N = slot_mapping.shape[0]
    k_new = randn(rng, (N, H, D), dt)
    v_new = randn(rng, (N, H, D), dt)
    q = randn(rng, (S, H, D), dt)
    paged = Paged(dt, q, k, v, table, lens, 1.0 / math.sqrt(D), B, 0,
                  k_new=k_new, v_new=v_new, slot_mapping=slot_mapping,
                  block_pairs=np.array(pairs, dtype=np.int32).reshape(-1, 2),
                  name="c4-beams-cow-f16")
    return BeamScenario(paged, groups, beams, prompt_len, stem, suffix, prompt_blocks,
                        stem_block, NB - len(free))


def random_shared(seed, dtype, groups, hq, hkv, d, block_size=16, extra_blocks=3):
    """Seeded decode batch whose sequences come in groups that share leading
    blocks (parallel samples or beams after a fork): ``groups`` =
    [(shared_blocks, [member context lengths]), ...] in batch order.  The
    members of a group name the same physical blocks in their first
    shared_blocks table entries, then blocks of their own; every block sits
    at a seeded place in the pool.  Shared blocks are filled whole (they hold
    a prefix every member has computed); a member's own blocks only up to
    its length, the rest of the pool is NaN.  Returns (Paged, group_start
    [G + 1], group_shared [G]) as int32 arrays."""
    rng = np.random.default_rng(seed)
    B = block_size
    lens = [int(n) for _, ms in groups for n in ms]
    S = len(lens)
    mbs = max(1, max(max(sb, max((int(n) + B - 1) // B for n in ms)) for sb, ms in groups))
    need = sum(sb + sum(max(0, (int(n) + B - 1) // B - sb) for n in ms) for sb, ms in groups)
    NB = need + extra_blocks
    ids = iter(rng.permutation(NB).astype(np.int32))
    table = np.full((S, mbs), -1, dtype=np.int32)
    k = nan_fill((NB, B, hkv, d), dtype)
    v = nan_fill((NB, B, hkv, d), dtype)
    starts, shared = [0], []
    s = 0
    for sb, ms in groups:
        common = [int(next(ids)) for _ in range(sb)]
        for b in common:
            k[b] = randn(rng, (B, hkv, d), dtype)
            v[b] = randn(rng, (B, hkv, d), dtype)
        for n in ms:
            table[s, :sb] = common
            for j in range(sb, (int(n) + B - 1) // B):
                b = int(next(ids))
                table[s, j] = b
                fill = min(B, int(n) - j * B)
                k[b, :fill] = randn(rng, (fill, hkv, d), dtype)
                v[b, :fill] = randn(rng, (fill, hkv, d), dtype)
            s += 1
        starts.append(s)
        shared.append(sb)
    q = randn(rng, (S, hq, d), dtype)
    p = Paged(dtype, q, k, v, table, np.array(lens, dtype=np.int32), 1.0 / math.sqrt(d), B, 0,
              name=f"shared-{dtype}-s{seed}")
    return p, np.array(starts, dtype=np.int32), np.array(shared, dtype=np.int32)


def config4_groups(sc: "BeamScenario"):
    """Config 4's sharing as groups: each prompt's beams, sharing its 512-token
    prompt (32 blocks; the partly filled stem block is copied on write)."""
    starts = np.arange(0, (sc.groups + 1) * sc.beams, sc.beams, dtype=np.int32)
    shared = np.full(sc.groups, sc.prompt_len // sc.paged.block_size, dtype=np.int32)
    return starts, shared


CONFIG5_LENS = (4096, 10000, 12000, 16384)


def config5(seed=505, poison=False, mixed=True, uniform_len=None) -> Paged:
    """Qwen2.5-1.5B-shaped GQA, bf16: 12 q heads / 2 kv heads, D 128, B 16,
    split-K over 512-token partitions.  Mixed batch: two sequences at each of
    4096/10000/12000/16384 tokens, seeded order; uniform: 8 x ``uniform_len``."""
    rng = np.random.default_rng(seed if uniform_len is None else seed + uniform_len)
    Hq, Hkv, D, B, MBS = 12, 2, 128, 16, 1024
    if uniform_len is None:
        lens = np.array(CONFIG5_LENS * 2, dtype=np.int32)
        rng.shuffle(lens)
    else:
        lens = np.full(8, uniform_len, dtype=np.int32)
    NB = int(sum((int(n) + B - 1) // B for n in lens))
    table = place(rng, lens, B, NB, mbs=MBS)
    k, v = fill_pool(rng, table, lens, NB, B, Hkv, D, "bf16", poison)
    q = randn(rng, (len(lens), Hq, D), "bf16")
    return Paged("bf16", q, k, v, table, lens, 1.0 / math.sqrt(D), B, 512,
                 name="c5-gqa-long-bf16" + ("" if uniform_len is None else f"-n{uniform_len}"))


# --------------------------------------------------------------------------
# small generic batches for edge cases


def random_paged(seed, dtype, lens, hq, hkv, d, block_size=16, extra_blocks=3,
                 mbs=None, poison=True, partition_size=0, scale=None) -> Paged:
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    need = int(sum((int(n) + block_size - 1) // block_size for n in lens))
    NB = max(1, need + extra_blocks)
    if mbs is None:
        mbs = max(1, max(((int(n) + block_size - 1) // block_size for n in lens), default=1))
    table = place(rng, lens, block_size, NB, mbs=mbs)
    k, v = fill_pool(rng, table, lens, NB, block_size, hkv, d, dtype, poison)
    q = randn(rng, (len(lens), hq, d), dtype)
    return Paged(dtype, q, k, v, table, lens,
                 (1.0 / math.sqrt(d)) if scale is None else scale, block_size,
                 partition_size, name=f"rand-{dtype}-s{seed}")


def random_with_dense(seed, dtype, lens, hq, hkv, d, block_size=16, smax=None,
                      extra_blocks=3, poison=True) -> Paged:
    """Ragged batch drawn in the dense layout [S, Smax, Hkv, D] (NaN beyond n
    when ``poison``), then placed block by block into a permuted pool, so the
    paged and dense inputs hold the same values."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    S, B = len(lens), block_size
    smax = smax or max(1, int(lens.max(initial=0)))
    shape = (S, smax, hkv, d)
    kd = nan_fill(shape, dtype) if poison else randn(rng, shape, dtype)
    vd = nan_fill(shape, dtype) if poison else randn(rng, shape, dtype)
    for s in range(S):
        n = int(lens[s])
        kd[s, :n] = randn(rng, (n, hkv, d), dtype)
        vd[s, :n] = randn(rng, (n, hkv, d), dtype)
    need = int(sum((int(n) + B - 1) // B for n in lens))
    NB = max(1, need + extra_blocks)
    mbs = max(1, max(((int(n) + B - 1) // B for n in lens), default=1))
    table = place(rng, lens, B, NB, mbs=mbs)
    pshape = (NB, B, hkv, d)
    k = nan_fill(pshape, dtype) if poison else randn(rng, pshape, dtype)
    v = nan_fill(pshape, dtype) if poison else randn(rng, pshape, dtype)
    for s in range(S):
        n = int(lens[s])
        for j in range((n + B - 1) // B):
            rows = min(B, n - j * B)
            k[table[s, j], :rows] = kd[s, j * B:j * B + rows]
            v[table[s, j], :rows] = vd[s, j * B:j * B + rows]
    q = randn(rng, (S, hq, d), dtype)
    return Paged(dtype, q, k, v, table, lens, 1.0 / math.sqrt(d), B, 0,
                 k_dense=kd, v_dense=vd, name=f"ragged-dense-{dtype}-s{seed}")


def config3_device(batch, ctx, seed=303, device="cuda"):
    """Config 3 point generated on the device (torch's Philox generator), for
    sizes whose host generation would take minutes.  Same structure as
    ``config3``: dense [S, n, 40, 128] fp16 values, cut into 16-token blocks,
    block i stored at pool id pi(i) (numpy PCG64 permutation).  Returns a dict
    of device tensors."""
    import torch

    H, D, B = 40, 128, 16
    assert ctx % B == 0
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + batch * 7919 + ctx)
    shape = (batch, ctx, H, D)
    k_dense = torch.randn(shape, generator=g, device=device, dtype=torch.float32).half()
    v_dense = torch.randn(shape, generator=g, device=device, dtype=torch.float32).half()
    q = torch.randn((batch, H, D), generator=g, device=device, dtype=torch.float32).half()
    NB = batch * ctx // B
    perm = np.random.default_rng(seed + 7919 * batch + ctx).permutation(NB).astype(np.int64)
    pt = torch.from_numpy(perm).to(device)
    k = torch.empty((NB, B, H, D), dtype=torch.float16, device=device)
    v = torch.empty_like(k)
    k[pt] = k_dense.view(NB, B, H, D)
    v[pt] = v_dense.view(NB, B, H, D)
    table = pt.to(torch.int32).view(batch, ctx // B).contiguous()
    lens = torch.full((batch,), ctx, dtype=torch.int32, device=device)
    return dict(q=q, k_cache=k, v_cache=v, block_tables=table, context_lens=lens,
                k_dense=k_dense, v_dense=v_dense, scale=1.0 / math.sqrt(D))


@dataclasses.dataclass
class Prefill:
    """Multi-token queries over a paged cache: sequence s owns query rows
    query_start[s] .. query_start[s+1]-1, the last chunk_lens[s] of its
    context_lens[s] cached tokens (their K/V already in the pool)."""
    dtype: str
    q: np.ndarray               # [rows, Hq, D]
    k_cache: np.ndarray         # [NB, B, Hkv, D] token-major
    v_cache: np.ndarray
    block_tables: np.ndarray    # [S, MBS] int32
    context_lens: np.ndarray    # [S] int32
    query_start: np.ndarray     # [S + 1] int32
    scale: float
    block_size: int
    name: str = ""

    @property
    def chunk_lens(self):
        return np.diff(self.query_start).astype(np.int32)


def random_prefill(seed, dtype, ctx_lens, chunk_lens, hq, hkv, d, block_size=16,
                   extra_blocks=3, poison=True, scale=None) -> Prefill:
    """Seeded pool and queries for a batch of chunks: placement and pool as
    random_paged, then one N(0,1) query row per chunk token."""
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    chunk_lens = np.asarray(chunk_lens, dtype=np.int32)
    assert np.all(chunk_lens <= ctx_lens) and np.all(chunk_lens >= 0)
    p = random_paged(seed, dtype, ctx_lens, hq, hkv, d, block_size=block_size,
                     extra_blocks=extra_blocks, poison=poison, scale=scale)
    rng = np.random.default_rng(seed + 7919)
    qs = np.zeros(len(chunk_lens) + 1, dtype=np.int32)
    qs[1:] = np.cumsum(chunk_lens)
    q = randn(rng, (int(qs[-1]), hq, d), dtype)
    return Prefill(dtype, q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, qs, p.scale,
                   block_size, name=f"prefill-{dtype}-s{seed}")
