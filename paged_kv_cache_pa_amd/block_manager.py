"""ctypes binding of the host KV block manager (``include/pa_block_manager.h``).

Argument marshalling only: every operation runs in the library's C++ code.
Arrays cross the boundary as numpy int32 buffers; a refused call raises
``PaError`` (its ``name`` is the pa_status name) and changes nothing.
"""
from __future__ import annotations

import ctypes

import numpy as np

__all__ = ["BlockManager", "declare"]

_I32 = ctypes.c_int32
_PI32 = ctypes.POINTER(ctypes.c_int32)


def declare(L):
    """Set the ctypes signatures of the pa_bm_* symbols on a loaded library."""
    P = ctypes.c_void_p
    sig = {
        "pa_bm_create": [_I32, _I32, _I32, P, ctypes.POINTER(P)],
        "pa_bm_new_seq": [P, _PI32],
        "pa_bm_fork": [P, _I32, _PI32],
        "pa_bm_free": [P, P, _I32],
        "pa_bm_reserve": [P, P, P, _I32, P, ctypes.c_int64, P, _I32, _PI32],
        "pa_bm_tables": [P, P, _I32, P, _I32, P],
        "pa_bm_swap_out": [P, P, _I32, P, _I32, _PI32],
        "pa_bm_swap_in": [P, P, _I32, P, _I32, _PI32],
        "pa_bm_num_free": [P, _PI32, _PI32],
        "pa_bm_ref_count": [P, _I32, _I32, _PI32],
        "pa_bm_seq_info": [P, _I32, _PI32, _PI32, _PI32],
        "pa_bm_block_table": [P, _I32, P, _I32],
        "pa_bm_free_list": [P, _I32, P, _I32, _PI32],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.pa_bm_destroy.argtypes = [P]
    L.pa_bm_destroy.restype = None


def _arr(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32).reshape(-1))
    return a, a.ctypes.data_as(ctypes.c_void_p)


class BlockManager:
    """One manager: a GPU block pool, a host swap pool, and the sequences."""

    def __init__(self, num_gpu_blocks: int, num_cpu_blocks: int, block_size: int,
                 gpu_free_order=None):
        from . import _check, lib

        self._L = lib()
        self._check = _check
        self._h = ctypes.c_void_p()
        order = None
        if gpu_free_order is not None:
            order, optr = _arr(gpu_free_order)
            if order.size != num_gpu_blocks:
                raise ValueError("gpu_free_order must list every block once")
        self._run("pa_bm_create", int(num_gpu_blocks), int(num_cpu_blocks), int(block_size),
                  None if order is None else optr, ctypes.byref(self._h))
        self.block_size = int(block_size)

    def _run(self, name, *args):
        self._check(getattr(self._L, name)(*args), name)

    def close(self):
        if self._h:
            self._L.pa_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- operations --------------------------------------------------------
    def new_seq(self) -> int:
        h = _I32()
        self._run("pa_bm_new_seq", self._h, ctypes.byref(h))
        return h.value

    def fork(self, parent: int) -> int:
        h = _I32()
        self._run("pa_bm_fork", self._h, int(parent), ctypes.byref(h))
        return h.value

    def free(self, seqs):
        a, p = _arr(seqs)
        self._run("pa_bm_free", self._h, p, a.size)

    def reserve(self, seqs, num_new):
        """Returns (slot_mapping [sum(num_new)], block_pairs [n_pairs, 2])."""
        s, sp = _arr(seqs)
        k, kp = _arr(num_new)
        if k.size != s.size:
            raise ValueError("one num_new per sequence")
        total = int(np.clip(k, 0, None).sum(dtype=np.int64))
        slots = np.empty(max(total, 1), np.int32)
        pairs = np.empty((max(s.size, 1), 2), np.int32)
        n = _I32()
        self._run("pa_bm_reserve", self._h, sp, kp, s.size,
                  slots.ctypes.data_as(ctypes.c_void_p), total,
                  pairs.ctypes.data_as(ctypes.c_void_p), s.size, ctypes.byref(n))
        return slots[:total], pairs[:n.value]

    def tables(self, seqs, max_blocks_per_seq: int):
        """Returns (block_tables [n, max_blocks_per_seq], context_lens [n])."""
        s, sp = _arr(seqs)
        bt = np.empty((max(s.size, 1), int(max_blocks_per_seq)), np.int32)
        cl = np.empty(max(s.size, 1), np.int32)
        self._run("pa_bm_tables", self._h, sp, s.size, bt.ctypes.data_as(ctypes.c_void_p),
                  int(max_blocks_per_seq), cl.ctypes.data_as(ctypes.c_void_p))
        return bt[:s.size], cl[:s.size]

    def _move(self, name, seqs):
        s, sp = _arr(seqs)
        cap = 0
        for h in s:
            cap += self.seq_info(int(h))[1]
        pairs = np.empty((max(cap, 1), 2), np.int32)
        n = _I32()
        self._run(name, self._h, sp, s.size, pairs.ctypes.data_as(ctypes.c_void_p), cap,
                  ctypes.byref(n))
        return pairs[:n.value]

    def swap_out(self, seqs):
        """Returns (gpu block, cpu block) pairs to copy device -> host."""
        return self._move("pa_bm_swap_out", seqs)

    def swap_in(self, seqs):
        """Returns (cpu block, gpu block) pairs to copy host -> device."""
        return self._move("pa_bm_swap_in", seqs)

    # -- observation -------------------------------------------------------
    def num_free(self):
        g, c = _I32(), _I32()
        self._run("pa_bm_num_free", self._h, ctypes.byref(g), ctypes.byref(c))
        return g.value, c.value

    def ref_count(self, block: int, on_cpu: bool = False) -> int:
        r = _I32()
        self._run("pa_bm_ref_count", self._h, int(block), int(bool(on_cpu)), ctypes.byref(r))
        return r.value

    def seq_info(self, seq: int):
        """(num_tokens, num_blocks, where) with where 0 = on GPU, 1 = swapped."""
        n, b, w = _I32(), _I32(), _I32()
        self._run("pa_bm_seq_info", self._h, int(seq), ctypes.byref(n), ctypes.byref(b),
                  ctypes.byref(w))
        return n.value, b.value, w.value

    def block_table(self, seq: int):
        nb = self.seq_info(seq)[1]
        t = np.empty(max(nb, 1), np.int32)
        self._run("pa_bm_block_table", self._h, int(seq), t.ctypes.data_as(ctypes.c_void_p), nb)
        return t[:nb].tolist()

    def free_list(self, on_cpu: bool = False):
        """The free stack, next-to-be-handed-out first."""
        g, c = self.num_free()
        cap = c if on_cpu else g
        ids = np.empty(max(cap, 1), np.int32)
        n = _I32()
        self._run("pa_bm_free_list", self._h, int(bool(on_cpu)),
                  ids.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(n))
        return ids[:n.value].tolist()
