"""The public headers are plain C: a C99 program that includes both,
compiled by gcc with warnings as errors and linked against libpa.so, drives
the host block manager through a copy-on-write fork and a swap and checks
the argument checks of the device entry points (no GPU call is made)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "paged_kv_cache_pa_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "pa.h"
#include "pa_block_manager.h"

#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); return 1; } } while (0)

int main(void) {
    pa_bm *bm = NULL;
    int32_t seq, child, n_pairs, nt, nb, where, gfree, cfree, refs;
    int32_t slots[64], pairs[16], table[8], lens[2], tables[16];
    CHECK(pa_bm_create(8, 4, 4, NULL, &bm) == PA_OK);
    CHECK(pa_bm_new_seq(bm, &seq) == PA_OK && seq == 0);
    /* 6 tokens at block size 4: blocks 0 and 1 (ascending free order) */
    int32_t six = 6;
    CHECK(pa_bm_reserve(bm, &seq, &six, 1, slots, 16, pairs, 8, &n_pairs) == PA_OK);
    CHECK(n_pairs == 0);
    for (int i = 0; i < 6; ++i) CHECK(slots[i] == i);
    /* a fork shares both blocks; the child's next token copies the shared,
       partly filled last block first */
    CHECK(pa_bm_fork(bm, seq, &child) == PA_OK && child == 1);
    CHECK(pa_bm_ref_count(bm, 1, 0, &refs) == PA_OK && refs == 2);
    int32_t one = 1;
    CHECK(pa_bm_reserve(bm, &child, &one, 1, slots, 16, pairs, 8, &n_pairs) == PA_OK);
    CHECK(n_pairs == 1 && pairs[0] == 1 && pairs[1] == 2 && slots[0] == 2 * 4 + 2);
    int32_t both[2] = {0, 1};
    CHECK(pa_bm_tables(bm, both, 2, tables, 8, lens) == PA_OK);
    CHECK(lens[0] == 6 && lens[1] == 7 && tables[0] == 0 && tables[1] == 1 && tables[2] == -1);
    CHECK(tables[8] == 0 && tables[9] == 2);
    /* swap the two out and back: 3 distinct blocks move, sharing kept */
    CHECK(pa_bm_swap_out(bm, both, 2, pairs, 8, &n_pairs) == PA_OK && n_pairs == 3);
    CHECK(pa_bm_seq_info(bm, 1, &nt, &nb, &where) == PA_OK && where == PA_SEQ_SWAPPED);
    CHECK(pa_bm_num_free(bm, &gfree, &cfree) == PA_OK && gfree == 8 && cfree == 1);
    CHECK(pa_bm_swap_in(bm, both, 2, pairs, 8, &n_pairs) == PA_OK && n_pairs == 3);
    CHECK(pa_bm_block_table(bm, 1, table, 8) == PA_OK);
    CHECK(pa_bm_ref_count(bm, table[0], 0, &refs) == PA_OK && refs == 2);
    /* all-or-nothing: 40 more tokens need more blocks than the pool holds */
    int32_t forty = 40;
    CHECK(pa_bm_reserve(bm, &seq, &forty, 1, slots, 64, pairs, 8, &n_pairs) == PA_ERR_NO_BLOCKS);
    CHECK(pa_bm_reserve(bm, &seq, &forty, 1, slots, 16, pairs, 8, &n_pairs) == PA_ERR_SHAPE);
    CHECK(pa_bm_seq_info(bm, 0, &nt, &nb, &where) == PA_OK && nt == 6 && nb == 2);
    CHECK(pa_bm_free(bm, both, 2) == PA_OK);
    CHECK(pa_bm_num_free(bm, &gfree, &cfree) == PA_OK && gfree == 8 && cfree == 4);
    pa_bm_destroy(bm);

    /* device entry points: host-side checks only */
    pa_decode_params p;
    memset(&p, 0, sizeof p);
    p.num_seqs = 2; p.num_q_heads = 8; p.num_kv_heads = 2; p.head_dim = 128;
    p.block_size = 16; p.max_blocks_per_seq = 4; p.num_blocks = 8; p.max_context_len = 64;
    p.partition_size = 16; p.dtype = PA_F16; p.layout = 0;
    size_t bytes = 0;
    CHECK(pa_decode_workspace_size(&p, &bytes) == PA_OK);
    CHECK(bytes == (size_t)2 * 8 * 4 * (128 + 2) * 4);
    p.head_dim = 96;
    CHECK(pa_decode(NULL, NULL, NULL, NULL, NULL, 1.0f, NULL, &p, NULL, 0, NULL) != PA_OK);
    CHECK(strlen(pa_status_string(PA_ERR_SHAPE)) > 0);
    CHECK(strlen(pa_build_info()) > 0);
    printf("ok\n");
    return 0;
}
"""


def test_headers_compile_as_c_and_drive_the_block_manager(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    lib = os.path.join(LIB_DIR, "libpa.so")
    if not os.path.exists(lib):
        pytest.skip("libpa.so is not built")
    src = tmp_path / "use_pa.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_pa"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", LIB_DIR, "-lpa", f"-Wl,-rpath,{LIB_DIR}",
           "-Wl,--allow-shlib-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
