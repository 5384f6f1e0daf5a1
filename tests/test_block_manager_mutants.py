"""Plant a mistake in a copy of the block-manager model (on the CPU) and
check that the pins in test_block_manager.py catch it.  Each mutant is a
one-line textual change of oracle/block_manager.py, loaded as a separate
module; the pins then run against the mutated class."""
from __future__ import annotations

import os
import random
import types

import pytest

import oracle.block_manager as OBM
import test_block_manager as T

SRC = OBM.__file__

# (name, original text, planted text)
MUTANTS = [
    ("copy_always", 'if s["n"] % B != 0 and self.refs["gpu"][s["table"][-1]] > 1:',
     'if s["n"] % B != 0 and self.refs["gpu"][s["table"][-1]] >= 1:'),
    ("copy_never", 'if s["n"] % B != 0 and self.refs["gpu"][s["table"][-1]] > 1:',
     'if s["n"] % B != 0 and self.refs["gpu"][s["table"][-1]] > 10**9:'),
    ("copy_full_block_too", 'if s["n"] % B != 0 and self.refs["gpu"][s["table"][-1]] > 1:',
     'if s["n"] > 0 and self.refs["gpu"][s["table"][-1]] > 1:'),
    ("fork_without_reference", 'self.refs["gpu"][b] += 1', 'self.refs["gpu"][b] += 0'),
    ("release_never_frees", "self.free[side].append(b)", "pass"),
    ("slot_transposed", "slots.append(s[\"table\"][t // B] * B + t % B)",
     "slots.append(s[\"table\"][t % len(s[\"table\"])] * B + t % B)"),
    ("one_block_too_many", 'while len(s["table"]) * B < s["n"] + k:',
     'while len(s["table"]) * B <= s["n"] + k:'),
    ("allocate_from_bottom", "b = self.free[side].pop()", "b = self.free[side].pop(0)"),
    ("swap_refs_not_moved", "self.refs[dst][c] = uses[b]", "self.refs[dst][c] = 1"),
    ("old_block_kept_referenced", 'pairs.append((old, new))\n                    self._release("gpu", old)',
     'pairs.append((old, new))'),
]


def load_mutant(orig, planted):
    with open(SRC) as f:
        text = f.read()
    assert text.count(orig) == 1, f"mutation site not unique: {orig!r}"
    mod = types.ModuleType("mutant_block_manager")
    exec(compile(text.replace(orig, planted), "mutant_block_manager.py", "exec"), mod.__dict__)
    return mod


def run_pins(cls):
    """Every pin of test_block_manager.py with `cls` as the oracle.
    Returns the names of the pins that failed."""
    class Adapter(cls):
        def ref(self, side, b):
            return self.refs[side][b]

    saved = T.OracleAdapter, T.BMError
    T.OracleAdapter, T.BMError = Adapter, cls.__init__.__globals__["BMError"]
    failed = []
    pins = [
        ("fig6", lambda: T.test_fig6_slots("oracle")),
        ("flowchart", lambda: T.test_internals_flowchart("oracle")),
        ("cow_trace", lambda: T.test_internals_cow_trace("oracle")),
        ("four_samples", lambda: T.test_res_four_samples("oracle", True)),
        ("two_prompts", lambda: T.test_res_two_prompts("oracle")),
        ("fig9", lambda: T.test_kwon_fig9_beam_update("oracle")),
        ("swap_sharing", lambda: T.test_swap_keeps_sharing_inside_the_group("oracle")),
        ("replay", lambda: T.random_ops(T.Replay(Adapter(12, 6, 4)), random.Random(1), 300)),
    ]
    try:
        for name, f in pins:
            try:
                f()
            except Exception:
                failed.append(name)
    finally:
        T.OracleAdapter, T.BMError = saved
    return failed


def test_unmutated_model_passes_every_pin():
    assert run_pins(OBM.OracleBlockManager) == []


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, planted):
    mod = load_mutant(orig, planted)
    assert run_pins(mod.OracleBlockManager), f"mutant {name} passed every pin"
