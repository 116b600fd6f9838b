"""Mutation check of the oracle's pins (CPU only).

Each mutant plants one plausible mistake in a copy of oracle/moonep_oracle.py (a source
edit applied to the text, loaded as a separate module; the real oracle is untouched) and
runs the pins of tests/test_oracle.py against it.  Every mutant must fail at least one pin:
a pin set that a dropped term, a wrong sign, index or order, or a transposed operand could
pass unnoticed would not be pinning the oracle.  The unmutated copy must pass them all.
"""

import os
import types

import pytest

from tests import adversarial
from tests import test_oracle as TO
from gen import TINY, SMALL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "moonep_oracle.py")).read()

# (name, text in the oracle, replacement)
MUTANTS = [
    ("tie order by id descending",
     "key=lambda e: (-int(load[e]), e)", "key=lambda e: (-int(load[e]), -e)"),
    ("shed the whole remaining excess, ignoring the expert's load",
     "shed[e] = min(load[e], x_left[h])", "shed[e] = x_left[h]"),
    ("highest-id receiver first",
     "r = with_slot[0]", "r = with_slot[-1]"),
    ("groups not aligned",
     "off[r, g + 1] = align_up(off[r, g] + group_size[r, g])",
     "off[r, g + 1] = off[r, g] + group_size[r, g]"),
    ("padding sized for home groups only",
     "return align_up(self.C + self.G * (ROW_ALIGN - 1))",
     "return align_up(self.C + self.E_loc * (ROW_ALIGN - 1))"),
    ("fallback pieces all start at the region's first row",
     "fbpos = int(fb_rows[r])", "fbpos = 0"),
    ("piece start not advanced",
     "            rem -= cnt\n            start += cnt\n", "            rem -= cnt\n"),
    ("combine sums k in reverse",
     "    for k in range(K):\n        rows = bf16_to_f32(y_bits[dst_row[:, k]])",
     "    for k in reversed(range(K)):\n        rows = bf16_to_f32(y_bits[dst_row[:, k]])"),
    ("reduce reads slot 0 for every replica",
     "home[e] = (home[e] + rep[r, slot]).astype(np.float32)",
     "home[e] = (home[e] + rep[r, 0]).astype(np.float32)"),
    ("bf16 by truncation",
     "rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)",
     "rounded = (u >> np.uint32(16)).astype(np.uint16)"),
    ("home experts laid out in reverse",
     "home_row0 = h * sz.NvS + p.off[h, e - h * sz.E_loc]",
     "home_row0 = h * sz.NvS + p.off[h, sz.E_loc - 1 - (e - h * sz.E_loc)]"),
    ("combine weights every k with column 0",
     "prod = (w[:, k:k + 1] * rows).astype(np.float32)",
     "prod = (w[:, 0:1] * rows).astype(np.float32)"),
    ("slot map ranks an expert's assignments in decreasing i",
     'by_expert = np.argsort(flat, kind="stable")',
     "by_expert = np.lexsort((-np.arange(flat.size), flat))"),
    ("dispatch copies token i % T instead of i // K",
     "src = np.repeat(np.arange(T), K)", "src = np.tile(np.arange(T), K)"),
    ("slot budget ignored (every receiver always has a free slot)",
     "with_slot = [r for r in range(R) if d_left[r] > 0 and used[r] < slots]",
     "with_slot = [r for r in range(R) if d_left[r] > 0]"),
    ("combine accumulates products in bf16 instead of fp32",
     "        acc = (acc + prod).astype(np.float32)",
     "        acc = bf16_to_f32(f32_to_bf16_rne((acc + prod).astype(np.float32)))"),
]


def _module(src, name):
    m = types.ModuleType(name)
    m.__file__ = os.path.join(ROOT, "oracle", "moonep_oracle.py")
    exec(compile(src, m.__file__, "exec"), m.__dict__)
    return m


def _pins():
    """(label, callable) for the pins of tests/test_oracle.py that run in about a second."""
    pins = [("golden " + n, lambda n=n: TO.test_golden_full_examples(n))
            for n in ("plan_r2_e4_k2_s4.json", "plan_r3_e6_fallback.json")]
    pins += [("golden slot exhaustion", TO.test_golden_slot_exhaustion)]
    pins += [(f"unit-step and merge, seed {s}", lambda s=s: TO.test_unit_step_and_merge_agree(s))
             for s in range(6)]
    pins += [(f"adversarial {c[0]}", lambda c=c: TO.test_adversarial_routings(c))
             for c in adversarial.routings()[:4]]
    pins += [("balanced and single rank", TO.test_balanced_and_single_rank_have_no_pieces),
             ("dispatch -> no-op -> combine", TO.test_dispatch_noop_combine_is_identity),
             ("combine closed form", TO.test_combine_equals_no_replication_closed_form),
             ("reduce closed form, several slots", TO.test_reduce_exercises_several_slots_per_rank),
             ("combine rounding golden", TO.test_combine_rounding_golden),
             ("bf16 against torch", TO.test_bf16_rne_matches_torch),
             ("workload tiny", lambda: TO.test_workload_plans(TINY, 0)),
             ("workload r8-e64-k6", lambda: TO.test_workload_plans(SMALL, 0))]
    return pins


def _run_pins(module, monkeypatch):
    """Labels of the pins that fail with `module` standing in for the oracle."""
    monkeypatch.setattr(TO, "O", module)
    failed = []
    for label, fn in _pins():
        try:
            fn()
        except Exception:          # an assertion, or the mutant breaking its own checks
            failed.append(label)
    return failed


def test_unmutated_copy_passes_every_pin(monkeypatch):
    assert _run_pins(_module(SRC, "oracle_copy"), monkeypatch) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, monkeypatch):
    assert SRC.count(old) == 1, f"mutation site not found exactly once: {old!r}"
    failed = _run_pins(_module(SRC.replace(old, new), "oracle_mutant"), monkeypatch)
    assert failed, f"no pin catches the mutant: {name}"
