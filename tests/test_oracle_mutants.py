"""Mutation check of the eviction pins.

Each mutant below is a plausible mistake in the oracle's capped eviction,
planted in a copy of oracle.c (on the CPU) and built with gcc.  Every mutant
must fail at least one of the eviction pins (the hand-worked examples, the
independent numpy eviction, the invariants), and the unmodified source must
pass the same pins, so that a pin that cannot tell the least-recently-selected
rule (pith.science paper page, "What carries the argument") from its
neighbours is noticed here."""
import json
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")
SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

CMP_STAMP = "if (a->stamp != b->stamp) return a->stamp < b->stamp ? -1 : 1;"
CMP_BLOCK = "return (a->logical < b->logical) ? -1 : (a->logical > b->logical);"
STAMP_HITS = "if (s >= 0) LS[s] = step;"
EMPTIES = """        for (int s = 0; s < K; ++s)
            if (P2L[s] < 0) order[nv++] = s;
"""
STALE_TAIL = "        for (int r = 0; r < no; ++r) order[nv++] = old[r].slot;\n"

MUTANTS = {
    "most_recently_selected_first": [(CMP_STAMP, CMP_STAMP.replace("a->stamp < b->stamp",
                                                                    "a->stamp > b->stamp"))],
    "stamps_ignored": [(CMP_STAMP, "")],
    "ties_to_higher_block": [(CMP_BLOCK, "return (a->logical > b->logical) ? -1 : "
                                         "(a->logical < b->logical);")],
    "empty_slots_last": [(EMPTIES, ""), (STALE_TAIL, STALE_TAIL + EMPTIES)],
    "selected_blocks_not_stamped": [(STAMP_HITS, "if (s >= 0) (void)step;")],
}


def build_variant(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutant {name}: the oracle no longer holds {old!r}"
        src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    c.write_text(src)
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-shared", "-fPIC", "-I",
                           os.path.dirname(SRC), str(c), "-o", str(so), "-lpthread", "-lm"])
    return str(so)


def eviction_pins():
    """Runs the eviction pins against whatever oracle build is loaded; returns
    the names of the pins that fail."""
    import evict_np
    from test_oracle_pins import check_evict_invariants, random_evict_case

    failed = []
    for name in ("evict_worked_example.json", "evict_lrs_order_example.json"):
        g = json.load(open(os.path.join(GOLDEN, name)))
        p2l = np.array([[g["p2l_before"]]], np.int32)
        ls = np.array([[g["last_sel_before"]]], np.int32)
        l2p = np.full((1, 1, g["n_blocks"]), -1, np.int32)
        for s, j in enumerate(g["p2l_before"]):
            if j >= 0:
                l2p[0, 0, j] = s
        admit, count = oracle.capped_evict(np.array([[g["topk"]]], np.int32), g["step"],
                                           g["max_admit"], l2p, p2l, ls)
        if (p2l[0, 0].tolist() != g["p2l_after"] or ls[0, 0].tolist() != g["last_sel_after"]
                or l2p[0, 0].tolist() != g["l2p_after"] or admit[0, 0].tolist() != g["admit"]
                or int(count[0, 0]) != g["admit_count"]):
            failed.append(name)
    for seed in range(40):
        rng = np.random.default_rng(700 + seed)
        T, step, m, l2p, p2l, ls = random_evict_case(rng)
        want = evict_np.capped_evict(T, step, m, l2p, p2l, ls)
        before = (l2p.copy(), p2l.copy(), ls.copy())
        admit, count = oracle.capped_evict(T, step, m, l2p, p2l, ls)
        if not all(np.array_equal(a, b) for a, b in zip((l2p, p2l, ls, admit, count), want)):
            failed.append(f"numpy eviction, seed {seed}")
        if np.all(before[2] < step):
            try:
                check_evict_invariants(T, step, m, before, (l2p, p2l, ls), admit, count)
            except AssertionError:
                failed.append(f"invariants, seed {seed}")
    return failed


def with_library(path, fn):
    saved = oracle._lib
    oracle._lib = oracle.load(path)
    try:
        return fn()
    finally:
        oracle._lib = saved


def test_unmodified_oracle_passes_the_eviction_pins(tmp_path):
    so = build_variant(tmp_path, "unmodified", [])
    assert with_library(so, eviction_pins) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_eviction_mutant_fails_a_pin(tmp_path, name):
    so = build_variant(tmp_path, name, MUTANTS[name])
    failed = with_library(so, eviction_pins)
    print(name, "caught by", failed[:6])
    assert failed, f"no eviction pin tells the mutant '{name}' from the oracle"
