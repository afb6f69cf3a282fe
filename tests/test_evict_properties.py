"""Property tests (hypothesis) of the oracle's capped eviction against the
independent numpy eviction and the invariants of the least-recently-selected
rule (pith.science paper page, "What carries the argument").  CPU only."""
import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import evict_np
import oracle
from test_oracle_pins import check_evict_invariants


@st.composite
def eviction_states(draw):
    K = draw(st.integers(1, 24))
    NB = draw(st.integers(1, 64))
    step = draw(st.integers(1, 10))
    n = draw(st.integers(0, min(K, NB)))
    blocks = draw(st.lists(st.integers(0, NB - 1), min_size=n, max_size=n, unique=True))
    slots = draw(st.permutations(list(range(K))))[:n]
    # stamps: mostly older than the step; sometimes equal or newer (never victims)
    stamp_hi = draw(st.sampled_from([step - 1, step + 1]))
    stamps = draw(st.lists(st.integers(0, max(0, stamp_hi)), min_size=K, max_size=K))
    top = draw(st.lists(st.integers(0, NB - 1), max_size=min(K, NB), unique=True))
    m = draw(st.integers(0, K + 1))
    l2p = np.full((1, 1, NB), -1, np.int32)
    p2l = np.full((1, 1, K), -1, np.int32)
    for s, j in zip(slots, blocks):
        p2l[0, 0, s] = j
        l2p[0, 0, j] = s
    ls = np.array(stamps, np.int32).reshape(1, 1, K)
    T = np.full((1, 1, K), -1, np.int32)
    T[0, 0, :len(top)] = top
    return T, step, m, l2p, p2l, ls


@settings(max_examples=400, deadline=None)
@given(eviction_states())
def test_oracle_eviction_equals_numpy_eviction(case):
    T, step, m, l2p, p2l, ls = case
    want = evict_np.capped_evict(T, step, m, l2p, p2l, ls)
    before = (l2p.copy(), p2l.copy(), ls.copy())
    admit, count = oracle.capped_evict(T, step, m, l2p, p2l, ls)
    for got, exp in zip((l2p, p2l, ls, admit, count), want):
        np.testing.assert_array_equal(got, exp)
    if np.all(before[2] < step):
        check_evict_invariants(T, step, m, before, (l2p, p2l, ls), admit, count)


@settings(max_examples=200, deadline=None)
@given(eviction_states(), st.integers(1, 6))
def test_repeated_steps_make_the_list_resident(case, extra):
    """With the same top-K list at every step, each step admits min(m, misses
    left) blocks and never evicts a listed block, so after ceil(|T|/m) steps
    the whole list is resident (m >= 1)."""
    T, step, m, l2p, p2l, ls = case
    m = max(1, m)
    ls = np.ascontiguousarray(np.minimum(ls, step - 1))     # every stamp older than the step
    listed = {int(j) for j in T[0, 0] if j >= 0}
    for t in range(step, step + len(listed) // m + extra + 1):
        missing = len(listed - {int(j) for j in p2l[0, 0] if j >= 0})
        _, count = oracle.capped_evict(T, t, m, l2p, p2l, ls)
        assert int(count[0, 0]) == min(m, missing)
    assert listed <= {int(j) for j in p2l[0, 0] if j >= 0}
