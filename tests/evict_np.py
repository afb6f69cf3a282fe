"""A second, independent implementation of the capped eviction, in numpy.

TEST INFRASTRUCTURE ONLY.  It exists to pin the C oracle's eviction: the two
are written separately (this one finds resident top-K members through the slot
map with set membership, orders victims with np.lexsort and applies the
admissions with array assignments; the oracle walks the top-K list through the
block map and sorts with qsort) and must agree bit for bit.

The rule (pith.science paper page, "What carries the argument": at most
cap*K admissions per step, each admitted non-resident block paired with a
least-recently-selected resident block), in the readings this project takes:
  - a block is selected at step t when it is in that step's top-K list; the
    slots holding such blocks are stamped t first, so no victim is selected;
  - the misses are admitted in top-K order, at most max_admit of them;
  - victims are the empty slots (slot order), then the slots whose stamp is
    older than t, least recently selected first (stamp ascending, ties by
    block index ascending).
"""
from __future__ import annotations

import numpy as np


def capped_evict_unit(T, step, max_admit, l2p, p2l, last_sel):
    """One unit.  T [K] top-K list (-1 unused), l2p [NB], p2l [K], last_sel [K].
    Returns new (l2p, p2l, last_sel, admit [K][3], count); inputs unchanged."""
    T = np.asarray(T, np.int64)
    l2p = np.array(l2p, np.int32)
    p2l = np.array(p2l, np.int32)
    ls = np.array(last_sel, np.int32)
    K = p2l.shape[0]
    sel = T[T >= 0]

    held = p2l >= 0
    in_top = held & np.isin(p2l, sel)
    ls[in_top] = step

    resident = set(p2l[held].tolist())
    misses = np.array([j for j in sel.tolist() if j not in resident], np.int64)

    empty = np.flatnonzero(~held)
    stale = np.flatnonzero(held & (ls < step))
    stale = stale[np.lexsort((p2l[stale], ls[stale]))]   # last key sorts first
    victims = np.concatenate([empty, stale]).astype(np.int64)

    a = int(max(0, min(max_admit, misses.size, victims.size)))
    admit = np.full((K, 3), -1, np.int32)
    slots = victims[:a]
    evicted = p2l[slots].copy()
    l2p[evicted[evicted >= 0]] = -1
    p2l[slots] = misses[:a]
    l2p[misses[:a]] = slots
    ls[slots] = step
    admit[:a, 0] = misses[:a]
    admit[:a, 1] = slots
    admit[:a, 2] = evicted
    return l2p, p2l, ls, admit, a


def capped_evict(T, step, max_admit, l2p, p2l, last_sel):
    """All units: T [B][H][K], l2p [B][H][NB], p2l and last_sel [B][H][K].
    Returns new (l2p, p2l, last_sel, admit [B][H][K][3], count [B][H])."""
    T = np.asarray(T)
    B, H, K = np.asarray(p2l).shape
    out_l2p = np.array(l2p, np.int32)
    out_p2l = np.array(p2l, np.int32)
    out_ls = np.array(last_sel, np.int32)
    admit = np.full((B, H, K, 3), -1, np.int32)
    count = np.zeros((B, H), np.int32)
    for b in range(B):
        for h in range(H):
            r = capped_evict_unit(T[b, h], step, max_admit, out_l2p[b, h], out_p2l[b, h],
                                  out_ls[b, h])
            out_l2p[b, h], out_p2l[b, h], out_ls[b, h], admit[b, h], count[b, h] = r
    return out_l2p, out_p2l, out_ls, admit, count
