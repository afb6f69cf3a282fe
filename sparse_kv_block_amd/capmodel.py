"""Host-link budget of the look-ahead decode step.

The pages assume the prefetch traffic of a decode step hides inside the
step's overlap window (pith.science paper page, "Assumptions & free
parameters": the window C_token), and their fetch-cap ablation (agihunt.info
summary) shows the host link bounding the step once the cap lets more bytes
through than the window hides.  With every unit admitting its full quota,
one decode step over L layers moves

    bytes(m) = L * units * m * record_bytes,   m = floor(cap * K),

and a pipelined step (prefetch on a side stream, layer-local waits) takes
about max(window, bytes / link_bandwidth), the window being the step's
compute (L fused layer steps).  The largest quota that hides is
m* = floor(bandwidth * window / (L * units * record_bytes)).
"""
from __future__ import annotations

import math


def bytes_per_step(layers: int, units: int, max_admit: int, record_bytes: int) -> int:
    """Host-link bytes of one decode step when every unit admits its quota."""
    return int(layers) * int(units) * int(max_admit) * int(record_bytes)


def largest_hidden_admit(bandwidth: float, window_s: float, layers: int, units: int,
                         record_bytes: int, k_resident: int) -> int:
    """Largest per-unit quota whose bytes move within the window (0..K)."""
    per_admit = float(layers) * units * record_bytes
    if per_admit <= 0 or bandwidth <= 0 or window_s <= 0:
        return 0
    m = math.floor(bandwidth * window_s / per_admit + 1e-9)
    return max(0, min(int(k_resident), m))


def predicted_step_s(window_s: float, nbytes: float, bandwidth: float,
                     overlap: bool = True) -> float:
    """Step time with the transfer overlapped with the compute window (the
    larger of the two), or serialised after it."""
    xfer = nbytes / bandwidth if bandwidth > 0 else math.inf
    return max(window_s, xfer) if overlap else window_s + xfer


def overlap_fraction(step_s: float, compute_s: float, xfer_s: float) -> float:
    """Share of the shorter of the compute window and the transfer that the
    pipelined step hid behind the other: (compute + transfer - step) /
    min(compute, transfer), clipped to [0, 1] (1 = fully hidden, 0 = serial)."""
    shorter = min(compute_s, xfer_s)
    if shorter <= 0:
        return 1.0
    return max(0.0, min(1.0, (compute_s + xfer_s - step_s) / shorter))
