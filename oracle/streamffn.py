"""Plain CPU oracle of the streaming-FFN schedule (launch threshold, final
flush, arrival order).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only the tests and the benchmark's CPU-baseline leg use
it.  It shares no code with the library.

Source: page "CascadeEP: Asynchronous Expert Execution for MoE Prefill under
Attention Imbalance", section 3.2 ("Launch threshold", "Multi-stream
execution") and Appendix C (per-replica readiness, grouped FFN invocations,
final flush).

Readings taken where the page leaves a step open:
* The "expert-token count" that the threshold and the throughput curve are
  measured in is the number of routed (token, local expert) rows one grouped
  FFN invocation computes on this GPU.
* Ready work is counted in whole replicas: a replica's routed rows become
  eligible together when its lane completes, and an invocation takes every
  row that is ready and not yet launched.
* A launch happens at the first arrival after which the ready, unlaunched
  rows reach the threshold (>= theta); after the last arrival whatever is
  left is launched regardless of the threshold (the final flush).
* Arrival order: attention time grows with a replica's load, so replicas
  arrive in ascending order of their token count (ties by replica index).
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

__all__ = ["threshold", "launch_groups", "arrival_order"]


def threshold(counts: Sequence[int], throughput: Sequence[float], rho: float) -> int:
    """Launch threshold theta: the smallest profiled expert-token count whose
    measured FFN throughput reaches rho times the highest throughput
    observed (CascadeEP section 3.2).  counts and throughput are the profile
    points, in any order."""
    c = np.asarray(counts, dtype=np.int64)
    tp = np.asarray(throughput, dtype=np.float64)
    if c.shape != tp.shape or c.size == 0:
        raise ValueError("one throughput per profiled count, at least one point")
    peak = tp.max()
    ok = tp >= rho * peak
    return int(c[ok].min())


def launch_groups(ready_rows: Sequence[int], theta: int) -> List[int]:
    """Invocations formed from arrivals in order.  ready_rows[i] is the
    number of routed rows that become ready with arrival i.  Returns the
    exclusive end index of each invocation's arrivals: invocation j covers
    arrivals [ends[j-1], ends[j]) (ends[-1] = number of arrivals).

    Rows accumulate until the ready, unlaunched count reaches theta, which
    launches them; after the last arrival the remainder is flushed even
    below theta.  (An arrival with no rows still counts as an arrival.)"""
    ends: List[int] = []
    pending = 0
    n = len(ready_rows)
    for i, r in enumerate(ready_rows):
        if r < 0:
            raise ValueError("negative row count")
        pending += int(r)
        last = i == n - 1
        if pending >= theta or last:
            ends.append(i + 1)
            pending = 0
    return ends


def arrival_order(replica_offsets: Sequence[int]) -> List[int]:
    """Replica indices in arrival order: ascending token count, ties by
    index.  replica_offsets [R + 1] are the token offsets of the replica-major
    split."""
    off = np.asarray(replica_offsets, dtype=np.int64)
    sizes = off[1:] - off[:-1]
    return sorted(range(len(sizes)), key=lambda r: (int(sizes[r]), r))
