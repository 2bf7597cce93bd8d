"""SLO-aware scheduler around the waterfill dispatcher, step by step (test infrastructure).

ConfluxServe §6.4 (Algorithm 1), §6.3 "Decode: dual-mode placement" with App. F
(Algorithm 3), and App. G (Algorithm 4, Moore-Hodgson admission).  Python integers
for token counts and capacities, Python floats (fp64) for times.  The dispatcher
calls go to ``oracle.waterfill.dispatch`` (Algorithm 2).

Readings of points the pages leave open:

* App. G's capacity before the deadline is K_i = max(0, floor((d_i - t) / tau)) * B0:
  the whole iterations left before d_i times the per-iteration budget (the printed
  formula lost its floor brackets).  The iteration count is clamped at 2**40.
* Orders and ties: EDF sorts by (deadline, request index); the max-heap gives up the
  largest remaining length, and among equal lengths the one later in EDF order; SJF
  sorts the removed requests by (remaining length, EDF position); placement ties go to
  the lowest rank index.
* Placement: a request that finishes its prompt keeps c + m KV tokens; rank r is
  feasible when kv_used + (c + m) + h <= kv_capacity (h: KV tokens kept free);
  "utilization" is kv_used / kv_capacity before the placement, compared with eta in
  fp64.  WorstFit takes the smallest aggregate decode context, BestFit the highest
  utilization.  A reserved placement adds c + m to the host's decode context and KV
  use in the tentative state.
* The dispatcher always sees the current decode state D (the new decodes start in
  the next iteration); only placement sees the tentative state.
* B0 is the dispatcher's budget with no candidate and nothing selected, its level
  search bounded by max_r n_d^r + sum_i m_i.
"""
from __future__ import annotations

import heapq
import math
from fractions import Fraction

from .waterfill import dispatch

__all__ = ["edf_order", "admission", "placement", "schedule"]

MAX_ITERATIONS = 2 ** 40


def edf_order(deadlines) -> list:
    """Request indices by earliest deadline first (ties: lower index first)."""
    return sorted(range(len(deadlines)), key=lambda i: (deadlines[i], i))


def admission(m_remaining, deadlines, ref_budget: int, now: float, tau: float):
    """Algorithm 4: returns (admitted in EDF order, removed in SJF order)."""
    edf = edf_order(deadlines)
    position = {i: k for k, i in enumerate(edf)}
    total = 0
    heap = []                                  # max-heap on (m, EDF position)
    removed = set()
    for i in edf:
        total += m_remaining[i]
        heapq.heappush(heap, (-m_remaining[i], -position[i], i))
        iterations = math.floor((deadlines[i] - now) / tau)
        iterations = min(max(0, iterations), MAX_ITERATIONS)
        if total > iterations * ref_budget:    # capacity before d_i exceeded
            _, _, j = heapq.heappop(heap)
            total -= m_remaining[j]
            removed.add(j)
    admitted = [i for i in edf if i not in removed]
    rejected = sorted(removed, key=lambda j: (m_remaining[j], position[j]))
    return admitted, rejected


def placement(decode_ctx_sum, kv_used, kv_capacity, need: int, eta: float, headroom: int):
    """Algorithm 3: the host rank of a request whose KV state is ``need`` tokens, or None
    (Infeasible)."""
    ranks = range(len(kv_used))
    feasible = [r for r in ranks if kv_used[r] + need + headroom <= kv_capacity[r]]
    if not feasible:
        return None
    low = [r for r in feasible if kv_used[r] / kv_capacity[r] < eta]
    if low:                                    # WorstFit: smallest aggregate decode context
        return min(low, key=lambda r: (decode_ctx_sum[r], r))
    # BestFit: highest utilization that still fits (exact fractions)
    return min(feasible, key=lambda r: (-Fraction(kv_used[r], kv_capacity[r]), r))


def schedule(*, n_decode_tokens, decode_ctx_sum, kv_used, kv_capacity, m_remaining, c_processed,
             deadlines, now, tau, quantum, eta, headroom, model) -> dict:
    """Algorithm 1: one iteration's prefill batch, its per-rank assignment and the decode
    hosts of the prompts it completes."""
    N, R = len(n_decode_tokens), len(m_remaining)
    # Line 2: reference budget B0
    level_hi = max(n_decode_tokens) + sum(m_remaining)
    b0 = dispatch(tau=tau, n_decode_tokens=n_decode_tokens, decode_ctx_sum=decode_ctx_sum,
                  existing=[0] * N, selected=(), candidate=None, quantum=quantum, model=model,
                  level_hi=level_hi)["budget"]
    # Lines 3-4: admission, EDF for the admitted, SJF for the rest
    admitted, rejected = admission(m_remaining, deadlines, b0, now, tau)
    order = admitted + rejected
    # tentative decode state for placement
    ctx_t, used_t = list(decode_ctx_sum), list(kv_used)
    a_p = [0] * N
    selected = []
    chunk = [0] * R
    host = [-1] * R
    req_assign = [[0] * N for _ in range(R)]
    stop, n_selected = "done", 0
    for k, i in enumerate(order):                 # Lines 5-13
        d = dispatch(tau=tau, n_decode_tokens=n_decode_tokens, decode_ctx_sum=decode_ctx_sum,
                     existing=a_p, selected=selected, candidate=(m_remaining[i], c_processed[i]),
                     quantum=quantum, model=model)
        length, a_i = d["chunk_len"], d["assign"]
        if length == 0:                           # budget exhausted
            stop = "budget"
            break
        if length == m_remaining[i]:              # the chunk completes the prompt
            need = c_processed[i] + m_remaining[i]
            g = placement(ctx_t, used_t, kv_capacity, need, eta, headroom)
            if g is None:                         # no feasible decode host
                stop = "no_host"
                break
            ctx_t[g] += need
            used_t[g] += need
            host[i] = g
        a_p = [a_p[r] + a_i[r] for r in range(N)]
        selected = selected + [(length, c_processed[i])]
        chunk[i] = length
        req_assign[i] = list(a_i)
        n_selected = k + 1
    return dict(ref_budget=b0, n_admitted=len(admitted), order=order, n_selected=n_selected, stop=stop,
                chunk_len=chunk, decode_rank=host, prefill_assign=a_p, request_assign=req_assign)
