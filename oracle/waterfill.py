"""Latency model and waterfill dispatch, step by step (test infrastructure).

ConfluxServe §6.2 (Eq. 2-6), App. D (Eq. 7-12), §6.3 and App. E (Algorithm 2).
Python integers for token counts, Python floats (fp64) for latencies.

Readings of points the pages leave open:

* Eq. 6 is read as T_P = f_comm(max_r n_p^r) + f_P((1/N) * sum_{i in P} l_i (c_i + (l_i + 1)/2)),
  with P the selected chunks plus the candidate's chunk when it is non-empty.
* A path with no work at all this iteration contributes 0 (no decode anywhere: T_D = 0;
  no prefill token anywhere: T_P = 0; no token on any rank: T_GEMM = 0); otherwise the
  affine base functions are evaluated as printed, intercepts included.
* Feasible(n) evaluates the model on the assignment the level-n dispatch actually makes
  (existing + WaterfillAssign of l(n) = min(m, B(n)) tokens toward n), so feasibility is
  monotone in n and binary search over levels 0, q, 2q, ... is valid.
* Search range: levels k*q for k = 0..ceil(hi/q) with hi = max_r load_r + m when a
  candidate is given, else the caller's level_hi.  If no level is feasible, n_target = 0.
* WaterfillAssign: the largest integer level L <= n_target with
  sum_r max(0, L - load_r) <= l; each rank gets max(0, L - load_r); the remaining tokens
  go one each to the ranks with load_r <= L in ascending rank order.
"""
from __future__ import annotations

__all__ = ["f_gemm", "f_d", "f_p", "f_comm", "prefill_work", "iteration_latency",
           "capacity", "waterfill_assign", "feasible", "dispatch"]


def f_gemm(model: dict, n: int) -> float:
    """Eq. 7: shared-linear latency of n rank-local tokens."""
    return model["gamma"] * n + model["gamma0"]


def f_d(model: dict, w: int) -> float:
    """Eq. 8: decode-attention latency of aggregate context w."""
    return model["a_d"] * w + model["a_d0"]


def f_p(model: dict, w: float) -> float:
    """Eq. 10: prefill-attention latency of per-rank workload w."""
    return model["a_p"] * w + model["a_p0"]


def f_comm(model: dict, n: int) -> float:
    """Eq. 11: All-to-All latency of the largest prefill shard n."""
    return model["a_comm"] * n + model["a_comm0"]


def prefill_work(length: int, ctx: int) -> int:
    """Eq. 9: causal-attention workload l (c + (l + 1)/2) of a chunk, as an exact integer
    l*c + l(l+1)/2 (the same count as Adaptive Context Parallelism §2.2 Eq. 1)."""
    return length * ctx + length * (length + 1) // 2


def iteration_latency(model: dict, n_decode_tokens, decode_ctx_sum, n_prefill_tokens, chunks) -> float:
    """Eq. 2-6: T_iter = L (T_GEMM + max(beta T_P, alpha T_D)) for per-rank decode token
    loads, per-rank aggregate decode context, per-rank prefill tokens and the list of
    scheduled chunks [(l, c)]."""
    N = len(n_decode_tokens)
    loads = [n_decode_tokens[r] + n_prefill_tokens[r] for r in range(N)]
    t_gemm = f_gemm(model, max(loads)) if max(loads) > 0 else 0.0                 # Eq. 3
    t_d = max(f_d(model, w) for w in decode_ctx_sum) if sum(n_decode_tokens) > 0 else 0.0  # Eq. 5
    if sum(n_prefill_tokens) > 0:                                                   # Eq. 6
        w = sum(prefill_work(l, c) for l, c in chunks)
        t_p = f_comm(model, max(n_prefill_tokens)) + f_p(model, w / N)
    else:
        t_p = 0.0
    t_attn = max(model["beta"] * t_p, model["alpha"] * t_d)                         # Eq. 4
    return model["n_layers"] * (t_gemm + t_attn)                                    # Eq. 2


def capacity(loads, n_target: int) -> list:
    """Per-rank additional capacity max(0, n_target - n_d^r - n_p^r(A_p)) (App. E)."""
    return [max(0, n_target - ld) for ld in loads]


def waterfill_assign(loads, tokens: int, n_target: int) -> list:
    """Distribute ``tokens`` toward the level n_target, filling the lowest ranks first."""
    N = len(loads)
    if tokens <= 0:
        return [0] * N
    if tokens > sum(capacity(loads, n_target)):
        raise ValueError("more tokens than capacity at n_target")
    lo, hi = min(loads), n_target            # largest L in [lo, hi] with fill(L) <= tokens
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if sum(capacity(loads, mid)) <= tokens:
            lo = mid
        else:
            hi = mid - 1
    level = lo
    out = capacity(loads, level)
    rest = tokens - sum(out)
    for r in range(N):
        if rest == 0:
            break
        if loads[r] <= level:
            out[r] += 1
            rest -= 1
    assert rest == 0
    return out


def _at_level(n, loads, n_decode_tokens, decode_ctx_sum, existing, selected, candidate, model):
    b = sum(capacity(loads, n))
    length = b if candidate is None else min(candidate[0], b)
    add = waterfill_assign(loads, length, n)
    n_p = [existing[r] + add[r] for r in range(len(loads))]
    chunks = list(selected)
    if candidate is not None and length > 0:
        chunks.append((length, candidate[1]))
    t = iteration_latency(model, n_decode_tokens, decode_ctx_sum, n_p, chunks)
    return b, length, add, t


def feasible(n, tau, n_decode_tokens, decode_ctx_sum, existing, selected, candidate, model) -> bool:
    loads = [n_decode_tokens[r] + existing[r] for r in range(len(n_decode_tokens))]
    return _at_level(n, loads, n_decode_tokens, decode_ctx_sum, existing, selected, candidate,
                     model)[3] <= tau


def dispatch(*, tau, n_decode_tokens, decode_ctx_sum, existing=None, selected=(), candidate=None,
             quantum=1, model, fixed_target=-1, level_hi=0) -> dict:
    """Algorithm 2 (App. E).  Returns n_target, budget B, chunk l (= B when there is no
    candidate) and the incremental per-rank assignment A_i."""
    N = len(n_decode_tokens)
    existing = [0] * N if existing is None else list(existing)
    loads = [n_decode_tokens[r] + existing[r] for r in range(N)]
    args = (n_decode_tokens, decode_ctx_sum, existing, selected, candidate, model)
    if fixed_target >= 0:
        n_target = fixed_target
    else:
        q = quantum
        hi = (max(loads) + candidate[0]) if candidate is not None else level_hi
        k_hi = -(-hi // q)
        if not feasible(0, tau, *args):
            n_target = 0
        else:
            lo_k, hi_k = 0, k_hi                   # invariant: level lo_k*q is feasible
            while lo_k < hi_k:
                mid = (lo_k + hi_k + 1) // 2
                if feasible(mid * q, tau, *args):
                    lo_k = mid
                else:
                    hi_k = mid - 1
            n_target = lo_k * q
    budget = sum(capacity(loads, n_target))
    length = budget if candidate is None else min(candidate[0], budget)
    assign = waterfill_assign(loads, length, n_target)
    return dict(n_target=n_target, budget=budget, chunk_len=length, assign=assign)
