"""Pins of oracle.waterfill (latency model Eq. 2-11, Algorithm 2) -- CPU only."""
import itertools
import json
import os
import random

import pytest

from oracle import waterfill as wf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "waterfill_worked_example.json")


def _model(**kw):
    m = dict(gamma=1.0, gamma0=0.0, a_d=0.0, a_d0=0.0, a_p=0.0, a_p0=0.0, a_comm=0.0,
             a_comm0=0.0, alpha=1.0, beta=1.0, n_layers=1)
    m.update(kw)
    return m


def test_worked_example_from_the_pages():
    g = json.load(open(GOLDEN))
    loads = g["n_decode_tokens"]
    assert wf.capacity(loads, g["n_target"]) == g["capacities"]
    r = wf.dispatch(tau=1.0, n_decode_tokens=loads, decode_ctx_sum=[0] * 4,
                    candidate=(g["candidate_remaining"], 0), model=_model(),
                    fixed_target=g["n_target"])
    assert r["budget"] == g["budget"]
    assert r["chunk_len"] == g["chunk_len"]
    assert r["assign"] == g["assign"]


def test_worked_example_shorter_prompt_level_fill():
    # Derived by hand (not printed): 1000 tokens toward 300 over loads 40/10/10/0 fill to
    # level 265: 225 + 255 + 255 + 265 = 1000.
    r = wf.dispatch(tau=1.0, n_decode_tokens=[40, 10, 10, 0], decode_ctx_sum=[0] * 4,
                    candidate=(1000, 0), model=_model(), fixed_target=300)
    assert r["budget"] == 1140 and r["chunk_len"] == 1000
    assert r["assign"] == [225, 255, 255, 265]


def test_remainder_goes_to_lowest_ranks_first():
    # loads 5/5/5, 7 tokens toward 100: level 7 takes 6, one left -> rank 0.
    assert wf.waterfill_assign([5, 5, 5], 7, 100) == [3, 2, 2]
    # a rank above the level gets nothing
    assert wf.waterfill_assign([50, 0, 0], 10, 100) == [0, 5, 5]
    assert wf.waterfill_assign([3, 0], 0, 10) == [0, 0]


def _brute_minmax(loads, tokens, n_target):
    caps = wf.capacity(loads, n_target)
    best = None
    for a in itertools.product(*[range(c + 1) for c in caps]):
        if sum(a) != tokens:
            continue
        v = max(l + x for l, x in zip(loads, a))
        best = v if best is None else min(best, v)
    return best


def test_assignment_is_minmax_optimal_against_enumeration():
    rnd = random.Random(7)
    for _ in range(150):
        n = rnd.randint(1, 4)
        loads = [rnd.randint(0, 12) for _ in range(n)]
        n_target = rnd.randint(max(loads), max(loads) + 10)
        cap = sum(wf.capacity(loads, n_target))
        tokens = rnd.randint(0, min(cap, 30))
        a = wf.waterfill_assign(loads, tokens, n_target)
        assert sum(a) == tokens
        assert all(0 <= x <= c for x, c in zip(a, wf.capacity(loads, n_target)))
        if tokens:
            assert max(l + x for l, x in zip(loads, a)) == _brute_minmax(loads, tokens, n_target)


def test_latency_model_closed_forms_two_ranks():
    m = dict(gamma=2.0, gamma0=3.0, a_d=0.5, a_d0=1.0, a_p=0.25, a_p0=2.0, a_comm=4.0,
             a_comm0=5.0, alpha=1.5, beta=2.0, n_layers=3)
    # rank loads: decode 3/1 tokens, prefill 2/4 tokens; contexts 10/30; one chunk (6, 8)
    t = wf.iteration_latency(m, [3, 1], [10, 30], [2, 4], [(6, 8)])
    t_gemm = 2.0 * 5 + 3.0                         # max(3+2, 1+4) = 5
    t_d = 0.5 * 30 + 1.0                           # slowest rank by aggregate context
    work = 6 * 8 + 6 * 7 // 2                      # l c + l(l+1)/2 = 69
    t_p = (4.0 * 4 + 5.0) + (0.25 * (work / 2) + 2.0)
    assert t == 3 * (t_gemm + max(2.0 * t_p, 1.5 * t_d))
    # no prefill anywhere: the prefill path contributes nothing
    t0 = wf.iteration_latency(m, [3, 1], [10, 30], [0, 0], [])
    assert t0 == 3 * (2.0 * 3 + 3.0 + 1.5 * t_d)


def test_prefill_work_matches_pair_count_forms():
    # ConfluxServe Eq. 9 and Adaptive Context Parallelism Eq. 1 count the same pairs
    for l in range(0, 40):
        for c in (0, 1, 5, 17):
            assert wf.prefill_work(l, c) == sum(c + t + 1 for t in range(l))


def _random_case(rnd):
    n = rnd.randint(1, 4)
    nd = [rnd.randint(0, 20) for _ in range(n)]
    ctx = [rnd.randint(0, 500) * (1 if nd[r] else 0) for r in range(n)]
    ex = [rnd.randint(0, 6) for _ in range(n)]
    sel = [(rnd.randint(1, 8), rnd.randint(0, 50))] if rnd.random() < 0.5 else []
    cand = (rnd.randint(1, 60), rnd.randint(0, 100)) if rnd.random() < 0.8 else None
    m = dict(gamma=rnd.choice([0.5, 1.0, 2.0]), gamma0=rnd.choice([0.0, 3.0]),
             a_d=rnd.choice([0.0, 0.125, 0.25]), a_d0=rnd.choice([0.0, 1.0]),
             a_p=rnd.choice([0.0, 0.0625]), a_p0=rnd.choice([0.0, 1.0]),
             a_comm=rnd.choice([0.0, 0.5]), a_comm0=rnd.choice([0.0, 2.0]),
             alpha=rnd.choice([1.0, 1.25]), beta=rnd.choice([1.0, 1.5]), n_layers=rnd.choice([1, 2]))
    tau = float(rnd.randint(10, 400))
    q = rnd.choice([1, 2, 4])
    return dict(tau=tau, n_decode_tokens=nd, decode_ctx_sum=ctx, existing=ex, selected=sel,
                candidate=cand, quantum=q, model=m, level_hi=0 if cand else 120)


def test_binary_search_equals_linear_scan_and_is_monotone():
    rnd = random.Random(11)
    for _ in range(300):
        kw = _random_case(rnd)
        r = wf.dispatch(**kw)
        loads = [a + b for a, b in zip(kw["n_decode_tokens"], kw["existing"])]
        hi = max(loads) + kw["candidate"][0] if kw["candidate"] else kw["level_hi"]
        q = kw["quantum"]
        levels = list(range(0, -(-hi // q) * q + 1, q))
        feas = [wf.feasible(n, kw["tau"], kw["n_decode_tokens"], kw["decode_ctx_sum"], kw["existing"],
                            kw["selected"], kw["candidate"], kw["model"]) for n in levels]
        for a, b in zip(feas, feas[1:]):
            assert a or not b, "feasibility must be monotone in the level"
        ok = [n for n, f in zip(levels, feas) if f]
        assert r["n_target"] == (max(ok) if ok else 0)
        assert r["budget"] == sum(wf.capacity(loads, r["n_target"]))
        if kw["candidate"]:
            assert r["chunk_len"] == min(kw["candidate"][0], r["budget"])
        else:
            assert r["chunk_len"] == r["budget"]
        assert sum(r["assign"]) == r["chunk_len"]


def test_even_dispatch_never_beats_waterfill_on_shared_linear_load():
    # ConfluxServe §8.3 Fig. 15a direction: an even split has a max combined load at least
    # as high as the waterfill split of the same tokens.
    rnd = random.Random(3)
    for _ in range(200):
        n = rnd.randint(2, 8)
        nd = [rnd.randint(0, 200) for _ in range(n)]
        tokens = rnd.randint(0, 2000)
        a = wf.waterfill_assign(nd, tokens, max(nd) + tokens)
        even = [tokens // n + (1 if r < tokens % n else 0) for r in range(n)]
        assert max(x + y for x, y in zip(nd, a)) <= max(x + y for x, y in zip(nd, even))


def test_budget_zero_is_not_an_error():
    # decode alone already violates the SLO: nothing is feasible, B = 0, chunk 0
    m = _model(gamma=1.0)
    r = wf.dispatch(tau=5.0, n_decode_tokens=[10, 10], decode_ctx_sum=[0, 0], candidate=(100, 0),
                    model=m)
    assert r == dict(n_target=0, budget=0, chunk_len=0, assign=[0, 0])


def test_overfull_assign_is_rejected():
    with pytest.raises(ValueError):
        wf.waterfill_assign([0, 0], 30, 10)
