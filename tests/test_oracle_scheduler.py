"""Pins of oracle.scheduler (Algorithms 1, 3 and 4 of ConfluxServe) -- CPU only.

Admission is pinned by brute force: Moore-Hodgson keeps the largest set of requests
that all meet their capacity bound in EDF order.  Placement and the scheduling loop
are pinned by small cases worked out by hand from the pages' definitions and by
invariants every iteration must satisfy (the batch is TBT-safe, assignments add up,
completed prompts have a host).
"""
import dataclasses
import itertools
import math
import random

import pytest

from oracle import scheduler as sch
from oracle import waterfill as wf
from synth import scheduler_case


def _model(**kw):
    m = dict(gamma=1.0, gamma0=0.0, a_d=0.0, a_d0=0.0, a_p=0.0, a_p0=0.0, a_comm=0.0,
             a_comm0=0.0, alpha=1.0, beta=1.0, n_layers=1)
    m.update(kw)
    return m


def _capacity(d, now, tau, b0):
    return max(0, math.floor((d - now) / tau)) * b0


def _edf_feasible(subset, m, d, now, tau, b0):
    total = 0
    for i in sorted(subset, key=lambda i: (d[i], i)):
        total += m[i]
        if total > _capacity(d[i], now, tau, b0):
            return False
    return True


def test_admission_keeps_a_largest_on_time_set_against_enumeration():
    rnd = random.Random(11)
    for _ in range(400):
        R = rnd.randint(0, 7)
        m = [rnd.randint(1, 12) for _ in range(R)]
        d = [rnd.choice([0.5, 1.0, 1.5, 2.0, 2.5, 3.0, 4.0, 6.0]) for _ in range(R)]
        b0 = rnd.randint(0, 10)
        adm, rej = sch.admission(m, d, b0, 0.0, 1.0)
        assert sorted(adm + rej) == list(range(R))
        assert _edf_feasible(adm, m, d, 0.0, 1.0, b0)
        best = max((len(s) for k in range(R + 1) for s in itertools.combinations(range(R), k)
                    if _edf_feasible(s, m, d, 0.0, 1.0, b0)), default=0)
        assert len(adm) == best
        assert adm == sorted(adm, key=lambda i: (d[i], i))                       # EDF
        assert [m[j] for j in rej] == sorted(m[j] for j in rej)                   # SJF


def test_admission_worked_case_with_a_tie():
    # B0 = 160, tau = 100, now = 0; d = 150/160/170 give one iteration each (K = 160).
    # EDF 0, 1, 2: after 1 the total 200 > 160, the two 100-token requests tie and the
    # later one in EDF order (1) leaves; 2 then fits (110 <= 160).
    adm, rej = sch.admission([100, 100, 10], [150.0, 160.0, 170.0], 160, 0.0, 100.0)
    assert (adm, rej) == ([0, 2], [1])
    # a deadline already passed gives K = 0: nothing with that deadline can stay
    adm, rej = sch.admission([5, 7], [-1.0, 250.0], 160, 0.0, 100.0)
    assert (adm, rej) == ([1], [0])


def test_placement_worst_fit_best_fit_and_infeasible_by_hand():
    cap = [1000, 1000, 1000]
    # all below eta = 0.5: worst fit on the smallest decode context (rank 2), not the
    # emptiest KV (rank 0)
    assert sch.placement([500, 400, 300], [100, 200, 300], cap, 50, 0.5, 0) == 2
    # rank 2 no longer fits with headroom 700 (300 + 50 + 700 > 1000): rank 1
    assert sch.placement([500, 400, 300], [100, 200, 300], cap, 50, 0.5, 700) == 1
    # every feasible rank at or above eta: best fit on the highest utilization that fits
    assert sch.placement([1, 2, 3], [600, 900, 700], cap, 50, 0.5, 0) == 1
    assert sch.placement([1, 2, 3], [600, 960, 700], cap, 50, 0.5, 0) == 2   # 960+50 > 1000
    # utilizations compare as fractions across capacities: 600/800 > 700/1000
    assert sch.placement([0, 0], [700, 600], [1000, 800], 10, 0.5, 0) == 1
    # mixed: only the low-utilization feasible ranks take part in worst fit
    assert sch.placement([10, 900, 20], [700, 100, 800], cap, 50, 0.5, 0) == 1
    # ties: lowest rank index
    assert sch.placement([5, 5], [100, 100], [1000, 1000], 1, 0.9, 0) == 0
    # nowhere to go
    assert sch.placement([0, 0], [990, 995], [1000, 1000], 20, 0.5, 0) is None


HAND = dict(n_decode_tokens=[10, 30], decode_ctx_sum=[10000, 30000], kv_used=[1000, 3000],
            kv_capacity=[10000, 10000], m_remaining=[100, 50, 40], c_processed=[0, 0, 0],
            deadlines=[150.0, 250.0, 120.0], now=0.0, tau=100.0, quantum=1, eta=0.5, headroom=0,
            model=_model())


def test_schedule_worked_case_by_hand():
    # T = max_r (n_d^r + n_p^r) with this model.  B0: level 100 -> 90 + 70 = 160.
    # EDF 2 (K 160), 0 (K 160), 1 (K 320): totals 40, 140, 190, all admitted.
    # Request 2 (m 40): level 70 fills [30, 10] -> loads 40/40; completes -> worst fit on
    #   decode context 10000 < 30000 -> rank 0 (context 10040, KV 1040 afterwards).
    # Request 0 (m 100): loads 40/40, level 140 fills [50, 50] -> 90/90; completes -> rank 0
    #   (context 10140 < 30000, utilization 0.104 < 0.5).
    # Request 1 (m 50): loads 90/90; level 100 is the largest with T <= 100 -> B = 20,
    #   chunk 20 = [10, 10]; does not complete.
    r = sch.schedule(**HAND)
    assert r["ref_budget"] == 160 and r["n_admitted"] == 3 and r["order"] == [2, 0, 1]
    assert r["chunk_len"] == [100, 20, 40] and r["decode_rank"] == [0, -1, 0]
    assert r["prefill_assign"] == [90, 70] and r["request_assign"] == [[50, 50], [10, 10], [30, 10]]
    assert (r["n_selected"], r["stop"]) == (3, "done")


def test_schedule_stops_when_no_host_fits():
    case = dict(HAND, kv_capacity=[1030, 3030])       # 40 more KV tokens fit nowhere
    r = sch.schedule(**case)
    assert r["stop"] == "no_host" and r["n_selected"] == 0 and r["chunk_len"] == [0, 0, 0]
    assert r["prefill_assign"] == [0, 0]


def test_schedule_stops_when_the_budget_is_exhausted():
    case = dict(HAND, tau=30.0)                        # rank 1 alone already reaches T = 30
    r = sch.schedule(**case)
    assert r["ref_budget"] == 20 and r["stop"] == "budget"
    # the first admitted request gets the 20 tokens of rank 0's headroom; the next one none
    assert sum(r["chunk_len"]) == 20 and r["prefill_assign"] == [20, 0]


def test_schedule_with_unbounded_slo_takes_every_prompt_whole():
    case = dict(HAND, tau=1e9)
    r = sch.schedule(**case)
    assert r["chunk_len"] == case["m_remaining"] and r["stop"] == "done"
    assert all(g >= 0 for g in r["decode_rank"])
    assert sum(r["prefill_assign"]) == sum(case["m_remaining"])


def _random_case(rnd):
    N, R = rnd.randint(1, 5), rnd.randint(0, 9)
    nd = [rnd.randint(0, 40) for _ in range(N)]
    return dict(n_decode_tokens=nd, decode_ctx_sum=[rnd.randint(0, 4000) * (n > 0) for n in nd],
                kv_used=[rnd.randint(0, 5000) for _ in range(N)], kv_capacity=[rnd.randint(5000, 9000) for _ in range(N)],
                m_remaining=[rnd.randint(1, 400) for _ in range(R)], c_processed=[rnd.randint(0, 900) for _ in range(R)],
                deadlines=[rnd.uniform(-50, 800) for _ in range(R)], now=0.0, tau=float(rnd.randint(40, 400)),
                quantum=rnd.choice([1, 4, 16]), eta=rnd.choice([0.3, 0.6, 0.9]), headroom=rnd.choice([0, 256]),
                model=_model(gamma=rnd.choice([0.5, 1.0]), gamma0=rnd.choice([0.0, 4.0]),
                             a_d=rnd.choice([0.0, 2.0 ** -8]), a_p=rnd.choice([0.0, 2.0 ** -12]),
                             a_comm=rnd.choice([0.0, 0.25]), beta=rnd.choice([1.0, 1.25])))


def test_schedule_invariants_on_random_iterations():
    rnd = random.Random(3)
    for _ in range(300):
        c = _random_case(rnd)
        r = sch.schedule(**c)
        R, N = len(c["m_remaining"]), len(c["n_decode_tokens"])
        chosen = r["order"][:r["n_selected"]]
        # the batch is a prefix of the consideration order; the rest is unscheduled
        assert all(r["chunk_len"][i] > 0 for i in chosen)
        assert all(r["chunk_len"][i] == 0 for i in r["order"][r["n_selected"]:])
        assert all(1 <= r["chunk_len"][i] <= c["m_remaining"][i] for i in chosen)
        # per-rank assignments add up to the chunks
        for i in range(R):
            assert sum(r["request_assign"][i]) == r["chunk_len"][i]
        assert [sum(r["request_assign"][i][k] for i in range(R)) for k in range(N)] == r["prefill_assign"]
        # a completed prompt has a host, an incomplete one has none
        for i in range(R):
            done = r["chunk_len"][i] == c["m_remaining"][i]
            assert (r["decode_rank"][i] >= 0) == done
        # the whole batch is TBT-safe under the model
        if chosen:
            t = wf.iteration_latency(c["model"], c["n_decode_tokens"], c["decode_ctx_sum"], r["prefill_assign"],
                                     [(r["chunk_len"][i], c["c_processed"][i]) for i in chosen])
            assert t <= c["tau"]
        # hosts keep their headroom, counting every placement made in the iteration
        used = list(c["kv_used"])
        for i in chosen:
            g = r["decode_rank"][i]
            if g >= 0:
                used[g] += c["c_processed"][i] + c["m_remaining"][i]
                assert used[g] + c["headroom"] <= c["kv_capacity"][g]


@pytest.mark.parametrize("depth", [10, 100])
def test_synthetic_iteration_is_budget_limited_and_safe(depth):
    c = dataclasses.asdict(scheduler_case(depth))
    c.pop("name")
    r = sch.schedule(**c)
    assert r["ref_budget"] > 0 and r["n_selected"] > 0
    chosen = r["order"][:r["n_selected"]]
    t = wf.iteration_latency(c["model"], c["n_decode_tokens"], c["decode_ctx_sum"], r["prefill_assign"],
                             [(r["chunk_len"][i], c["c_processed"][i]) for i in chosen])
    assert t <= c["tau"]
