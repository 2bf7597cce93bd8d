"""The C-ABI library on the host: it loads, exports every declared symbol, its host-only
entry points (waterfill, latency model, validation) agree with the oracle -- CPU only."""
import os
import random
import re

import numpy as np
import pytest

import mixed_prefill_decode_amd as X
from oracle import waterfill as wf
from synth import get_workload, make_instance, waterfill_cases

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "xp.h")


def test_library_exports_every_declared_symbol():
    decl = set(re.findall(r"^\s*(?:xp_status|const char\*|size_t)\s+(xp_\w+)\s*\(", open(HEADER).read(), re.M))
    assert decl == set(X.EXPORTED)
    L = X.lib()
    for name in decl:
        assert getattr(L, name) is not None
    assert "gfx950" in X.xp_build_info()


def test_stage_names_follow_the_header():
    # the binding's stage names are indexed by the header's XP_STAGE_* values
    defs = dict((m, int(v)) for m, v in re.findall(r"^#define XP_STAGE_(\w+) (\d+)", open(HEADER).read(), re.M))
    assert defs.pop("COUNT") == X.XP_STAGE_COUNT == len(X.STAGES)
    assert {X.STAGES[v]: v for v in defs.values()} == {m.lower(): v for m, v in defs.items()}


def test_waterfill_worked_example():
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "waterfill_worked_example.json")))
    m = dict(gamma=1.0, gamma0=0.0, a_d=0.0, a_d0=0.0, a_p=0.0, a_p0=0.0, a_comm=0.0, a_comm0=0.0,
             alpha=1.0, beta=1.0, n_layers=1)
    r = X.xp_waterfill(tau=1.0, n_decode_tokens=g["n_decode_tokens"], decode_ctx_sum=[0] * 4,
                       candidate=(g["candidate_remaining"], 0), model=m, fixed_target=g["n_target"])
    assert (r["budget"], r["chunk_len"], r["assign"]) == (g["budget"], g["chunk_len"], g["assign"])


def _rand_model(rnd):
    # arbitrary (non-dyadic) coefficients: both sides evaluate the same IEEE operations
    return dict(gamma=rnd.uniform(0.1, 3), gamma0=rnd.uniform(0, 5), a_d=rnd.uniform(0, 0.3),
                a_d0=rnd.uniform(0, 2), a_p=rnd.uniform(0, 0.1), a_p0=rnd.uniform(0, 2),
                a_comm=rnd.uniform(0, 1), a_comm0=rnd.uniform(0, 3), alpha=rnd.uniform(1, 1.5),
                beta=rnd.uniform(1, 2), n_layers=rnd.randint(1, 4))


def test_waterfill_bit_exact_with_oracle_on_random_cases():
    rnd = random.Random(5)
    for _ in range(600):
        n = rnd.randint(1, 8)
        nd = [rnd.randint(0, 300) for _ in range(n)]
        ctx = [rnd.randint(0, 100000) if nd[r] else 0 for r in range(n)]
        ex = [rnd.randint(0, 50) for _ in range(n)] if rnd.random() < 0.5 else None
        sel = [(rnd.randint(1, 400), rnd.randint(0, 5000)) for _ in range(rnd.randint(0, 2))]
        cand = (rnd.randint(0, 5000), rnd.randint(0, 20000)) if rnd.random() < 0.8 else None
        kw = dict(tau=rnd.uniform(50, 5000), n_decode_tokens=nd, decode_ctx_sum=ctx, existing=ex,
                  selected=sel, candidate=cand, quantum=rnd.choice([1, 8, 16, 64]), model=_rand_model(rnd),
                  fixed_target=rnd.choice([-1, -1, -1, rnd.randint(0, 1000)]),
                  level_hi=0 if cand else rnd.randint(0, 3000))
        assert X.xp_waterfill(**kw) == wf.dispatch(**kw)


def test_waterfill_bit_exact_on_the_c5_cases():
    for c in waterfill_cases():
        kw = dict(tau=c.tbt_slo, n_decode_tokens=c.n_decode_tokens, decode_ctx_sum=c.decode_ctx_sum,
                  existing=c.existing_assign, selected=c.selected, candidate=c.candidate, quantum=c.quantum,
                  model=c.model, fixed_target=c.fixed_target, level_hi=c.level_hi)
        r = X.xp_waterfill(**kw)
        assert r == wf.dispatch(**kw), c.name
        assert sum(r["assign"]) == r["chunk_len"]


def test_iteration_latency_bit_exact_with_oracle():
    rnd = random.Random(9)
    for _ in range(300):
        n = rnd.randint(1, 8)
        nd = [rnd.randint(0, 100) for _ in range(n)]
        cs = [rnd.randint(0, 10 ** 6) for _ in range(n)]
        npf = [rnd.randint(0, 2000) * rnd.randint(0, 1) for _ in range(n)]
        ch = [(rnd.randint(1, 4096), rnd.randint(0, 60000)) for _ in range(rnd.randint(0, 3))]
        m = _rand_model(rnd)
        assert X.xp_iteration_latency(m, nd, cs, npf, ch) == wf.iteration_latency(m, nd, cs, npf, ch)


def test_waterfill_rejects_bad_arguments():
    m = dict(gamma=1, gamma0=0, a_d=0, a_d0=0, a_p=0, a_p0=0, a_comm=0, a_comm0=0, alpha=1, beta=1, n_layers=1)
    with pytest.raises(X.XpError) as e:
        X.xp_waterfill(tau=1.0, n_decode_tokens=[1, 2], decode_ctx_sum=[0, 0], candidate=(10, 0), quantum=0, model=m)
    assert e.value.status == -1
    with pytest.raises(X.XpError):
        X.xp_waterfill(tau=1.0, n_decode_tokens=[-1, 2], decode_ctx_sum=[0, 0], candidate=(10, 0), model=m)


def _host_desc(inst, **over):
    wl = inst.wl
    fields = dict(x=1, n_prefill_local=wl.n_prefill_local, n_decode=wl.n_decode, dec_ctx=1, dec_pages=1,
                  dec_max_blocks=inst.dec_max_blocks, chunk_len=wl.chunk_len, prior_len=wl.prior_len,
                  sp_degree=wl.sp_degree, sp_rank=wl.sp_rank, local_row_offset=wl.local_row_offset,
                  pre_pages=1, pre_max_blocks=inst.pre_max_blocks, peer_qkv_in=1, peer_qkv_out=1,
                  peer_attn_in=1, peer_attn_out=1)
    fields.update(over)
    return X.BatchDesc(**fields)


def _shape(wl, **over):
    f = dict(hidden=wl.hidden, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
             ffn_dim=wl.ffn_dim, page_size=wl.page_size, rms_eps=wl.rms_eps, rope_base=wl.rope_base,
             dtype=X.XP_BF16 if wl.dtype == "bf16" else X.XP_F32)
    f.update(over)
    return X.LayerShape(**f)


def test_host_validation_accepts_generated_batches_and_rejects_broken_ones():
    inst = make_instance(get_workload("P1"))
    wl = inst.wl
    sh, d = _shape(wl), _host_desc(inst)
    ok = X.xp_validate_batch(sh, d, inst.pool.n_pages, inst.dec_ctx, inst.dec_pages, inst.pre_pages)
    assert ok == 0, X.xp_last_error()
    bad = inst.dec_pages.copy(); bad[1, 0, 0] = inst.pool.n_pages            # out of range
    assert X.xp_validate_batch(sh, d, inst.pool.n_pages, inst.dec_ctx, bad, inst.pre_pages) == -3
    dup = inst.pre_pages.copy(); dup[0, 1] = dup[0, 0]                        # a page named twice
    assert X.xp_validate_batch(sh, d, inst.pool.n_pages, inst.dec_ctx, inst.dec_pages, dup) == -3
    long_ctx = inst.dec_ctx.copy(); long_ctx[0] = inst.dec_max_blocks * 16    # table too short
    assert X.xp_validate_batch(sh, d, inst.pool.n_pages, long_ctx, inst.dec_pages, inst.pre_pages) == -3
    assert X.xp_validate_batch(_shape(wl, n_kv_heads=3), d, inst.pool.n_pages, inst.dec_ctx,
                               inst.dec_pages, inst.pre_pages) == -2          # Hq % Hkv != 0
    assert X.xp_validate_batch(sh, _host_desc(inst, sp_degree=3, sp_rank=0), inst.pool.n_pages,
                               inst.dec_ctx, inst.dec_pages, inst.pre_pages) == -2   # heads % P != 0
    assert X.xp_validate_batch(sh, _host_desc(inst, local_row_offset=150), inst.pool.n_pages,
                               inst.dec_ctx, inst.dec_pages, inst.pre_pages) == -2   # rows outside chunk
    assert X.xp_validate_batch(sh, _host_desc(inst, pre_max_blocks=3), inst.pool.n_pages,
                               inst.dec_ctx, inst.dec_pages, inst.pre_pages) == -3   # prefill table short
    assert X.xp_validate_batch(_shape(wl, head_dim=96), d, inst.pool.n_pages, inst.dec_ctx,
                               inst.dec_pages, inst.pre_pages) == -5
    assert X.xp_validate_batch(_shape(wl, page_size=32), d, inst.pool.n_pages, inst.dec_ctx,
                               inst.dec_pages, inst.pre_pages) == -5


def test_workspace_layout_is_host_only_and_consistent():
    for name in ("P1", "C2", "C5"):
        wl = get_workload(name)
        inst = make_instance(wl) if name == "P1" else None
        dmb = inst.dec_max_blocks if inst is not None else 4097
        d = X.BatchDesc(x=1, n_prefill_local=wl.n_prefill_local, n_decode=wl.n_decode, dec_ctx=1, dec_pages=1,
                        dec_max_blocks=dmb, chunk_len=wl.chunk_len, prior_len=wl.prior_len,
                        sp_degree=wl.sp_degree, sp_rank=wl.sp_rank, local_row_offset=wl.local_row_offset,
                        pre_pages=1, pre_max_blocks=-(-(wl.prior_len + wl.chunk_len) // 16), peer_qkv_in=1,
                        peer_qkv_out=1, peer_attn_in=1, peer_attn_out=1)
        L = X.xp_layer_workspace_layout(None, _shape(wl), d).as_dict()
        offs = sorted((v, k) for k, v in L.items() if k not in ("total", "dec_splits", "dec_pages_per_split"))
        assert all(o % 256 == 0 for o, _ in offs)
        assert offs[-1][0] < L["total"]
        pps = L["dec_pages_per_split"]
        assert 8 <= pps <= 64
        assert L["dec_splits"] == -(-dmb // pps)
        # the per-batch choice grows with the decode work and saturates at 64
        expect = min(64, max(8, wl.n_decode * wl.n_kv_heads * dmb // 1600))
        assert pps == expect, (name, pps, expect)


def test_decode_workspace_size_matches_layer_layout():
    # host-only: the kernel-level size for a split choice equals the layer layout's regions
    wl = get_workload("C2")
    for pps in (0, 1, 8, 64):
        n = X.xp_decode_workspace_size(wl.n_decode, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, 513, pps)
        splits = -(-513 // (pps or min(64, max(8, wl.n_decode * wl.n_kv_heads * 513 // 1600))))
        units = wl.n_decode * wl.n_q_heads * splits
        assert n == -(-units * 8 // 256) * 256 + -(-units * wl.head_dim * 4 // 256) * 256
    assert X.xp_decode_workspace_size(0, 8, 2, 128, 10, 0) == 0
    assert X.xp_decode_workspace_size(4, 8, 2, 128, 10, -1) == 0


# The work unit the launcher picks for the QKV, O, gate/up and down projections of the
# 8B (1040 and 128 rows), 14B (536 and 8216 rows) and 32B (544 rows) layer shapes: the
# fastest tile measured on MI355X for each (the 14B gate/up projection: within 1%).
LAYER_TILES = [
    # (epilogue, M, N, K) -> (rows, cols, K splits)
    ((X.XP_EPI_F32, 1040, 6144, 4096), (128, 256, 1)), ((X.XP_EPI_ADD_T, 1040, 4096, 4096), (192, 128, 1)),
    ((X.XP_EPI_SWIGLU, 1040, 14336, 4096), (128, 128, 1)), ((X.XP_EPI_ADD_F32, 1040, 4096, 14336), (192, 128, 1)),
    ((X.XP_EPI_F32, 536, 7168, 5120), (192, 128, 1)), ((X.XP_EPI_ADD_T, 536, 5120, 5120), (96, 128, 1)),
    ((X.XP_EPI_SWIGLU, 536, 17408, 5120), (128, 128, 1)), ((X.XP_EPI_ADD_F32, 536, 5120, 17408), (192, 192, 3)),
    ((X.XP_EPI_F32, 128, 6144, 4096), (64, 128, 1)), ((X.XP_EPI_ADD_T, 128, 4096, 4096), (64, 128, 1)),
    ((X.XP_EPI_SWIGLU, 128, 14336, 4096), (128, 64, 1)), ((X.XP_EPI_ADD_F32, 128, 4096, 14336), (64, 128, 4)),
    ((X.XP_EPI_F32, 544, 10240, 5120), (192, 128, 1)), ((X.XP_EPI_ADD_T, 544, 5120, 8192), (96, 128, 1)),
    ((X.XP_EPI_SWIGLU, 544, 25600, 5120), (128, 128, 1)), ((X.XP_EPI_ADD_F32, 544, 5120, 25600), (192, 192, 3)),
    ((X.XP_EPI_F32, 8216, 7168, 5120), (256, 256, 1)), ((X.XP_EPI_SWIGLU, 8216, 17408, 5120), (256, 128, 1)),
]


def test_gemm_tile_choice_on_the_layer_shapes():
    # host-only (no device visible here: the launcher assumes 256 CUs)
    for (epi, M, N, K), want in LAYER_TILES:
        assert X.xp_gemm_tile(X.XP_BF16, epi, M, N, K) == want, (epi, M, N, K)
    with pytest.raises(X.XpError):
        X.xp_gemm_tile(X.XP_BF16, 9, 64, 64, 64)
    with pytest.raises(X.XpError):
        X.xp_gemm_tile(X.XP_BF16, X.XP_EPI_F32, 0, 64, 64)


def test_gemm_workspace_follows_the_split_choice():
    # host-only: long-K products are summed over K chunks that follow the weight shape
    # (N, K); few rows run one unit per chunk, whose fp32 partials take chunks x weights
    # x M x N, and many rows fold the chunks inside one unit per tile (no workspace)
    for M in (16, 300):
        assert X.xp_gemm_workspace_size(X.XP_BF16, X.XP_EPI_ADD_F32, M, 4096, 14336) == 4 * M * 4096 * 4
        assert X.xp_gemm_workspace_size(X.XP_BF16, X.XP_EPI_ADD_F32, M, 5120, 25600) == 3 * M * 5120 * 4
    assert X.xp_gemm_workspace_size(X.XP_BF16, X.XP_EPI_ADD_F32, 1040, 4096, 14336) == 0
    assert X.xp_gemm_tile(X.XP_BF16, X.XP_EPI_ADD_F32, 1040, 4096, 14336)[2] == 1
    for M in (16, 300, 1040):
        assert X.xp_gemm_workspace_size(X.XP_BF16, X.XP_EPI_F32, M, 6144, 4096) == 0     # K < 3N: not chunked
        assert X.xp_gemm_workspace_size(X.XP_BF16, X.XP_EPI_SWIGLU, M, 14336, 4096) == 0
        assert X.xp_gemm_workspace_size(X.XP_BF16, X.XP_EPI_SWIGLU, M, 512, 4096) == 4 * 2 * M * 512 * 4
    assert X.xp_gemm_workspace_size(X.XP_BF16, X.XP_EPI_F32, 64, 512, 512) == 0   # too few K stages
    assert X.xp_gemm_workspace_size(X.XP_BF16, 9, 64, 512, 4096) == 0


def test_gemm_rejects_unsupported_k_before_launching():
    with pytest.raises(X.XpError) as e:
        X.xp_gemm(X.XP_BF16, X.XP_EPI_F32, 16, 16, None, None, 16, 4, 4, 100, stream=0)
    assert e.value.status == -5
    with pytest.raises(X.XpError):
        X.xp_gemm(X.XP_BF16, 9, 16, 16, None, None, 16, 4, 4, 64, stream=0)


# ---- SLO-aware scheduler (Algorithms 1, 3, 4) ---------------------------------------

def _sched_case(rnd):
    N, R = rnd.randint(1, 8), rnd.randint(0, 24)
    nd = [rnd.randint(0, 64) for _ in range(N)]
    return dict(n_decode_tokens=nd, decode_ctx_sum=[rnd.randint(0, 200000) * (n > 0) for n in nd],
                kv_used=[rnd.randint(0, 400000) for _ in range(N)],
                kv_capacity=[rnd.randint(300000, 600000) for _ in range(N)],
                m_remaining=[rnd.randint(1, 20000) for _ in range(R)],
                c_processed=[rnd.choice([0, 0, rnd.randint(1, 30000)]) for _ in range(R)],
                deadlines=[rnd.uniform(-0.5, 3.0) for _ in range(R)], now=0.0,
                tau=rnd.uniform(0.02, 0.3), quantum=rnd.choice([1, 8, 16, 64]), eta=rnd.uniform(0.2, 1.0),
                headroom=rnd.choice([0, 1024, 8192]), model=_rand_model(rnd))


def test_schedule_bit_exact_with_oracle_on_random_iterations():
    from oracle import scheduler as sch
    rnd = random.Random(21)
    stops, selected = {}, 0
    for _ in range(300):
        c = _sched_case(rnd)
        # keep the synthetic coefficients in a range where some chunks fit
        c["model"] = dict(c["model"], gamma=c["model"]["gamma"] * 1e-6, gamma0=c["model"]["gamma0"] * 1e-4,
                          a_d=c["model"]["a_d"] * 1e-8, a_d0=c["model"]["a_d0"] * 1e-4,
                          a_p=c["model"]["a_p"] * 1e-10, a_p0=c["model"]["a_p0"] * 1e-4,
                          a_comm=c["model"]["a_comm"] * 1e-7, a_comm0=c["model"]["a_comm0"] * 1e-4)
        got = X.xp_schedule(**c)
        assert got == sch.schedule(**c)
        stops[got["stop"]] = stops.get(got["stop"], 0) + 1
        selected += got["n_selected"] > 0
    # the cases reach every way an iteration can end, and most select something
    assert set(stops) == {"done", "budget", "no_host"} and selected > 150


@pytest.mark.parametrize("depth", [10, 50, 100, 500])
def test_schedule_bit_exact_on_synthetic_queues(depth):
    import dataclasses
    from oracle import scheduler as sch
    from synth import scheduler_case
    for seed in range(3):
        c = dataclasses.asdict(scheduler_case(depth, seed=seed))
        c.pop("name")
        got = X.xp_schedule(**c)
        assert got == sch.schedule(**c)
        assert got["n_selected"] > 0


def test_admission_and_placement_bit_exact_with_oracle():
    from oracle import scheduler as sch
    rnd = random.Random(8)
    for _ in range(500):
        R = rnd.randint(0, 30)
        m = [rnd.randint(1, 50) for _ in range(R)]
        d = [rnd.choice([rnd.uniform(-1, 10), float(rnd.randint(0, 6))]) for _ in range(R)]
        b0, tau, now = rnd.randint(0, 60), rnd.choice([0.5, 1.0, 0.3]), rnd.choice([0.0, 0.7])
        assert X.xp_admission(m, d, b0, now, tau) == sch.admission(m, d, b0, now, tau)
        N = rnd.randint(1, 8)
        cap = [rnd.randint(100, 2000) for _ in range(N)]
        used = [rnd.randint(0, c) for c in cap]
        ctx = [rnd.randint(0, 50) for _ in range(N)]
        need, eta, h = rnd.randint(0, 400), rnd.uniform(0, 1), rnd.choice([0, 50])
        assert X.xp_decode_placement(ctx, used, cap, need, eta, h) == sch.placement(ctx, used, cap, need, eta, h)


def test_scheduler_rejects_bad_arguments():
    good = dict(n_decode_tokens=[1, 2], decode_ctx_sum=[10, 20], kv_used=[0, 0], kv_capacity=[100, 100],
                m_remaining=[5], c_processed=[0], deadlines=[1.0], now=0.0, tau=0.1, quantum=1, eta=0.5,
                headroom=0, model=_rand_model(random.Random(0)))
    X.xp_schedule(**good)
    for bad in (dict(kv_capacity=[100, 0]), dict(m_remaining=[0]), dict(c_processed=[-1]),
                dict(deadlines=[float("nan")]), dict(tau=0.0), dict(quantum=0), dict(headroom=-1),
                dict(n_decode_tokens=[-1, 2])):
        with pytest.raises(X.XpError) as e:
            X.xp_schedule(**dict(good, **bad))
        assert e.value.status == -1
    with pytest.raises(X.XpError):
        X.xp_admission([3], [1.0], -1, 0.0, 1.0)
    with pytest.raises(X.XpError):
        X.xp_decode_placement([0], [0], [10], -5, 0.5, 0)
    assert X.xp_decode_placement([0], [95], [100], 10, 0.5, 0) is None      # Infeasible is a result


# ---- latency-estimator fitting ---------------------------------------------------------

def _noisy_profile(rnd, a, b, lo, hi, n):
    x = [rnd.uniform(lo, hi) for _ in range(n)]
    return x, [(a * v + b) * rnd.uniform(0.85, 1.2) for v in x]


def test_fit_affine_agrees_with_oracle():
    from oracle import estimator as est
    rnd = random.Random(31)
    for _ in range(300):
        n = rnd.randint(0, 40)
        scale = 10 ** rnd.uniform(0, 9)
        x, t = _noisy_profile(rnd, rnd.uniform(1e-12, 1e-6), rnd.uniform(1e-6, 1e-3), 1, scale, n)
        if rnd.random() < 0.1 and n:
            x = [x[0]] * n
        ga, gb = X.xp_fit_affine(x, t)
        oa, ob = est.fit_affine(x, t)
        assert ga == pytest.approx(oa, rel=1e-8, abs=1e-300) and gb == pytest.approx(ob, rel=1e-8, abs=1e-300)


def test_fit_latency_model_agrees_with_oracle():
    from oracle import estimator as est
    rnd = random.Random(32)
    for _ in range(20):
        gemm = _noisy_profile(rnd, 2e-7, 3e-5, 16, 10000, 20)
        dec = _noisy_profile(rnd, 8e-10, 1e-5, 1000, 2e6, 20)
        pre = _noisy_profile(rnd, 6e-11, 9e-6, 500, 5e7, 20)
        comm = _noisy_profile(rnd, 1e-8, 5e-6, 16, 5000, rnd.choice([0, 10]))
        mixed = []
        for _ in range(rnd.randint(0, 30)):
            g, d, p = rnd.randint(64, 10000), rnd.choice([-1.0, rnd.uniform(1e3, 2e6)]), rnd.choice([-1.0, rnd.uniform(5e2, 5e7)])
            tg = 2e-7 * g + 3e-5
            t = tg + max(1.4 * (6e-11 * p + 9e-6) * (p >= 0), 1.2 * (8e-10 * d + 1e-5) * (d >= 0))
            mixed.append((g, d, p, rnd.uniform(16, 5000), t * rnd.uniform(0.9, 1.1)))
        got = X.xp_fit_latency_model(gemm, dec, pre, comm, mixed, n_layers=1, ab_max=2.5)
        ref = est.fit_model(gemm, dec, pre, comm, mixed, n_layers=1, ab_max=2.5)
        for k in ("gamma", "gamma0", "a_d", "a_d0", "a_p", "a_p0", "a_comm", "a_comm0"):
            assert got[k] == pytest.approx(ref[k], rel=1e-8, abs=1e-300), k
        assert (got["alpha"], got["beta"], got["n_layers"]) == (ref["alpha"], ref["beta"], 1)


def test_fit_rejects_bad_samples():
    with pytest.raises(X.XpError):
        X.xp_fit_affine([1.0, 2.0], [1.0, 0.0])
    with pytest.raises(X.XpError):
        X.xp_fit_latency_model(([], []), ([], []), ([], []), ([], []), [], n_layers=0)
    with pytest.raises(X.XpError):
        X.xp_fit_latency_model(([], []), ([], []), ([], []), ([], []), [(1, 1, 1, 1, -1.0)])


def test_chunk_list_layout_is_host_only_and_validated():
    shape = X.layer_shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn_dim=1024)
    x = np.zeros((300, 512), dtype=np.uint16)
    t1, t2 = np.zeros((2, 7), dtype=np.int32), np.zeros((2, 30), dtype=np.int32)

    class T:  # table stand-in: only the address and the block count reach the library
        def __init__(self, a):
            self.a, self.shape = a, a.shape

        def data_ptr(self):
            return self.a.ctypes.data

        def dim(self):
            return self.a.ndim

    desc = X.batch_desc(x=x.ctypes.data, n_prefill_local=0, n_decode=0, dec_ctx=None, dec_pages=None,
                        chunk_len=0, prior_len=0)
    ok = X.chunk_array([(97, 0, T(t1)), (203, 270, T(t2))])
    L = X.xp_layer_workspace_layout_chunks(None, shape, desc, ok)
    L1 = X.xp_layer_workspace_layout(None, shape, X.batch_desc(x=x.ctypes.data, n_prefill_local=300, n_decode=0,
                                                               dec_ctx=None, dec_pages=None, chunk_len=300,
                                                               prior_len=0, pre_pages=T(t2)))
    assert L.q_pre == L1.q_pre and L.attn - L.q_pre == L1.attn - L1.q_pre     # same rows, same query bytes
    with pytest.raises(X.XpError) as e:                                      # 270 + 203 > 30 blocks * 16
        X.xp_layer_workspace_layout_chunks(None, shape, desc, X.chunk_array([(203, 280, T(t2))]))
    assert e.value.status == -3
    sp2 = X.batch_desc(x=x.ctypes.data, n_prefill_local=0, n_decode=0, dec_ctx=None, dec_pages=None, chunk_len=0,
                       prior_len=0, sp_degree=2)
    with pytest.raises(X.XpError) as e:
        X.xp_layer_workspace_layout_chunks(None, shape, sp2, ok)
    assert e.value.status == -5
    with pytest.raises(X.XpError):
        X.xp_layer_workspace_layout_chunks(None, shape, desc, X.chunk_array([(0, 0, T(t1))]))


def test_chunk_tables_are_validated_on_the_host():
    from synth import MULTI_CHUNK_WORKLOADS, make_multi_instance
    inst = make_multi_instance(MULTI_CHUNK_WORKLOADS["M4"])
    wl = inst.wl
    shape = X.layer_shape(hidden=wl.hidden, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                          ffn_dim=wl.ffn_dim)

    class T:  # host table stand-in: only the address and the block count reach the structs
        def __init__(self, a):
            self.a, self.shape = a, a.shape

        def data_ptr(self):
            return self.a.ctypes.data

        def dim(self):
            return self.a.ndim

    dec_pages = inst.dec_pages
    desc = X.batch_desc(x=inst.x.ctypes.data, n_prefill_local=0, n_decode=wl.n_decode, dec_ctx=T(inst.dec_ctx),
                        dec_pages=T(dec_pages), chunk_len=0, prior_len=0)
    chunks = X.chunk_array([(l, c, T(t)) for (l, c), t in zip(wl.chunks, inst.chunk_pages)])
    n = inst.pool.n_pages
    assert X.xp_validate_chunks(shape, desc, chunks, n, inst.dec_ctx, dec_pages, inst.chunk_pages) == 0
    bad = [t.copy() for t in inst.chunk_pages]
    bad[9][1, 0] = n                                                   # outside the pool
    assert X.xp_validate_chunks(shape, desc, chunks, n, inst.dec_ctx, dec_pages, bad) == -3
    bad = [t.copy() for t in inst.chunk_pages]
    bad[3][0, 1] = int(inst.chunk_pages[0][0, 0])                      # named twice
    assert X.xp_validate_chunks(shape, desc, chunks, n, inst.dec_ctx, dec_pages, bad) == -3


def test_calibration_entry_points_check_their_arguments_on_the_host():
    # every check below fails before the library touches a device
    L = X.lib()
    import ctypes as C
    cv = X.CuCurve()
    kk = C.c_int32()
    args = [0, X.XP_BF16, 1, 1, 10, 16, 1, 4, 1, 2, 8, 2, 128, 1, 1024, 1, 0]
    assert L.xp_calibrate_decode_cus(*args, 0.9, 32, 5, 1, None, C.byref(cv)) == -1       # null output
    assert L.xp_calibrate_decode_cus(*args, 1.5, 32, 5, 1, C.byref(kk), C.byref(cv)) == -1  # fraction > 1
    assert L.xp_calibrate_decode_cus(*args, 0.9, 0, 5, 1, C.byref(kk), C.byref(cv)) == -1   # cu_step 0
    assert L.xp_calibrate_decode_cus(*args, 0.9, 32, 0, 1, C.byref(kk), C.byref(cv)) == -1  # no repeats
    assert L.xp_probe_read_curve(0, 1, 15, 1, 32, 5, C.byref(cv)) == -1                     # bytes % 16
    assert L.xp_probe_read_curve(0, None, 16, 1, 32, 5, C.byref(cv)) == -1
    assert "xp_probe_read_curve" in X.xp_last_error()
