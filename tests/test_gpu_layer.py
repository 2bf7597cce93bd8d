"""Layer-step parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: attention rows and exported peer buffers rel-Frobenius <= 5e-3; bf16 layer outputs
(fp32 residual stream) rel-Frobenius <= 5e-3 end to end, and on the last stage (out =
h1 + act W_down^T from the GPU's own h1 and act) a max-abs error at most TF_FACTOR times that
of an independent fp32 product of the same operands (tests.helpers.down_stage_errors); fp32
layer outputs max-abs <= 2e-2 end to end.  Pages no append touches stay bit-identical.
"""
import json
import os

import numpy as np
import pytest
import torch

import mixed_prefill_decode_amd as X
from oracle import layer as L
from oracle.numerics import to_f64
from synth import get_workload, make_instance
from synth.device import make_step, to_host_bits, upload
from tests.helpers import down_stage_errors, oracle_kwargs, rel_fro, shared_ctx, k_slots

pytestmark = pytest.mark.gpu

SMALL = ["P1", "P2", "P3", "P4", "P5", "P6", "E1", "E2", "E3", "E4", "C1"]
ctx = shared_ctx


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def record(name, metrics):
    """Appends a parity record to $XP_METRICS_OUT (a JSON-lines file) when it is set."""
    path = os.environ.get("XP_METRICS_OUT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(case=name, **metrics)) + "\n")


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def check_layer(inst, step, ref, rows=None):
    wl, dt = inst.wl, inst.wl.dtype
    M, H, Hq, d, F = wl.n_rows, wl.hidden, wl.n_q_heads, wl.head_dim, wl.ffn_dim
    rows = np.arange(M) if rows is None else np.asarray(rows)
    out = step.out.cpu().numpy().astype(np.float64)
    attn = to_f64(to_host_bits(step.ws_view("attn", (M, Hq * d), _tdt(dt))), dt)
    h1 = step.ws_view("h1", (M, H), torch.float32).cpu().numpy().astype(np.float64)
    act = to_f64(to_host_bits(step.ws_view("act", (M, F), _tdt(dt))), dt)
    assert step.status() == 0
    assert np.isfinite(out).all()
    r = dict(attn=rel_fro(attn[rows], ref["attn"][rows]), out=rel_fro(out[rows], ref["out"][rows]),
             out_maxabs=float(np.abs(out[rows] - ref["out"][rows]).max()))
    # teacher-forced last stage
    r["tf_maxabs"], r["tf_f32_maxabs"], tf_bar = down_stage_errors(out[rows], h1[rows], act[rows],
                                                                   to_f64(inst.weights["w_down"], dt))
    assert r["attn"] < 5e-3, r
    assert r["tf_maxabs"] <= tf_bar, r
    if dt == "f32":
        assert r["out_maxabs"] < 2e-2, r
    else:
        assert r["out"] < 5e-3, r
    return r


@pytest.mark.parametrize("name", SMALL)
def test_layer_matches_oracle(name):
    inst = make_instance(get_workload(name))
    wl, dt = inst.wl, inst.wl.dtype
    step, dev = make_step(inst, ctx(0))
    step.run()
    torch.cuda.synchronize()
    ref = L.layer_forward(**oracle_kwargs(inst))
    r = check_layer(inst, step, ref)
    record(name, r)
    # exported stand-in buffers
    if wl.chunk_len - wl.n_prefill_local > 0:
        got = to_f64(to_host_bits(dev.peer_attn_out), dt)
        assert rel_fro(got, ref["peer_attn_out"]) < 5e-3
    if wl.sp_degree > 1 and wl.n_prefill_local > 0:
        got = to_f64(to_host_bits(dev.peer_qkv_out), dt)
        assert rel_fro(got, ref["peer_qkv_out"]) < 5e-3
    # the pool: appended slots close to the oracle's, every other slot bit-identical
    pool = to_host_bits(dev.pool)
    kv = ref["kv"]
    S, dd = wl.page_size, wl.head_dim
    for p in range(inst.pool.n_pages):
        want = kv.stored_page(p)
        if p not in kv.overlay:
            assert pool[p].tobytes() == inst.pool[[p]][0].tobytes(), p
            continue
        gk, gv = k_slots(pool[p, 0], S, dd, dt), pool[p, 1].reshape(dd, S).T
        wk, wv = k_slots(want[0], S, dd, dt), want[1].reshape(dd, S).T
        same = np.all(_bits(gk) == _bits(wk), axis=1) & np.all(_bits(gv) == _bits(wv), axis=1)
        for s in np.nonzero(~same)[0]:      # appended slots: values within bf16 rounding of the oracle's
            a = np.concatenate([to_f64(gk[s], dt), to_f64(gv[s], dt)])
            b = np.concatenate([to_f64(wk[s], dt), to_f64(wv[s], dt)])
            assert np.isfinite(a).all() and rel_fro(a, b) < 1e-2, (p, s)


def test_split_attention_modes_agree():
    """Serialized, unmasked and CU-partitioned steps: decode rows bit-identical (the
    dense path is batch invariant and decode's splits do not depend on the mode); the
    prefill rows and the exported peer rows within merge-order rounding (a partition's
    prefill plans its key splits for the CUs it has)."""
    inst = make_instance(get_workload("P1"))
    n_pl = inst.wl.n_prefill_local
    outs = []
    for mode in (0, -1, 64):
        step, dev = make_step(inst, ctx(mode))
        step.run()
        torch.cuda.synchronize()
        assert step.status() == 0
        outs.append((step.out.clone(), dev.peer_attn_out.clone()))
    for o, p in outs[1:]:
        assert torch.equal(o[n_pl:], outs[0][0][n_pl:])
        assert rel_fro(o.cpu().numpy(), outs[0][0].cpu().numpy()) < 1e-3
        assert rel_fro(p.float().cpu().numpy(), outs[0][1].float().cpu().numpy()) < 1e-3


def test_stage_timing_counts_and_leaves_results_unchanged():
    """xp_ctx_stage_timing: the first `capacity` runs of every stage are timed (on the
    attention streams too in a partitioned context), later runs are not, and timing
    changes no bit of the step's output."""
    inst = make_instance(get_workload("P1"))
    for mode in (0, 64):
        c = X.Ctx(0, mode, 0)
        try:
            step, dev = make_step(inst, c)
            ref = step.run().clone()
            c.stage_timing(3)
            for _ in range(4):
                out = step.run()
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
            t = c.stage_times()
            assert set(t) == set(X.STAGES)
            for name, (n, ms) in t.items():
                assert n == 3 and ms >= 0, (mode, name, n, ms)
            for name in ("norm1", "qkv", "rope_append", "decode", "prefill", "o", "norm2", "gate_up", "down"):
                assert t[name][1] > 0, (mode, name)
            c.stage_timing(0)
            step.run()
            torch.cuda.synchronize()
            assert all(n == 0 for n, _ in c.stage_times().values())
            with pytest.raises(X.XpError):
                c.stage_timing(-1)
        finally:
            c.close()


def test_repeat_calls_are_deterministic_and_idempotent():
    inst = make_instance(get_workload("P3"))
    step, dev = make_step(inst, ctx(0))
    a = step.run().clone()
    b = step.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_cobatched_rows_equal_separate_batches_on_gpu():
    inst = make_instance(get_workload("P1"))
    wl = inst.wl
    n_pl = wl.n_prefill_local
    step, dev = make_step(inst, ctx(0))
    full = step.run().clone()
    sh = step.shape
    w = step.weights
    pre_desc = X.batch_desc(x=dev.x, n_prefill_local=n_pl, n_decode=0, dec_ctx=None, dec_pages=None,
                            chunk_len=wl.chunk_len, prior_len=wl.prior_len, sp_degree=wl.sp_degree,
                            sp_rank=wl.sp_rank, local_row_offset=wl.local_row_offset, pre_pages=dev.pre_pages,
                            peer_qkv_in=dev.peer_qkv_in, peer_qkv_out=dev.peer_qkv_out,
                            peer_attn_in=dev.peer_attn_in, peer_attn_out=dev.peer_attn_out)
    xd = dev.x[n_pl:].contiguous()
    dec_desc = X.batch_desc(x=xd, n_prefill_local=0, n_decode=wl.n_decode, dec_ctx=dev.dec_ctx,
                            dec_pages=dev.dec_pages, chunk_len=0, prior_len=0)
    pre = X.LayerStep(ctx(0), sh, pre_desc, w, dev.pool, inst.pool.n_pages, keep=(dev,))
    dec = X.LayerStep(ctx(0), sh, dec_desc, w, dev.pool, inst.pool.n_pages, keep=(dev, xd))
    a, b = pre.run().clone(), dec.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(full[:n_pl], a)
    assert torch.equal(full[n_pl:], b)


def test_out_of_range_page_is_flagged_not_dereferenced():
    inst = make_instance(get_workload("E1"))
    step, dev = make_step(inst, ctx(0))
    bad = dev.dec_pages.clone()
    bad[2, 1, 0] = inst.pool.n_pages + 1000
    desc = X.batch_desc(x=dev.x, n_prefill_local=0, n_decode=inst.wl.n_decode, dec_ctx=dev.dec_ctx,
                        dec_pages=bad, chunk_len=0, prior_len=0)
    s2 = X.LayerStep(ctx(0), step.shape, desc, step.weights, dev.pool, inst.pool.n_pages, keep=(dev, bad))
    out = s2.run()
    torch.cuda.synchronize()
    assert s2.status() & X.XP_DEV_BAD_PAGE
    o = out.cpu().numpy()
    assert np.isnan(o[2]).any()                       # the affected request is poisoned
    assert np.isfinite(np.delete(o, 2, axis=0)).all()  # the others are not


def test_host_validation_rejects_before_launch():
    inst = make_instance(get_workload("P1"))
    step, dev = make_step(inst, ctx(0))
    desc = X.batch_desc(x=dev.x, n_prefill_local=inst.wl.n_prefill_local, n_decode=inst.wl.n_decode,
                        dec_ctx=dev.dec_ctx, dec_pages=dev.dec_pages, chunk_len=inst.wl.chunk_len,
                        prior_len=inst.wl.prior_len, sp_degree=3, sp_rank=0, pre_pages=dev.pre_pages)
    with pytest.raises(X.XpError) as e:
        X.xp_layer_forward(step.ctx, step.shape, desc, step.weights, step.kv, step.out, step.workspace,
                           step.layout.total)
    assert e.value.status == -2
    with pytest.raises(X.XpError) as e:
        X.xp_layer_forward(step.ctx, step.shape, step.desc, step.weights, step.kv, step.out, step.workspace,
                           step.layout.total - 256)
    assert e.value.status == -6


def test_cu_masks_partition_the_chip():
    c = ctx(64)
    dec, pre, n = c.cu_masks()
    bits_d = sum(bin(w).count("1") for w in dec)
    bits_p = sum(bin(w).count("1") for w in pre)
    assert bits_d == 64 and bits_d + bits_p == n
    assert all((a & b) == 0 for a, b in zip(dec, pre))


def test_host_table_copies_validate_before_launch():
    """With host copies of its tables the step checks every page id on the host and
    launches nothing on a bad one (XP_EPAGE); without them the device check flags it."""
    inst = make_instance(get_workload("P1"))
    ref_step, dev = make_step(inst, ctx(0))
    ref = ref_step.run().clone()
    torch.cuda.synchronize()
    step, _ = make_step(inst, ctx(0), dev, host_tables=True)
    got = step.run()
    torch.cuda.synchronize()
    assert step.status() == 0
    assert torch.equal(got, ref)                       # valid copies: the same step
    wl = inst.wl
    for what in ("range", "twice", "short"):
        dec_pages, pre_pages, dec_ctx = inst.dec_pages.copy(), inst.pre_pages.copy(), inst.dec_ctx.copy()
        if what == "range":
            dec_pages[1, 0, 0] = inst.pool.n_pages
        elif what == "twice":
            pre_pages[0, 1] = pre_pages[0, 0]
        else:
            dec_ctx[0] = inst.dec_max_blocks * wl.page_size
        desc = X.batch_desc(x=dev.x, n_prefill_local=wl.n_prefill_local, n_decode=wl.n_decode,
                            dec_ctx=dev.dec_ctx, dec_pages=dev.dec_pages, chunk_len=wl.chunk_len,
                            prior_len=wl.prior_len, sp_degree=wl.sp_degree, sp_rank=wl.sp_rank,
                            local_row_offset=wl.local_row_offset, pre_pages=dev.pre_pages,
                            peer_qkv_in=dev.peer_qkv_in, peer_qkv_out=dev.peer_qkv_out,
                            peer_attn_in=dev.peer_attn_in, peer_attn_out=dev.peer_attn_out,
                            dec_ctx_host=dec_ctx, dec_pages_host=dec_pages, pre_pages_host=pre_pages)
        pool0 = dev.pool.clone()
        step.out.fill_(7.0)
        torch.cuda.synchronize()
        with pytest.raises(X.XpError) as e:
            X.xp_layer_forward(step.ctx, step.shape, desc, step.weights, step.kv, step.out, step.workspace,
                               step.layout.total)
        torch.cuda.synchronize()
        assert e.value.status == -3, what
        assert bool((step.out == 7.0).all()), what           # nothing was launched
        assert torch.equal(dev.pool.view(torch.int16), pool0.view(torch.int16)), what
    # copies of only some of the tables the step reads
    part = X.batch_desc(x=dev.x, n_prefill_local=wl.n_prefill_local, n_decode=wl.n_decode, dec_ctx=dev.dec_ctx,
                        dec_pages=dev.dec_pages, chunk_len=wl.chunk_len, prior_len=wl.prior_len,
                        sp_degree=wl.sp_degree, sp_rank=wl.sp_rank, local_row_offset=wl.local_row_offset,
                        pre_pages=dev.pre_pages, peer_qkv_in=dev.peer_qkv_in, peer_qkv_out=dev.peer_qkv_out,
                        peer_attn_in=dev.peer_attn_in, peer_attn_out=dev.peer_attn_out,
                        dec_ctx_host=inst.dec_ctx, dec_pages_host=inst.dec_pages)
    with pytest.raises(X.XpError) as e:
        X.xp_layer_forward(step.ctx, step.shape, part, step.weights, step.kv, step.out, step.workspace,
                           step.layout.total)
    assert e.value.status == -1


def test_ctx_create_rejects_out_of_range_decode_cus():
    n = ctx(0).cu_masks()[2]
    for k in (n, n + 5, -2):
        with pytest.raises(X.XpError) as e:
            X.Ctx(0, k, 0)
        assert e.value.status == -1
        assert str(n - 1) in str(e.value)


def test_calibrate_decode_cus_through_the_abi():
    """The pages' rule measured by the library: the chosen k is the first CU count whose
    decode time is within 1/0.9 of the all-CU time (or the largest tried), and the
    calibration's launches compute what a plain decode-attention call computes."""
    inst = make_instance(get_workload("E1"))
    step, dev = make_step(inst, ctx(0))
    step.run()
    torch.cuda.synchronize()
    wl, lay = inst.wl, step.layout
    q = int(step.workspace.data_ptr()) + lay.q_dec
    dws = torch.empty(X.xp_decode_workspace_size(wl.n_decode, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                                 inst.dec_max_blocks, 0), dtype=torch.uint8, device="cuda")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dt = X.XP_BF16 if wl.dtype == "bf16" else X.XP_F32
    ref = torch.empty((wl.n_decode, wl.n_q_heads * wl.head_dim), dtype=tdt, device="cuda")
    X.xp_decode_attention(dt, q, dev.pool, inst.pool.n_pages, wl.page_size, dev.dec_pages, inst.dec_max_blocks,
                          dev.dec_ctx, wl.n_decode, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, ref,
                          wl.n_q_heads * wl.head_dim, dws, 0)
    torch.cuda.synchronize()
    out = torch.full_like(ref, float("nan"))
    k, curve = X.xp_calibrate_decode_cus(0, dt, q, dev.pool, inst.pool.n_pages, wl.page_size, dev.dec_pages,
                                         inst.dec_max_blocks, dev.dec_ctx, wl.n_decode, wl.n_q_heads,
                                         wl.n_kv_heads, wl.head_dim, out, wl.n_q_heads * wl.head_dim, dws,
                                         keep_fraction=0.9, cu_step=64, repeats=3, stop_at_rule=False)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    pts = curve["points"]
    assert sorted(pts) == list(range(64, curve["n_cus"], 64))
    ok = [c for c in sorted(pts) if curve["us_all"] >= 0.9 * pts[c]]
    assert k == (ok[0] if ok else max(pts))
    assert all(t > 0 for t in pts.values()) and curve["us_all"] > 0
    with pytest.raises(X.XpError):
        X.xp_calibrate_decode_cus(0, dt, q, dev.pool, inst.pool.n_pages, wl.page_size, dev.dec_pages,
                                  inst.dec_max_blocks, dev.dec_ctx, wl.n_decode, wl.n_q_heads, wl.n_kv_heads,
                                  wl.head_dim, out, wl.n_q_heads * wl.head_dim, dws, keep_fraction=1.5)


def test_probe_read_curve_through_the_abi():
    buf = torch.zeros(1 << 26, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    curve = X.xp_probe_read_curve(0, buf, buf.numel(), sink, cu_step=128, repeats=2)
    assert sorted(curve["points"]) == list(range(128, curve["n_cus"], 128))
    assert int(sink.item()) == 0                       # zeros never reach the sink
