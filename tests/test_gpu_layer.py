"""Layer-step parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: attention rows and exported peer buffers rel-Frobenius <= 5e-3; bf16 layer outputs
(fp32 residual stream) rel-Frobenius <= 5e-3 end to end, and max-abs <= 2e-2 teacher-forced
on the last stage (out = h1 + act W_down^T recomputed in fp64 from the GPU's own h1 and act);
fp32 layer outputs max-abs <= 2e-2 end to end.  Pages no append touches stay bit-identical.
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
from tests.helpers import oracle_kwargs, rel_fro

pytestmark = pytest.mark.gpu

SMALL = ["P1", "P2", "P3", "P4", "P5", "P6", "E1", "E2", "E3", "E4", "C1"]
_CTX = {}


def ctx(decode_cus=0):
    if decode_cus not in _CTX:
        _CTX[decode_cus] = X.Ctx(0, decode_cus, 0)
    return _CTX[decode_cus]


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
    wd = to_f64(inst.weights["w_down"], dt)
    tf = h1[rows] + act[rows] @ wd.T
    r["tf_maxabs"] = float(np.abs(out[rows] - tf).max())
    assert r["attn"] < 5e-3, r
    assert r["tf_maxabs"] < 2e-2, r
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
        gk, gv = pool[p, 0].reshape(S, dd), pool[p, 1].reshape(dd, S).T
        wk, wv = want[0].reshape(S, dd), want[1].reshape(dd, S).T
        same = np.all(_bits(gk) == _bits(wk), axis=1) & np.all(_bits(gv) == _bits(wv), axis=1)
        for s in np.nonzero(~same)[0]:      # appended slots: values within bf16 rounding of the oracle's
            a = np.concatenate([to_f64(gk[s], dt), to_f64(gv[s], dt)])
            b = np.concatenate([to_f64(wk[s], dt), to_f64(wv[s], dt)])
            assert np.isfinite(a).all() and rel_fro(a, b) < 1e-2, (p, s)


def test_split_attention_modes_give_identical_results():
    inst = make_instance(get_workload("P1"))
    outs = []
    for mode in (0, -1, 64):
        step, dev = make_step(inst, ctx(mode))
        step.run()
        torch.cuda.synchronize()
        outs.append((step.out.clone(), dev.peer_attn_out.clone()))
    for o, p in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(p, outs[0][1])


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
