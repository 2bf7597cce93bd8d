"""GPU parity of the multi-chunk layer step (xp_layer_forward_chunks) against the oracle.

Several requests' prefill chunks in one step (ConfluxServe §6.2 Eq. 6, §6.4): every
chunk attends over its own request's keys through its own table.  Checked at the
tolerances of the single-chunk step, plus bit-identity with separately run
single-chunk steps (the kernels are batch invariant) and across split-attention modes.
"""
import numpy as np
import pytest
import torch

import mixed_prefill_decode_amd as X
from oracle import layer as L
from oracle.numerics import to_f64
from synth import MULTI_CHUNK_WORKLOADS, make_multi_instance
from synth.device import make_chunked_step, to_host_bits
from tests.helpers import chunk_oracle_kwargs, down_stage_errors, rel_fro, shared_ctx, k_slots

pytestmark = pytest.mark.gpu

ctx = shared_ctx


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _ws(step, name, shape, dtype):
    off = getattr(step.layout, name)
    n = int(np.prod(shape))
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return step.workspace[off:off + nbytes].view(dtype).view(*shape)


def _check(inst, step, ref, rows):
    wl, dt = inst.wl, inst.wl.dtype
    M, H, Hq, d, F = wl.n_rows, wl.hidden, wl.n_q_heads, wl.head_dim, wl.ffn_dim
    out = step.out.cpu().numpy().astype(np.float64)
    attn = to_f64(to_host_bits(_ws(step, "attn", (M, Hq * d), _tdt(dt))), dt)
    h1 = _ws(step, "h1", (M, H), torch.float32).cpu().numpy().astype(np.float64)
    act = to_f64(to_host_bits(_ws(step, "act", (M, F), _tdt(dt))), dt)
    assert step.status() == 0
    assert np.isfinite(out).all()
    r = dict(attn=rel_fro(attn[rows], ref["attn"][rows]), out=rel_fro(out[rows], ref["out"][rows]),
             out_maxabs=float(np.abs(out[rows] - ref["out"][rows]).max()))
    r["tf_maxabs"], r["tf_f32_maxabs"], tf_bar = down_stage_errors(out[rows], h1[rows], act[rows],
                                                                   to_f64(inst.weights["w_down"], dt))
    assert r["attn"] < 5e-3, r
    assert r["tf_maxabs"] <= tf_bar, r
    if dt == "f32":
        assert r["out_maxabs"] < 2e-2, r
    else:
        assert r["out"] < 5e-3, r
    return r


@pytest.mark.parametrize("name", ["M1", "M2", "M3", "M4"])
def test_chunked_layer_matches_oracle(name):
    inst = make_multi_instance(MULTI_CHUNK_WORKLOADS[name])
    wl, dt = inst.wl, inst.wl.dtype
    print(f"[chunks] {name}: chunks {wl.chunks}, decodes {wl.n_decode}", flush=True)
    step = make_chunked_step(inst, ctx(0))
    step.run()
    torch.cuda.synchronize()
    ref = L.layer_forward_chunks(**chunk_oracle_kwargs(inst))
    _check(inst, step, ref, np.arange(wl.n_rows))
    # the pool: appended slots within rounding of the oracle's, every other slot untouched
    pool = to_host_bits(step.pool)
    kv = ref["kv"]
    S, dd = wl.page_size, wl.head_dim
    for p in range(inst.pool.n_pages):
        if p not in kv.overlay:
            assert pool[p].tobytes() == inst.pool[[p]][0].tobytes(), p
            continue
        want = kv.stored_page(p)
        gk, gv = k_slots(pool[p, 0], S, dd, dt), pool[p, 1].reshape(dd, S).T
        wk, wv = k_slots(want[0], S, dd, dt), want[1].reshape(dd, S).T
        same = np.all(_bits(gk) == _bits(wk), axis=1) & np.all(_bits(gv) == _bits(wv), axis=1)
        for s in np.nonzero(~same)[0]:
            a = np.concatenate([to_f64(gk[s], dt), to_f64(gv[s], dt)])
            b = np.concatenate([to_f64(wk[s], dt), to_f64(wv[s], dt)])
            assert np.isfinite(a).all() and rel_fro(a, b) < 1e-2, (p, s)


def test_chunked_step_equals_single_chunk_steps():
    """Each chunk's rows, and the decode rows, equal their own steps bit for bit; and the
    single-chunk steps (RoPE and appends in the QKV GEMM's epilogue) rewrite every page of
    the pool with the bits the multi-chunk step (the stand-alone RoPE/append kernel) wrote."""
    inst = make_multi_instance(MULTI_CHUNK_WORKLOADS["M1"])
    wl = inst.wl
    step = make_chunked_step(inst, ctx(0))
    full = step.run().clone()
    torch.cuda.synchronize()
    pool0 = step.pool.clone().view(torch.uint8)          # bits (unused slots hold NaN)
    starts = np.cumsum([0] + [l for l, _ in wl.chunks])
    x = step.x
    for j, (l, c) in enumerate(wl.chunks):
        xj = x[starts[j]:starts[j + 1]].contiguous()
        t = step.tables[j]
        desc = X.batch_desc(x=xj, n_prefill_local=l, n_decode=0, dec_ctx=None, dec_pages=None, chunk_len=l,
                            prior_len=c, pre_pages=t)
        one = X.LayerStep(ctx(0), step.shape, desc, step.weights, step.pool, inst.pool.n_pages, keep=(xj, t))
        got = one.run().clone()
        torch.cuda.synchronize()
        assert torch.equal(full[starts[j]:starts[j + 1]], got), j
    xd = x[starts[-1]:].contiguous()
    dec_ctx, dec_pages = step.dec_ctx, step.dec_pages
    desc = X.batch_desc(x=xd, n_prefill_local=0, n_decode=wl.n_decode, dec_ctx=dec_ctx, dec_pages=dec_pages,
                        chunk_len=0, prior_len=0)
    dec = X.LayerStep(ctx(0), step.shape, desc, step.weights, step.pool, inst.pool.n_pages, keep=(xd,))
    got = dec.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(full[starts[-1]:], got)
    assert torch.equal(step.pool.view(torch.uint8), pool0)


def test_chunked_split_attention_modes_agree():
    inst = make_multi_instance(MULTI_CHUNK_WORKLOADS["M1"])
    outs = []
    for mode in (0, -1, 64):
        step = make_chunked_step(inst, ctx(mode))
        outs.append(step.run().clone())
        torch.cuda.synchronize()
    # decode rows bit-identical; chunk rows within merge-order rounding (a partition's
    # prefill plans its key splits for the CUs it has); the co-resident step plans for
    # every CU, like the serialized one, and its kernels sum in the same order
    n_pre = inst.wl.n_prefill_rows
    for o in outs[1:]:
        assert torch.equal(o[n_pre:], outs[0][n_pre:])
        assert rel_fro(o.cpu().numpy(), outs[0].cpu().numpy()) < 1e-3
    assert torch.equal(outs[1], outs[0])


def test_chunked_8b_step_on_sampled_rows():
    inst = make_multi_instance(MULTI_CHUNK_WORKLOADS["C2x4"])
    wl = inst.wl
    print(f"[chunks] C2x4: {wl.n_rows} rows", flush=True)
    step = make_chunked_step(inst, ctx(0))
    step.run()
    torch.cuda.synchronize()
    starts = np.cumsum([0] + [l for l, _ in wl.chunks])
    rows = sorted({0, 1, 255, 256, 300, 511, 512, 767, 768, 1000, 1023, 1024, 1031, 1039})
    ref = L.layer_forward_chunks(**chunk_oracle_kwargs(inst, rows=rows))
    _check(inst, step, ref, np.asarray(rows))
    assert starts[-1] == 1024


def test_chunk_list_is_validated_before_launch():
    inst = make_multi_instance(MULTI_CHUNK_WORKLOADS["M2"])
    step = make_chunked_step(inst, ctx(0))
    bad = X.chunk_array([(5, 200, step.tables[0])])     # table too short for 205 positions
    with pytest.raises(X.XpError) as e:
        X.xp_layer_workspace_layout_chunks(ctx(0), step.shape, step.desc, bad)
    assert e.value.status == -3
    sp2 = X.batch_desc(x=step.x, n_prefill_local=0, n_decode=0, dec_ctx=None, dec_pages=None,
                       chunk_len=0, prior_len=0, sp_degree=2)
    with pytest.raises(X.XpError) as e:
        X.xp_layer_workspace_layout_chunks(ctx(0), step.shape, sp2, step.chunks)
    assert e.value.status == -5
