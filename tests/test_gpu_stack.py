"""GPU parity of layer stacks (xp_stack_forward) and of their piecewise graph replay
(xp_stack_graph_create / xp_graph_launch) against the oracle.

A stack runs one batch through several layers, each with its own weights and KV pool;
the residual stream stays fp32 between layers (ConfluxServe §4 Fig. 7 layer after
layer; §6.1 Fig. 10: the shared-linear segments captured in graphs, the attention
region eager between them).  Checked: the last layer's output and every layer's pool
against the oracle; graph launches bit-identical to the eager stack, launch after
launch with other work in between, in serialized and CU-partitioned contexts.
"""
import json
import os

import numpy as np
import pytest
import torch

import mixed_prefill_decode_amd as X
from oracle import layer as L
from oracle.numerics import to_f64
from synth import get_workload, make_stack_instance
from synth.device import make_stack_step, to_host_bits
from tests.helpers import rel_fro, stack_oracle_kwargs, shared_ctx, k_slots

pytestmark = pytest.mark.gpu

ctx = shared_ctx


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _same_bits(a, b):
    # pools hold NaN in slots past each page's cached tokens: compare bit patterns
    it = torch.int16 if a.element_size() == 2 else torch.int32
    return torch.equal(a.view(it), b.view(it))


def _check_pool(sinst, l, got_pool, kv):
    wl, dt = sinst.wl, sinst.wl.dtype
    S, d = wl.page_size, wl.head_dim
    base = sinst.layers[l]["pool"]
    got = to_host_bits(got_pool)
    for p in range(base.n_pages):
        if p not in kv.overlay:
            assert got[p].tobytes() == base[[p]][0].tobytes(), (l, p)
            continue
        want = kv.stored_page(p)
        gk, gv = k_slots(got[p, 0], S, d, dt), got[p, 1].reshape(d, S).T
        wk, wv = k_slots(want[0], S, d, dt), want[1].reshape(d, S).T
        same = np.all(_bits(gk) == _bits(wk), axis=1) & np.all(_bits(gv) == _bits(wv), axis=1)
        for s in np.nonzero(~same)[0]:
            a = np.concatenate([to_f64(gk[s], dt), to_f64(gv[s], dt)])
            b = np.concatenate([to_f64(wk[s], dt), to_f64(wv[s], dt)])
            assert np.isfinite(a).all() and rel_fro(a, b) < 1e-2, (l, p, s)


# (workload, layers): bf16 with decodes at page edges and a chunk, fp32, decode only,
# prefill only with two waves per head
@pytest.mark.parametrize("name,n_layers", [("P2", 3), ("C1", 3), ("E1", 2), ("P5", 2)])
def test_stack_matches_oracle(name, n_layers):
    sinst = make_stack_instance(get_workload(name), n_layers)
    print(f"[stack] {name}: {n_layers} layers", flush=True)
    step = make_stack_step(sinst, ctx(0))
    step.run()
    torch.cuda.synchronize()
    assert step.status() == 0
    ref = L.stack_forward(**stack_oracle_kwargs(sinst))
    out = step.out.cpu().numpy().astype(np.float64)
    assert np.isfinite(out).all()
    err = rel_fro(out, ref["out"])
    print(f"[stack] {name}: rel err {err:.2e}", flush=True)
    path = os.environ.get("XP_METRICS_OUT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": f"stack {name} x{n_layers}", "out": err}) + "\n")
    # the single-layer bar of the dtype, not one that grows with depth: the residual
    # stream between layers is fp32 on both sides, so a layer adds its own rounding only
    assert err < (5e-3 if sinst.wl.dtype == "bf16" else 1e-5), err
    for l in range(n_layers):
        _check_pool(sinst, l, step.pool_tensors[l], ref["layers"][l]["kv"])


def test_graph_launches_equal_the_eager_stack():
    sinst = make_stack_instance(get_workload("P2"), 3)
    step = make_stack_step(sinst, ctx(0))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = step.run(s).clone()
        pools = [p.clone() for p in step.pool_tensors]
    s.synchronize()
    graph = step.capture(s)
    for i in range(3):
        step.out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.launch(s)
        s.synchronize()
        assert torch.equal(step.out, eager), i
        for a, b in zip(step.pool_tensors, pools):
            assert _same_bits(a, b), i
        # other work between launches: an eager stack on the same buffers
        step.run(s)
        s.synchronize()
        assert torch.equal(step.out, eager), i
    graph.close()


def test_graph_with_a_cu_partition_agrees_with_serialized():
    # partitioned (64 decode CUs) and co-resident (-1) attention between the graphs
    sinst = make_stack_instance(get_workload("P2"), 2)
    outs = []
    for mode in (0, 64, -1):
        step = make_stack_step(sinst, ctx(mode))
        s = torch.cuda.Stream()
        graph = step.capture(s)
        graph.launch(s)
        graph.launch(s)
        s.synchronize()
        outs.append(step.out.clone())
        graph.close()
    # decode rows bit-identical; chunk rows within merge-order rounding
    n_pl = sinst.wl.n_prefill_local
    for o in outs[1:]:
        assert torch.equal(outs[0][n_pl:], o[n_pl:])
        assert rel_fro(o.cpu().numpy(), outs[0].cpu().numpy()) < 1e-3


def test_stack_arguments_are_checked_before_launch():
    sinst = make_stack_instance(get_workload("P2"), 1)
    step = make_stack_step(sinst, ctx(0))
    with pytest.raises(X.XpError) as e:                 # the null stream cannot be captured
        X.xp_stack_graph_create(step.ctx, step.shape, step.desc, step.weights, step.pools, step.out,
                                step.workspace, step.layout.total, 0)
    assert e.value.status == -1
    with pytest.raises(X.XpError) as e:                 # workspace too small
        X.xp_stack_forward(step.ctx, step.shape, step.desc, step.weights, step.pools, step.out, step.workspace,
                           step.layout.total - 1)
    assert e.value.status == -6
    sp2 = X.batch_desc(x=step.x, n_prefill_local=0, n_decode=0, dec_ctx=None, dec_pages=None, chunk_len=0,
                       prior_len=0, sp_degree=2)
    with pytest.raises(X.XpError) as e:
        X.xp_stack_forward(step.ctx, step.shape, sp2, step.weights, step.pools, step.out, step.workspace,
                           step.layout.total)
    assert e.value.status == -5
    with pytest.raises(ValueError):
        X.xp_stack_forward(step.ctx, step.shape, step.desc, step.weights, X.pools_array([]), step.out,
                           step.workspace, step.layout.total)


def test_stack_status_keeps_a_bad_page_of_any_layer():
    """The device status word is cleared once per stack call: a page id that only layer
    0's pool lacks is still reported after the last layer."""
    sinst = make_stack_instance(get_workload("P2"), 2)
    step = make_stack_step(sinst, ctx(0))
    base = sinst.base
    used = np.concatenate([base.dec_pages.reshape(-1), base.pre_pages.reshape(-1)])
    top = int(used[used >= 0].max())
    pools = [(step.pool_tensors[0], top)] + [(p, l["pool"].n_pages) for p, l in
                                             zip(step.pool_tensors[1:], sinst.layers[1:])]
    step.pools = X.pools_array(pools)              # layer 0's pool ends below the largest id
    step.run()
    torch.cuda.synchronize()
    assert step.status() & X.XP_DEV_BAD_PAGE
    ok = make_stack_step(sinst, ctx(0))
    ok.run()
    torch.cuda.synchronize()
    assert ok.status() == 0
