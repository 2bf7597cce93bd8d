"""GPU parity at the measured workloads' full sizes (C2, C3, C4, C5), in the launch
configurations bench.py times: the layer step serialized and with the split attention
on a 128-CU decode partition (bit-identical to each other), checked against the oracle
on sampled rows the oracle computes one by one (first, last and interior prefill rows,
rows at page and tile edges, first/middle/last decode rows, and for the SP workloads
exported peer rows).  Tolerances are the ones of the small-workload layer tests.
"""
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

_CTX = {}


def ctx(decode_cus):
    if decode_cus not in _CTX:
        _CTX[decode_cus] = X.Ctx(0, decode_cus, 0)
    return _CTX[decode_cus]


def _sample_rows(wl):
    n_pl, n_d = wl.n_prefill_local, wl.n_decode
    pre = {0, 1, 15, 16, 31, 32, n_pl // 2, n_pl - 2, n_pl - 1} if n_pl else set()
    pre = {r for r in pre if 0 <= r < n_pl}
    dec = {n_pl, n_pl + n_d // 2, n_pl + n_d - 1} if n_d else set()
    return sorted(pre | dec)


@pytest.mark.parametrize("name", ["C2", "C3", "C4", "C5"])
def test_full_size_layer_on_sampled_rows(name):
    wl = get_workload(name)
    print(f"[full] {name}: drawing inputs", flush=True)
    inst = make_instance(wl)
    dev = upload(inst)
    rows = _sample_rows(wl)
    n_peer = wl.chunk_len - wl.n_prefill_local
    peer_rows = sorted({0, n_peer // 2, n_peer - 1}) if n_peer > 0 else None
    outs = {}
    for mode in (0, 128):
        step, _ = make_step(inst, ctx(mode), dev)
        print(f"[full] {name}: layer step, decode_cus {mode}", flush=True)
        step.run()
        torch.cuda.synchronize()
        assert step.status() == 0
        outs[mode] = (step, step.out.clone(), dev.peer_attn_out.clone())
    assert torch.equal(outs[0][1], outs[128][1])
    assert torch.equal(outs[0][2], outs[128][2])
    step = outs[0][0]
    print(f"[full] {name}: oracle on rows {rows}", flush=True)
    ref = L.layer_forward(**oracle_kwargs(inst, rows=rows, peer_rows=peer_rows))
    dt = wl.dtype
    M, H, Hq, d, F = wl.n_rows, wl.hidden, wl.n_q_heads, wl.head_dim, wl.ffn_dim
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = outs[0][1].cpu().numpy().astype(np.float64)
    attn = to_f64(to_host_bits(step.ws_view("attn", (M, Hq * d), tdt)), dt)
    h1 = step.ws_view("h1", (M, H), torch.float32).cpu().numpy().astype(np.float64)
    act = to_f64(to_host_bits(step.ws_view("act", (M, F), tdt)), dt)
    r = dict(attn=rel_fro(attn[rows], ref["attn"][rows]), out=rel_fro(out[rows], ref["out"][rows]),
             out_maxabs=float(np.abs(out[rows] - ref["out"][rows]).max()))
    r["tf_maxabs"] = float(np.abs(out[rows] - (h1[rows] + act[rows] @ to_f64(inst.weights["w_down"], dt).T)).max())
    print(f"[full] {name}: {r}", flush=True)
    assert np.isfinite(out).all()
    assert r["attn"] < 5e-3, r
    assert r["tf_maxabs"] < 2e-2, r
    assert r["out"] < 5e-3, r
    if peer_rows:
        got = to_f64(to_host_bits(outs[0][2]), dt)[peer_rows]
        assert rel_fro(got, ref["peer_attn_out"][peer_rows]) < 5e-3
