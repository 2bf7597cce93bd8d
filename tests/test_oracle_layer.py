"""Pins of oracle.layer.layer_forward -- CPU only.

* a pure-Python loop formulation (oracle.brute) on tiny paged inputs;
* the transformers library's Llama decoder layer (float64), run request by request with
  its own KV cache, against the co-batched, paged oracle step;
* invariants: co-batched rows = separately computed rows; SP-rank outputs reassembled
  = single-rank outputs; zero projections pass the residual through.
"""
import numpy as np
import pytest
import torch

from oracle import brute
from oracle import layer as L
from synth import Workload, make_instance
from tests.helpers import ArrayPool, oracle_kwargs, k_slots

TINY = Workload("tiny", 901, "f32", 16, 4, 2, 4, 24, n_decode=3, ctx=("list", [0, 6, 9]),
                chunk_len=5, prior_len=7, page_size=4, spare_pages=2)


def test_layer_matches_pure_python_loops():
    inst = make_instance(TINY)
    ref = L.layer_forward(**oracle_kwargs(inst))
    kw = oracle_kwargs(inst)
    for k in ("sp_degree", "sp_rank", "n_prefill_local", "local_row_offset", "peer_qkv_in", "peer_attn_in"):
        kw.pop(k)
    outs = brute.brute_layer(**kw)
    assert np.allclose(ref["out"], np.array(outs), atol=1e-12, rtol=0)
    assert np.isfinite(ref["out"]).all()


def test_appends_land_in_the_right_slots_and_nothing_else_changes():
    inst = make_instance(TINY)
    res = L.layer_forward(**oracle_kwargs(inst))
    kv, S, d = res["kv"], TINY.page_size, TINY.head_dim
    touched = set()
    for i, c in enumerate(inst.dec_ctx):
        for g in range(TINY.n_kv_heads):
            p = int(inst.dec_pages[i, g, c // S]); touched.add(p)
            page = kv.stored_page(p)
            assert np.array_equal(k_slots(page[0], S, d, TINY.dtype)[c % S],
                                  res["k"][TINY.n_prefill_local + i, g].astype(np.float32))
    for t in range(TINY.chunk_len):
        pos = TINY.prior_len + t
        for g in range(TINY.n_kv_heads):
            p = int(inst.pre_pages[g, pos // S]); touched.add(p)
            page = kv.stored_page(p)
            assert np.array_equal(page[1].reshape(d, S)[:, pos % S], res["v"][t, g].astype(np.float32))
    for p in range(inst.pool.n_pages):
        if p not in touched:
            assert np.array_equal(kv.stored_page(p), inst.pool.array[p], equal_nan=True)


def _hf_layer(H, Hq, Hkv, d, F, W):
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaDecoderLayer, LlamaRotaryEmbedding
    cfg = LlamaConfig(hidden_size=H, intermediate_size=F, num_attention_heads=Hq,
                      num_key_value_heads=Hkv, head_dim=d, rms_norm_eps=1e-5, rope_theta=10000.0,
                      attention_bias=False, mlp_bias=False)
    cfg._attn_implementation = "sdpa"
    layer = LlamaDecoderLayer(cfg, 0).double().eval()
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    with torch.no_grad():
        layer.self_attn.q_proj.weight.copy_(t(W["w_qkv"][:Hq * d]))
        layer.self_attn.k_proj.weight.copy_(t(W["w_qkv"][Hq * d:(Hq + Hkv) * d]))
        layer.self_attn.v_proj.weight.copy_(t(W["w_qkv"][(Hq + Hkv) * d:]))
        layer.self_attn.o_proj.weight.copy_(t(W["w_o"]))
        layer.mlp.gate_proj.weight.copy_(t(W["w_gate"]))
        layer.mlp.up_proj.weight.copy_(t(W["w_up"]))
        layer.mlp.down_proj.weight.copy_(t(W["w_down"]))
        layer.input_layernorm.weight.copy_(t(W["g_attn"]))
        layer.post_attention_layernorm.weight.copy_(t(W["g_ffn"]))
    return cfg, layer, LlamaRotaryEmbedding(cfg)


def _hf_run(cfg, layer, rot, X, n0):
    """Run tokens X[:n0] to fill a cache, then X[n0:] against it; return (outputs of the
    second run, cached K, V of the first n0 positions)."""
    from transformers import DynamicCache
    cache = DynamicCache(config=cfg)
    X = torch.from_numpy(X)[None]
    Kc = Vc = None
    with torch.no_grad():
        if n0 > 0:
            pos = torch.arange(n0)[None]
            layer(X[:, :n0], attention_mask=None, position_ids=pos, past_key_values=cache,
                  use_cache=True, position_embeddings=rot(X, pos))
            Kc = cache.layers[0].keys[0].clone().numpy()
            Vc = cache.layers[0].values[0].clone().numpy()
        n = X.shape[1]
        pos = torch.arange(n0, n)[None]
        vis = torch.arange(n)[None, :] <= torch.arange(n0, n)[:, None]
        mask = torch.where(vis, 0.0, float("-inf")).double()[None, None]
        y = layer(X[:, n0:], attention_mask=mask, position_ids=pos, past_key_values=cache,
                  use_cache=True, position_embeddings=rot(X, pos))
    return y[0].numpy(), Kc, Vc


def test_layer_matches_library_llama_layer_run_per_request():
    r = np.random.default_rng(21)
    H, Hq, Hkv, d, F, S = 64, 4, 2, 16, 128, 16
    f32 = lambda *s, sc=1.0: (r.standard_normal(s) * sc).astype(np.float32)
    W = dict(w_qkv=f32((Hq + 2 * Hkv) * d, H, sc=0.1), w_o=f32(H, Hq * d, sc=0.1),
             w_gate=f32(F, H, sc=0.1), w_up=f32(F, H, sc=0.1), w_down=f32(H, F, sc=0.1),
             g_attn=(1 + f32(H, sc=0.1)), g_ffn=(1 + f32(H, sc=0.1)))
    cfg, layer, rot = _hf_layer(H, Hq, Hkv, d, F, W)
    c, l = 20, 13
    dec_ctx = np.array([0, 37, 16])
    XA = f32(c + l, H)
    XD = [f32(cc + 1, H) for cc in dec_ctx]
    yA, KA, VA = _hf_run(cfg, layer, rot, XA.astype(np.float64), c)
    yD = [_hf_run(cfg, layer, rot, X.astype(np.float64), int(cc)) for X, cc in zip(XD, dec_ctx)]

    # paged pool holding the library's cached (rotated) K and V, ABI layout, NaN elsewhere
    nb_pre = -(-(c + l) // S)
    nb_dec = [-(-(cc + 1) // S) for cc in dec_ctx]
    n_pages = Hkv * (nb_pre + sum(nb_dec)) + 2
    perm = r.permutation(n_pages)
    pool = np.full((n_pages, 2, S * d), np.nan, dtype=np.float32)
    pre_pages = np.full((Hkv, nb_pre), -1, dtype=np.int32)
    dec_pages = np.full((len(dec_ctx), Hkv, max(nb_dec)), -1, dtype=np.int32)
    it = iter(perm)

    def put(table_row, nb, K, V, n):
        for b in range(nb):
            table_row[b] = next(it)
        for pos in range(n):
            p, s = table_row[pos // S], pos % S
            pool[p, 0, ((np.arange(d) // 4) * S + s) * 4 + np.arange(d) % 4] = K[pos]   # chunk-major K, fp32
            pool[p, 1, np.arange(d) * S + s] = V[pos]

    for g in range(Hkv):
        put(pre_pages[g], nb_pre, KA[g] if c else None, VA[g] if c else None, c)
    for i, cc in enumerate(dec_ctx):
        _, Kc, Vc = yD[i]
        for g in range(Hkv):
            put(dec_pages[i, g], nb_dec[i], Kc[g] if cc else None, Vc[g] if cc else None, int(cc))

    x = np.concatenate([XA[c:]] + [X[-1:] for X in XD])
    res = L.layer_forward(hidden=H, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, ffn_dim=F, page_size=S,
                          rms_eps=1e-5, rope_base=10000.0, dtype="f32", x=x, weights=W, dec_ctx=dec_ctx,
                          dec_pages=dec_pages, chunk_len=l, prior_len=c, sp_degree=1, sp_rank=0,
                          n_prefill_local=l, local_row_offset=0, pre_pages=pre_pages,
                          peer_qkv_in=np.zeros((0, (Hq + 2 * Hkv) * d), np.float32),
                          peer_attn_in=np.zeros((l, 0), np.float32), pool=ArrayPool(pool))
    ref = np.concatenate([yA] + [y[0] for y in yD])
    err = np.abs(res["out"] - ref).max()
    assert err < 1e-4, err


def _variant(inst, keep_prefill: bool, keep_decode: bool):
    kw = oracle_kwargs(inst)
    wl = inst.wl
    n_pl = wl.n_prefill_local
    rows = []
    if keep_prefill:
        rows += list(range(n_pl))
    else:
        kw.update(chunk_len=0, n_prefill_local=0, local_row_offset=0,
                  peer_qkv_in=inst.peer_qkv_in[:0], peer_attn_in=inst.peer_attn_in[:0])
    if keep_decode:
        rows += list(range(n_pl, n_pl + wl.n_decode))
    else:
        kw.update(dec_ctx=inst.dec_ctx[:0], dec_pages=inst.dec_pages[:0])
    kw["x"] = inst.x[rows]
    return kw


def test_cobatched_rows_equal_separately_computed_rows():
    from synth import get_workload
    inst = make_instance(get_workload("P1"))
    n_pl = inst.wl.n_prefill_local
    full = L.layer_forward(**oracle_kwargs(inst))
    pre = L.layer_forward(**_variant(inst, True, False))
    dec = L.layer_forward(**_variant(inst, False, True))
    assert np.allclose(full["out"][:n_pl], pre["out"], atol=1e-12, rtol=0)
    assert np.allclose(full["out"][n_pl:], dec["out"], atol=1e-12, rtol=0)
    assert np.allclose(full["peer_attn_out"], pre["peer_attn_out"], atol=1e-12, rtol=0)


def test_sp_ranks_reassemble_single_rank_result():
    from dataclasses import replace
    wl1 = Workload("sp-ref", 902, "f32", 64, 4, 2, 16, 96, n_decode=2, ctx=("list", [3, 30]),
                   chunk_len=12, prior_len=9)
    inst = make_instance(wl1)
    ref = L.layer_forward(**oracle_kwargs(inst))
    P, l, Hq, Hkv, d = 2, 12, 4, 2, 16
    hq, hkv = Hq // P, Hkv // P
    n_pl = l // P
    for r in range(P):
        own_q = list(range(r * hq, (r + 1) * hq)); own_kv = list(range(r * hkv, (r + 1) * hkv))
        oth_q = [h for h in range(Hq) if h not in own_q]
        local = list(range(r * n_pl, (r + 1) * n_pl))
        peer = [t for t in range(l) if t not in local]
        f32 = lambda a: np.asarray(a, dtype=np.float32)
        peer_qkv_in = f32(np.concatenate([ref["q"][peer][:, own_q].reshape(len(peer), -1),
                                          ref["k"][peer][:, own_kv].reshape(len(peer), -1),
                                          ref["v"][peer][:, own_kv].reshape(len(peer), -1)], axis=1))
        attn = ref["attn"][local].reshape(n_pl, Hq, d)
        peer_attn_in = f32(attn[:, oth_q].reshape(n_pl, -1))
        rows = local + list(range(l, l + wl1.n_decode))
        kw = oracle_kwargs(inst, sp_degree=P, sp_rank=r, n_prefill_local=n_pl, local_row_offset=r * n_pl,
                           pre_pages=inst.pre_pages[own_kv], peer_qkv_in=peer_qkv_in,
                           peer_attn_in=peer_attn_in, x=inst.x[rows])
        res = L.layer_forward(**kw)
        assert np.allclose(res["out"], ref["out"][rows], atol=2e-6, rtol=0)
        pao = ref["attn"][peer].reshape(len(peer), Hq, d)[:, own_q].reshape(len(peer), -1)
        assert np.allclose(res["peer_attn_out"], pao, atol=2e-6, rtol=0)
        exp_out = np.concatenate([ref["q"][local][:, oth_q].reshape(n_pl, -1),
                                  ref["k"][local][:, [g for g in range(Hkv) if g not in own_kv]].reshape(n_pl, -1),
                                  ref["v"][local][:, [g for g in range(Hkv) if g not in own_kv]].reshape(n_pl, -1)], axis=1)
        assert np.allclose(res["peer_qkv_out"], exp_out, atol=1e-12, rtol=0)


def test_zero_projections_pass_the_residual_through():
    inst = make_instance(TINY)
    kw = oracle_kwargs(inst)
    w = dict(inst.weights)
    w["w_o"] = np.zeros_like(w["w_o"]); w["w_down"] = np.zeros_like(w["w_down"])
    res = L.layer_forward(**dict(kw, weights=w))
    assert np.array_equal(res["out"], inst.x.astype(np.float64))
    w2 = dict(inst.weights); w2["w_down"] = np.zeros_like(w2["w_down"])
    res2 = L.layer_forward(**dict(kw, weights=w2))
    assert np.array_equal(res2["out"], res2["h1"])


def test_row_sampling_matches_full_computation():
    from synth import get_workload
    inst = make_instance(get_workload("P1"))
    full = L.layer_forward(**oracle_kwargs(inst))
    rows = [0, 3, inst.wl.n_rows - 1, inst.wl.n_prefill_local]
    part = L.layer_forward(**oracle_kwargs(inst, rows=rows, peer_rows=[0, 5]))
    # equal up to summation order (BLAS blocks differently for fewer rows)
    assert np.allclose(part["out"][rows], full["out"][rows], atol=1e-12, rtol=0)
    assert np.allclose(part["peer_attn_out"][[0, 5]], full["peer_attn_out"][[0, 5]], atol=1e-12, rtol=0)
