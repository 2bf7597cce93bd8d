"""Pins of oracle.layer.layer_forward_chunks (several prefill chunks in one step) -- CPU only.

A multi-chunk step is pinned to the single-chunk step, itself pinned by pure-Python loops
and a library Llama layer: every chunk's rows, run as a step of their own with the same
pool and table, and the decode rows, run alone, must come out the same (rows of a
co-batched step are independent, ConfluxServe §4), and so must every page the step
appends to.
"""
import numpy as np
import pytest

from oracle import layer as L
from synth import MULTI_CHUNK_WORKLOADS, make_multi_instance
from tests.helpers import chunk_oracle_kwargs


def _single(inst, j):
    """Keyword arguments of layer_forward for chunk j alone (sp_degree 1, no decode)."""
    wl = inst.wl
    starts = np.cumsum([0] + [l for l, _ in wl.chunks])
    l, c = wl.chunks[j]
    return dict(hidden=wl.hidden, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                ffn_dim=wl.ffn_dim, page_size=wl.page_size, rms_eps=wl.rms_eps, rope_base=wl.rope_base,
                dtype=wl.dtype, x=inst.x[starts[j]:starts[j + 1]], weights=inst.weights,
                dec_ctx=inst.dec_ctx[:0], dec_pages=inst.dec_pages[:0], chunk_len=l, prior_len=c, sp_degree=1,
                sp_rank=0, n_prefill_local=l, local_row_offset=0, pre_pages=inst.chunk_pages[j],
                peer_qkv_in=inst.x[:0], peer_attn_in=inst.x[:0], pool=inst.pool)


@pytest.mark.parametrize("name", ["M1", "M2", "M3", "M4"])
def test_each_chunk_equals_its_own_single_chunk_step(name):
    inst = make_multi_instance(MULTI_CHUNK_WORKLOADS[name])
    wl = inst.wl
    full = L.layer_forward_chunks(**chunk_oracle_kwargs(inst))
    starts = np.cumsum([0] + [l for l, _ in wl.chunks])
    for j in range(len(wl.chunks)):
        one = L.layer_forward(**_single(inst, j))
        assert np.allclose(full["out"][starts[j]:starts[j + 1]], one["out"], atol=1e-11, rtol=0)
        assert np.allclose(full["attn"][starts[j]:starts[j + 1]], one["attn"], atol=1e-12, rtol=0)
        for p in inst.chunk_pages[j].reshape(-1):
            assert np.array_equal(full["kv"].stored_page(p).view(np.uint8), one["kv"].stored_page(p).view(np.uint8))
    if wl.n_decode:
        dec = L.layer_forward(**dict(_single(inst, 0), x=inst.x[starts[-1]:], dec_ctx=inst.dec_ctx,
                                     dec_pages=inst.dec_pages, chunk_len=0, prior_len=0, n_prefill_local=0,
                                     pre_pages=inst.chunk_pages[0][:, :0]))
        assert np.allclose(full["out"][starts[-1]:], dec["out"], atol=1e-11, rtol=0)


def test_chunk_positions_and_sampled_rows():
    inst = make_multi_instance(MULTI_CHUNK_WORKLOADS["M1"])
    wl = inst.wl
    full = L.layer_forward_chunks(**chunk_oracle_kwargs(inst))
    expect = np.concatenate([c + np.arange(l) for l, c in wl.chunks] + [inst.dec_ctx.astype(np.int64)])
    assert np.array_equal(full["positions"], expect)
    rows = [0, 96, 97, 160, 200, 343, 344, 348]
    part = L.layer_forward_chunks(**chunk_oracle_kwargs(inst, rows=rows))
    assert np.allclose(part["out"][rows], full["out"][rows], atol=1e-12, rtol=0)
