"""Marshalling of a layer step into the C structs of include/xp.h.

``LayerStep`` keeps the descriptor structs, the workspace and the output
buffer of one batch and enqueues ``xp_layer_forward`` on a stream.  All
buffers are caller-provided torch device tensors; nothing is computed here.
"""
from __future__ import annotations

from . import _lib as X

__all__ = ["layer_shape", "layer_weights", "batch_desc", "LayerStep", "ChunkedStep", "StackStep"]


def layer_shape(*, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, page_size=16, rms_eps=1e-5,
                rope_base=10000.0, dtype="bf16") -> X.LayerShape:
    return X.LayerShape(hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, page_size, rms_eps, rope_base,
                        X.XP_BF16 if dtype == "bf16" else X.XP_F32)


def layer_weights(w: dict) -> X.LayerWeights:
    return X.LayerWeights(*[X._ptr(w[k]) for k in ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_ffn")])


def batch_desc(*, x, n_prefill_local, n_decode, dec_ctx, dec_pages, chunk_len, prior_len, sp_degree=1,
               sp_rank=0, local_row_offset=0, pre_pages=None, peer_qkv_in=None, peer_qkv_out=None,
               peer_attn_in=None, peer_attn_out=None, dec_ctx_host=None, dec_pages_host=None,
               pre_pages_host=None) -> X.BatchDesc:
    """The descriptor struct; the optional ``*_host`` numpy copies of the tables make the
    step validate every page id on the host before it launches anything."""
    import numpy as np
    dmb = int(dec_pages.shape[-1]) if (dec_pages is not None and dec_pages.dim() == 3) else 0
    pmb = int(pre_pages.shape[-1]) if (pre_pages is not None and pre_pages.dim() == 2) else 0
    P = X._ptr
    host = [None if a is None else np.ascontiguousarray(a, dtype=np.int32)
            for a in (dec_ctx_host, dec_pages_host, pre_pages_host)]
    d = X.BatchDesc(P(x), n_prefill_local, n_decode, P(dec_ctx), P(dec_pages), dmb, chunk_len, prior_len,
                    sp_degree, sp_rank, local_row_offset, P(pre_pages), pmb, P(peer_qkv_in), P(peer_qkv_out),
                    P(peer_attn_in), P(peer_attn_out), *[P(a) for a in host])
    d._host = host            # the host copies live as long as the struct
    return d


class LayerStep:
    """One batch's descriptor + workspace + output, ready to enqueue."""

    def __init__(self, ctx: X.Ctx, shape: X.LayerShape, desc: X.BatchDesc, weights: X.LayerWeights,
                 pool, n_pages: int, keep=()):
        import torch
        self.ctx, self.shape, self.desc, self.weights = ctx, shape, desc, weights
        self.kv = X.KvPages(X._ptr(pool), n_pages)
        self.layout = X.xp_layer_workspace_layout(ctx, shape, desc)
        dev = torch.device("cuda", ctx.device)
        self.workspace = torch.empty(self.layout.total, dtype=torch.uint8, device=dev)
        M = desc.n_prefill_local + desc.n_decode
        self.out = torch.empty((M, shape.hidden), dtype=torch.float32, device=dev)
        self._keep = (pool,) + tuple(keep)   # keeps the buffers the structs point to alive

    def run(self, stream=None):
        X.xp_layer_forward(self.ctx, self.shape, self.desc, self.weights, self.kv, self.out, self.workspace,
                           self.layout.total, stream)
        return self.out

    def status(self, stream=None) -> int:
        return X.xp_layer_read_status(self.workspace, self.layout, stream)

    def ws_view(self, name: str, shape, dtype):
        """A typed view of one intermediate in the workspace (after the stream completed)."""
        import torch
        off = getattr(self.layout, name)
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype).view(*shape)


class ChunkedStep:
    """A multi-chunk batch (xp_layer_forward_chunks): rows [chunk 0 || ... || decode],
    ``chunks`` = [(chunk_len, prior_len, table tensor [Hkv, blocks])], sp_degree 1."""

    def __init__(self, ctx: X.Ctx, shape: X.LayerShape, desc: X.BatchDesc, chunks, weights: X.LayerWeights,
                 pool, n_pages: int, keep=()):
        import torch
        self.ctx, self.shape, self.desc, self.weights = ctx, shape, desc, weights
        self.chunks = X.chunk_array(chunks)
        self.kv = X.KvPages(X._ptr(pool), n_pages)
        self.layout = X.xp_layer_workspace_layout_chunks(ctx, shape, desc, self.chunks)
        dev = torch.device("cuda", ctx.device)
        self.workspace = torch.empty(self.layout.total, dtype=torch.uint8, device=dev)
        M = sum(int(l) for l, _, _ in chunks) + desc.n_decode
        self.out = torch.empty((M, shape.hidden), dtype=torch.float32, device=dev)
        self._keep = (pool,) + tuple(t for _, _, t in chunks) + tuple(keep)

    def run(self, stream=None):
        X.xp_layer_forward_chunks(self.ctx, self.shape, self.desc, self.chunks, self.weights, self.kv, self.out,
                                  self.workspace, self.layout.total, stream)
        return self.out

    def status(self, stream=None) -> int:
        return X.xp_layer_read_status(self.workspace, self.layout, stream)


class StackStep:
    """One batch through a stack of layers (xp_stack_forward): a weight set and a KV pool
    per layer (``pools`` = [(pool tensor, n_pages)]), one layer's workspace and the fp32
    output that carries the residual stream between layers.  ``capture`` records the
    shared-linear segments in HIP graphs (xp_stack_graph_create) for ``Graph.launch``."""

    def __init__(self, ctx: X.Ctx, shape: X.LayerShape, desc: X.BatchDesc, weights, pools, keep=()):
        import torch
        self.ctx, self.shape, self.desc = ctx, shape, desc
        self.weights = X.weights_array(weights)
        self.pools = X.pools_array(pools)
        self.layout = X.xp_layer_workspace_layout(ctx, shape, desc)
        dev = torch.device("cuda", ctx.device)
        self.workspace = torch.empty(self.layout.total, dtype=torch.uint8, device=dev)
        M = desc.n_prefill_local + desc.n_decode
        self.out = torch.empty((M, shape.hidden), dtype=torch.float32, device=dev)
        self._keep = tuple(p for p, _ in pools) + tuple(keep)

    def run(self, stream=None):
        X.xp_stack_forward(self.ctx, self.shape, self.desc, self.weights, self.pools, self.out, self.workspace,
                           self.layout.total, stream)
        return self.out

    def capture(self, stream) -> X.Graph:
        return X.xp_stack_graph_create(self.ctx, self.shape, self.desc, self.weights, self.pools, self.out,
                                       self.workspace, self.layout.total, stream)

    def status(self, stream=None) -> int:
        return X.xp_layer_read_status(self.workspace, self.layout, stream)
