"""Device copies of a drawn instance, in the C-ABI storage formats (torch tensors).

Only copies: bf16 bit patterns are reinterpreted as torch.bfloat16, pools that
are a seeded bank of pages are expanded on the device by indexing.  Nothing
here computes any part of the layer.
"""
from __future__ import annotations

import numpy as np
import torch

from .workloads import Instance

__all__ = ["to_device", "upload_pool", "DeviceInstance", "upload", "make_step", "make_chunked_step"]


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)
    if dtype == "i32":
        return torch.from_numpy(a.astype(np.int32, copy=False)).to(device)
    raise ValueError(dtype)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy storage array (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload_pool(inst: Instance, device="cuda") -> torch.Tensor:
    pool = inst.pool
    if pool.array is not None:
        return to_device(pool.array, inst.wl.dtype, device)
    tdt = torch.bfloat16 if inst.wl.dtype == "bf16" else torch.float32
    out = torch.empty((pool.n_pages,) + tuple(pool.row_shape), dtype=tdt, device=device)
    bank = to_device(pool.bank, inst.wl.dtype, device)
    idx = torch.from_numpy(pool.bank_idx).to(device)
    step = 1 << 16
    for p0 in range(0, pool.n_pages, step):
        out[p0:p0 + step] = bank[idx[p0:p0 + step]]
    ids = pool.poisoned_pages()
    for p0 in range(0, len(ids), step):
        sel = ids[p0:p0 + step]
        out[torch.from_numpy(sel).to(device)] = to_device(pool[sel], inst.wl.dtype, device)
    return out


class DeviceInstance:
    """Every input of an instance on the device, plus the output stand-in buffers."""

    def __init__(self, inst: Instance, device="cuda"):
        wl, dt = inst.wl, inst.wl.dtype
        self.inst = inst
        self.x = to_device(inst.x, dt, device)
        self.weights = {k: to_device(v, dt, device) for k, v in inst.weights.items()}
        self.dec_ctx = to_device(inst.dec_ctx, "i32", device)
        self.dec_pages = to_device(inst.dec_pages, "i32", device)
        self.pre_pages = to_device(inst.pre_pages, "i32", device)
        self.pool = upload_pool(inst, device)
        self.peer_qkv_in = to_device(inst.peer_qkv_in, dt, device)
        self.peer_attn_in = to_device(inst.peer_attn_in, dt, device)
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
        n_pl, n_peer = wl.n_prefill_local, wl.chunk_len - wl.n_prefill_local
        self.peer_qkv_out = torch.full((n_pl, (Hq - wl.hq_loc + 2 * (Hkv - wl.hkv_loc)) * d), float("nan"),
                                       dtype=tdt, device=device)
        self.peer_attn_out = torch.full((n_peer, wl.hq_loc * d), float("nan"), dtype=tdt, device=device)


def upload(inst: Instance, device="cuda") -> DeviceInstance:
    return DeviceInstance(inst, device)


def make_step(inst: Instance, ctx, dev: DeviceInstance | None = None, host_tables: bool = False):
    """A LayerStep of the package for this instance (imports the HIP binding).  With
    ``host_tables`` the descriptor also carries host copies of the page tables, so the
    step checks every page id on the host before it launches."""
    from mixed_prefill_decode_amd import LayerStep, batch_desc, layer_shape, layer_weights
    wl = inst.wl
    dev = dev or upload(inst)
    shape = layer_shape(hidden=wl.hidden, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                        head_dim=wl.head_dim, ffn_dim=wl.ffn_dim, page_size=wl.page_size, rms_eps=wl.rms_eps,
                        rope_base=wl.rope_base, dtype=wl.dtype)
    desc = batch_desc(x=dev.x, n_prefill_local=wl.n_prefill_local, n_decode=wl.n_decode, dec_ctx=dev.dec_ctx,
                      dec_pages=dev.dec_pages if wl.n_decode else None, chunk_len=wl.chunk_len,
                      prior_len=wl.prior_len, sp_degree=wl.sp_degree, sp_rank=wl.sp_rank,
                      local_row_offset=wl.local_row_offset, pre_pages=dev.pre_pages if wl.chunk_len else None,
                      peer_qkv_in=dev.peer_qkv_in, peer_qkv_out=dev.peer_qkv_out,
                      peer_attn_in=dev.peer_attn_in, peer_attn_out=dev.peer_attn_out,
                      dec_ctx_host=inst.dec_ctx if host_tables else None,
                      dec_pages_host=inst.dec_pages if host_tables else None,
                      pre_pages_host=inst.pre_pages if host_tables else None)
    step = LayerStep(ctx, shape, desc, layer_weights(dev.weights), dev.pool, inst.pool.n_pages,
                     keep=(dev,))
    return step, dev


def make_chunked_step(inst, ctx):
    """A ChunkedStep of the package for a multi-chunk instance (device copies only)."""
    from mixed_prefill_decode_amd import ChunkedStep, batch_desc, layer_shape, layer_weights
    wl, dt = inst.wl, inst.wl.dtype
    x = to_device(inst.x, dt)
    weights = {k: to_device(v, dt) for k, v in inst.weights.items()}
    dec_ctx = to_device(inst.dec_ctx, "i32")
    dec_pages = to_device(inst.dec_pages, "i32")
    tables = [to_device(t, "i32") for t in inst.chunk_pages]
    pool = to_device(inst.pool.array, dt)
    shape = layer_shape(hidden=wl.hidden, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                        head_dim=wl.head_dim, ffn_dim=wl.ffn_dim, page_size=wl.page_size, rms_eps=wl.rms_eps,
                        rope_base=wl.rope_base, dtype=dt)
    desc = batch_desc(x=x, n_prefill_local=0, n_decode=wl.n_decode, dec_ctx=dec_ctx,
                      dec_pages=dec_pages if wl.n_decode else None, chunk_len=0, prior_len=0)
    chunks = [(l, c, t) for (l, c), t in zip(wl.chunks, tables)]
    step = ChunkedStep(ctx, shape, desc, chunks, layer_weights(weights), pool, inst.pool.n_pages,
                       keep=(x, weights, dec_ctx, dec_pages))
    step.pool, step.x, step.tables, step.dec_ctx, step.dec_pages = pool, x, tables, dec_ctx, dec_pages
    return step


def make_stack_step(sinst, ctx):
    """A StackStep of the package for a layer-stack instance (device copies only)."""
    import types
    from mixed_prefill_decode_amd import StackStep, batch_desc, layer_shape, layer_weights
    base, wl, dt = sinst.base, sinst.wl, sinst.wl.dtype
    x = to_device(base.x, dt)
    dec_ctx = to_device(base.dec_ctx, "i32")
    dec_pages = to_device(base.dec_pages, "i32")
    pre_pages = to_device(base.pre_pages, "i32")
    weights = [{k: to_device(v, dt) for k, v in layer["weights"].items()} for layer in sinst.layers]
    pools = [upload_pool(types.SimpleNamespace(pool=layer["pool"], wl=wl)) for layer in sinst.layers]
    shape = layer_shape(hidden=wl.hidden, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                        head_dim=wl.head_dim, ffn_dim=wl.ffn_dim, page_size=wl.page_size, rms_eps=wl.rms_eps,
                        rope_base=wl.rope_base, dtype=dt)
    desc = batch_desc(x=x, n_prefill_local=wl.n_prefill_local, n_decode=wl.n_decode, dec_ctx=dec_ctx,
                      dec_pages=dec_pages if wl.n_decode else None, chunk_len=wl.chunk_len,
                      prior_len=wl.prior_len, pre_pages=pre_pages if wl.chunk_len else None)
    step = StackStep(ctx, shape, desc, [layer_weights(w) for w in weights],
                     [(p, layer["pool"].n_pages) for p, layer in zip(pools, sinst.layers)],
                     keep=(x, dec_ctx, dec_pages, pre_pages, weights))
    step.x, step.pool_tensors = x, pools
    return step
