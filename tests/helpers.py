"""Marshalling helpers shared by the tests, and the teacher-forced check of the last stage."""
import numpy as np

# Teacher-forced last stage: out = h1 + act W_down^T from the GPU's own h1 and act.  The
# kernel multiplies bf16 (or fp32) operands and accumulates in fp32, so its error against
# the fp64 value is a few fp32 roundings of the partial sums.  The bar compares it with the
# same arithmetic done by an independent fp32 accumulation (numpy's float32 product of the
# same operands, another summation order): the kernel's worst row error may be at most
# TF_FACTOR times the fp32 product's, with one fp32 rounding of the largest output as a
# floor.  Accumulating in a narrower type, or dropping or repeating a term, fails it.
TF_FACTOR = 4.0
U32 = 2.0 ** -24


def down_stage_errors(out, h1, act, wd):
    """(the GPU's max-abs error, the fp32 product's max-abs error, the bar) of the last
    stage on the given rows, all against fp64; `out`, `h1`, `act` are the rows' values as
    the GPU holds them (act already rounded to its dtype), `wd` the stored down weight."""
    out, h1, act, wd = (np.asarray(a, dtype=np.float64) for a in (out, h1, act, wd))
    exact = h1 + act @ wd.T
    f32 = h1.astype(np.float32) + act.astype(np.float32) @ wd.astype(np.float32).T
    e_gpu = float(np.abs(out - exact).max())
    e_f32 = float(np.abs(f32.astype(np.float64) - exact).max())
    return e_gpu, e_f32, TF_FACTOR * max(e_f32, U32 * float(np.abs(exact).max()))


def oracle_kwargs(inst, **extra):
    """Keyword arguments of ``oracle.layer.layer_forward`` for a drawn instance."""
    wl = inst.wl
    kw = dict(hidden=wl.hidden, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
              head_dim=wl.head_dim, ffn_dim=wl.ffn_dim, page_size=wl.page_size,
              rms_eps=wl.rms_eps, rope_base=wl.rope_base, dtype=wl.dtype, x=inst.x,
              weights=inst.weights, dec_ctx=inst.dec_ctx, dec_pages=inst.dec_pages,
              chunk_len=wl.chunk_len, prior_len=wl.prior_len, sp_degree=wl.sp_degree,
              sp_rank=wl.sp_rank, n_prefill_local=wl.n_prefill_local,
              local_row_offset=wl.local_row_offset, pre_pages=inst.pre_pages,
              peer_qkv_in=inst.peer_qkv_in, peer_attn_in=inst.peer_attn_in, pool=inst.pool)
    kw.update(extra)
    return kw


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


class ArrayPool:
    """``pool[ids]`` over a plain stored array (for tests that build their own pool)."""

    def __init__(self, array):
        self.array = array

    def __getitem__(self, ids):
        return self.array[np.asarray(ids, dtype=np.int64)]


def chunk_oracle_kwargs(inst, **extra):
    """Keyword arguments of ``oracle.layer.layer_forward_chunks`` for a multi-chunk instance."""
    wl = inst.wl
    kw = dict(hidden=wl.hidden, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
              head_dim=wl.head_dim, ffn_dim=wl.ffn_dim, page_size=wl.page_size,
              rms_eps=wl.rms_eps, rope_base=wl.rope_base, dtype=wl.dtype, x=inst.x,
              weights=inst.weights, dec_ctx=inst.dec_ctx, dec_pages=inst.dec_pages,
              chunks=[(l, c, t) for (l, c), t in zip(wl.chunks, inst.chunk_pages)], pool=inst.pool)
    kw.update(extra)
    return kw


def stack_oracle_kwargs(sinst, **extra):
    """Keyword arguments of ``oracle.layer.stack_forward`` for a drawn stack instance."""
    kw = oracle_kwargs(sinst.base)
    for k in ("weights", "pool"):
        kw.pop(k)
    kw["layers"] = sinst.layers
    kw.update(extra)
    return kw


# Contexts shared by the GPU test modules, keyed by decode CU count; closed at the end
# of the session (conftest.pytest_sessionfinish), before interpreter exit.
_CTXS = {}


def shared_ctx(decode_cus=0):
    import mixed_prefill_decode_amd as X
    c = _CTXS.get(decode_cus)
    if c is None or c.handle is None:
        c = _CTXS[decode_cus] = X.Ctx(0, decode_cus, 0)
    return c


def close_shared_ctxs():
    for c in _CTXS.values():
        c.close()
    _CTXS.clear()


class DevicePages:
    """``pool[ids]`` over a device pool tensor: copies just those pages to the host in the
    storage format (for oracle checks on pools too large to copy whole)."""

    def __init__(self, tensor):
        self.tensor = tensor

    def __getitem__(self, ids):
        import torch
        from synth.device import to_host_bits
        idx = torch.as_tensor(np.asarray(ids, dtype=np.int64), device=self.tensor.device)
        return to_host_bits(self.tensor[idx])


def k_slots(plane, page_size, head_dim, dtype):
    """A stored K plane (flat, the ABI's chunk-major page format) as [slot, dim]."""
    E = 8 if dtype == "bf16" else 4
    return np.asarray(plane).reshape(head_dim // E, page_size, E).transpose(1, 0, 2).reshape(page_size, head_dim)
