"""xp_decode_attention_static, the decode-attention entry point that allocates nothing (its
split partials live in a static device buffer of the library): through the C ABI, its
output equals xp_decode_attention's with a caller workspace, bit for bit, on two calls in
a row (the second on a smaller batch), device memory stays put, and a batch whose
partials do not fit the buffer is refused before anything is launched."""
import numpy as np
import pytest
import torch

import mixed_prefill_decode_amd as X
from oracle import layer as L
from oracle.numerics import to_f64
from synth import f32_to_bf16_bits, get_workload, make_instance
from synth.device import to_device, to_host_bits, upload_pool
from tests.helpers import rel_fro
from tests.test_gpu_kernels import _append_decode_tokens

pytestmark = pytest.mark.gpu


def _decode(inst, q, dpool, n_d, pps, static):
    wl = inst.wl
    out = torch.full((n_d, wl.n_q_heads * wl.head_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
    args = (X.XP_BF16, q, dpool, inst.pool.n_pages, wl.page_size, to_device(inst.dec_pages[:n_d], "i32"),
            inst.dec_max_blocks, to_device(inst.dec_ctx[:n_d], "i32"), n_d, wl.n_q_heads, wl.n_kv_heads,
            wl.head_dim, out, wl.n_q_heads * wl.head_dim)
    if static:
        X.xp_decode_attention_static(*args, pps)
    else:
        ws = torch.empty(X.xp_decode_workspace_size(n_d, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                                    inst.dec_max_blocks, pps), dtype=torch.uint8, device="cuda")
        X.xp_decode_attention(*args, ws, pps)
    torch.cuda.synchronize()
    return out


def test_static_scratch_decode_matches_the_workspace_entry_point():
    inst = make_instance(get_workload("L1"))
    wl = inst.wl
    dpool = upload_pool(inst)
    rng = np.random.default_rng(11)
    kv = L.PagedKV(inst.pool, "bf16", wl.page_size, wl.head_dim)
    _append_decode_tokens(inst, dpool, rng, kv)          # each request's own token at position c_i
    qh = f32_to_bf16_bits(rng.standard_normal((wl.n_decode, wl.n_q_heads, wl.head_dim)).astype(np.float32))
    q = to_device(qh, "bf16")
    ref = L.decode_attention(to_f64(qh, "bf16"), kv, inst.dec_pages, inst.dec_ctx, wl.n_kv_heads)
    for n_d, pps in ((wl.n_decode, 0), (2, 5)):            # the second call: a smaller batch
        print(f"[no-alloc] {n_d} decodes, pages_per_split {pps}", flush=True)
        got = _decode(inst, q, dpool, n_d, pps, static=True)
        want = _decode(inst, q, dpool, n_d, pps, static=False)
        assert torch.equal(got, want)
        g = to_f64(to_host_bits(got), "bf16").reshape(n_d, wl.n_q_heads, wl.head_dim)
        for i in range(n_d):
            assert rel_fro(g[i], ref[i]) < 5e-3, i
    # no device memory is taken by further calls
    _decode(inst, q, dpool, wl.n_decode, 0, static=True)
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        X.xp_decode_attention_static(X.XP_BF16, q, dpool, inst.pool.n_pages, wl.page_size,
                                     to_device(inst.dec_pages, "i32"), inst.dec_max_blocks,
                                     to_device(inst.dec_ctx, "i32"), wl.n_decode, wl.n_q_heads, wl.n_kv_heads,
                                     wl.head_dim, torch.empty((wl.n_decode, wl.n_q_heads * wl.head_dim),
                                                              dtype=torch.bfloat16, device="cuda"),
                                     wl.n_q_heads * wl.head_dim, 0)
    torch.cuda.synchronize()
    del_free = free0 - torch.cuda.mem_get_info()[0]
    assert del_free <= 0 or del_free < (1 << 20), del_free


def test_static_scratch_decode_refuses_a_batch_too_large():
    # 128 requests of 2049 pages on the 8B head layout: 70 MB of partials > 64 MiB
    dummy = torch.zeros(256, dtype=torch.int32, device="cuda")
    need = X.xp_decode_workspace_size(128, 32, 8, 128, 2049, 0)
    assert need > X.XP_DECODE_STATIC_SCRATCH_BYTES
    with pytest.raises(X.XpError) as e:
        X.xp_decode_attention_static(X.XP_BF16, dummy, dummy, 16, 16, dummy, 2049, dummy, 128, 32, 8, 128, dummy,
                                     32 * 128, 0)
    assert e.value.status == -6 and "static scratch" in str(e.value)
