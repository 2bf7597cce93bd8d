"""Kernel-level parity of the HIP path against the fp64 oracle, through the C ABI.

Tolerances: integer addressing (KV append / gather) bit-exact; attention rel-Frobenius
<= 5e-3 (bf16) / 1e-4 (fp32); GEMM outputs in fp32 rel-Frobenius <= 1e-5, in bf16 <= 5e-3.
"""
import numpy as np
import pytest
import torch

import mixed_prefill_decode_amd as X
from oracle import layer as L
from oracle.numerics import to_f64
from synth import f32_to_bf16_bits, get_workload, make_instance
from synth.device import to_device, to_host_bits, upload_pool
from tests.helpers import rel_fro

pytestmark = pytest.mark.gpu

DT = {"bf16": X.XP_BF16, "f32": X.XP_F32}
ATTN_TOL = {"bf16": 5e-3, "f32": 1e-4}


def _stored(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else a32.astype(np.float32)


def _rand(rng, shape, dtype, scale=1.0):
    return _stored((rng.standard_normal(shape) * scale).astype(np.float32), dtype)


def _sync():
    torch.cuda.synchronize()


def _gemm_ws(dtype, epi, M, N, K):
    n = X.xp_gemm_workspace_size(DT[dtype], epi, M, N, K)
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda"), n


# (300, 512, 4096) is split over K in every epilogue (4 splits), (260, 512, 2048) in
# the single-weight ones (bf16: 2, fp32: 4); 260 and 1040 rows leave the last
# 256-row tile with 4 and 16 live rows
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (67, 200, 256), (130, 257, 192), (300, 512, 1024),
                                   (300, 512, 4096), (260, 512, 2048), (1040, 1024, 1024)])
def test_gemm_epilogues(dtype, M, N, K):
    rng = np.random.default_rng(M * 7919 + N)
    A, B, B2 = _rand(rng, (M, K), dtype), _rand(rng, (N, K), dtype, 0.05), _rand(rng, (N, K), dtype, 0.05)
    Rt, Rf = _rand(rng, (M, N), dtype), rng.standard_normal((M, N)).astype(np.float32)
    a64, b64, b264 = (to_f64(v, dtype) for v in (A, B, B2))
    acc = a64 @ b64.T
    dA, dB, dB2 = (to_device(v, dtype) for v in (A, B, B2))
    dRt, dRf = to_device(Rt, dtype), torch.from_numpy(Rf).cuda()
    C32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    for epi, R, ref in ((X.XP_EPI_F32, None, acc), (X.XP_EPI_ADD_T, dRt, to_f64(Rt, dtype) + acc),
                        (X.XP_EPI_ADD_F32, dRf, Rf.astype(np.float64) + acc)):
        ws, n = _gemm_ws(dtype, epi, M, N, K)
        X.xp_gemm(DT[dtype], epi, dA, dB, None, R, C32, M, N, K, ws, n)
        _sync()
        assert rel_fro(C32.cpu().numpy(), ref) < 1e-5, epi
    Cs = torch.empty((M, N), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    ws, n = _gemm_ws(dtype, X.XP_EPI_SWIGLU, M, N, K)
    X.xp_gemm(DT[dtype], X.XP_EPI_SWIGLU, dA, dB, dB2, None, Cs, M, N, K, ws, n)
    _sync()
    g, u = acc, a64 @ b264.T
    ref = g / (1 + np.exp(-g)) * u
    assert rel_fro(to_f64(to_host_bits(Cs), dtype), ref) < (5e-3 if dtype == "bf16" else 1e-5)


# (M, N) pairs whose unsplit products make the launcher take each of its work-unit
# shapes (found with xp_gemm_tile; the choice does not depend on K when K is not split)
GEMM_TILE_SHAPES = {"single": [(128, 6144), (536, 5120), (1040, 6144), (1040, 4096), (536, 14336), (8216, 7168)],
                    "dual": [(128, 14336), (1040, 14336), (536, 5120), (536, 7168), (8216, 17408)]}


@pytest.mark.parametrize("kind", ["single", "dual"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gemm_every_tile_shape(kind, dtype):
    # every work-unit shape of the launcher, against the fp64 product on sampled rows
    K = 128
    epi = X.XP_EPI_SWIGLU if kind == "dual" else X.XP_EPI_F32
    seen = set()
    for M, N in GEMM_TILE_SHAPES[kind]:
        bm, bn, sp = X.xp_gemm_tile(DT[dtype], epi, M, N, K)
        assert sp == 1
        seen.add((bm, bn))
        rng = np.random.default_rng(M + N)
        A, B, B2 = _rand(rng, (M, K), dtype), _rand(rng, (N, K), dtype, 0.05), _rand(rng, (N, K), dtype, 0.05)
        odt = torch.bfloat16 if (epi == X.XP_EPI_SWIGLU and dtype == "bf16") else torch.float32
        C = torch.empty((M, N), dtype=odt, device="cuda")
        X.xp_gemm(DT[dtype], epi, to_device(A, dtype), to_device(B, dtype), to_device(B2, dtype) if kind == "dual"
                  else None, None, C, M, N, K)
        _sync()
        rows = np.unique(np.concatenate([np.arange(min(M, 40)), rng.integers(0, M, 200), np.arange(max(0, M - 40), M)]))
        a64 = to_f64(A, dtype)[rows]
        g = a64 @ to_f64(B, dtype).T
        if kind == "dual":
            ref = g / (1 + np.exp(-g)) * (a64 @ to_f64(B2, dtype).T)
            got = to_f64(to_host_bits(C), dtype)[rows] if dtype == "bf16" else C.cpu().numpy()[rows].astype(np.float64)
            tol = 5e-3 if dtype == "bf16" else 1e-5
        else:
            ref, got, tol = g, C.cpu().numpy()[rows].astype(np.float64), 1e-5
        assert rel_fro(got, ref) < tol, (M, N, bm, bn)
    want = {"single": {(64, 128), (96, 128), (128, 256), (192, 128), (192, 192), (256, 256)},
            "dual": {(128, 64), (128, 128), (192, 64), (192, 128), (256, 128)}}[kind]
    assert seen == want


def test_gemm_rows_do_not_depend_on_the_batch():
    # the same rows inside batches of 40 (64-row tiles) and 300 (128-row tiles): bit-identical
    rng = np.random.default_rng(3)
    K, N = 512, 384
    A = _rand(rng, (300, K), "bf16")
    B = _rand(rng, (N, K), "bf16", 0.05)
    dA, dB = to_device(A, "bf16"), to_device(B, "bf16")
    full = torch.empty((300, N), dtype=torch.float32, device="cuda")
    X.xp_gemm(X.XP_BF16, X.XP_EPI_F32, dA, dB, None, None, full, 300, N, K)
    part = torch.empty((40, N), dtype=torch.float32, device="cuda")
    X.xp_gemm(X.XP_BF16, X.XP_EPI_F32, dA[100:140].contiguous(), dB, None, None, part, 40, N, K)
    _sync()
    assert torch.equal(full[100:140], part)


@pytest.mark.parametrize("epi", [X.XP_EPI_F32, X.XP_EPI_ADD_F32, X.XP_EPI_SWIGLU])
def test_gemm_split_rows_do_not_depend_on_the_batch(epi):
    # long-K products summed over K chunks (the down-projection shape of an 8B layer,
    # and a gate/up shape with chunks): rows inside a 1040-row batch equal the same rows
    # computed alone, bit for bit, whether the chunks ran as separate units (16 rows)
    # or folded inside one unit per tile (1040 rows of the single-weight products)
    N, K = (4096, 14336) if epi != X.XP_EPI_SWIGLU else (512, 4096)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    A = torch.randn(1040, K, device="cuda", generator=gen).bfloat16()
    B = (torch.randn(N, K, device="cuda", generator=gen) * 0.05).bfloat16()
    B2 = (torch.randn(N, K, device="cuda", generator=gen) * 0.05).bfloat16() if epi == X.XP_EPI_SWIGLU else None
    R = torch.randn(1040, N, device="cuda", generator=gen)
    odt = torch.bfloat16 if epi == X.XP_EPI_SWIGLU else torch.float32
    outs = []
    for lo, hi in ((0, 1040), (1024, 1040)):
        M = hi - lo
        ws, n = _gemm_ws("bf16", epi, M, N, K)
        split = X.xp_gemm_tile(X.XP_BF16, epi, M, N, K)[2] > 1
        assert split == (M == 16 or epi == X.XP_EPI_SWIGLU)
        assert (n > 0) == split
        C = torch.empty((M, N), dtype=odt, device="cuda")
        X.xp_gemm(X.XP_BF16, epi, A[lo:hi].contiguous(), B, B2, R[lo:hi].contiguous() if epi == X.XP_EPI_ADD_F32
                  else None, C, M, N, K, ws, n)
        outs.append(C)
    _sync()
    view = torch.int16 if odt == torch.bfloat16 else torch.int32
    assert torch.equal(outs[0][1024:].view(view), outs[1].view(view))
    if epi != X.XP_EPI_SWIGLU:
        # and against the fp64 product on a few rows (fp32 output)
        rows = [0, 517, 1039]
        ref = A[rows].double() @ B.double().T + (R[rows].double() if epi == X.XP_EPI_ADD_F32 else 0)
        assert rel_fro(outs[0][rows].double().cpu().numpy(), ref.cpu().numpy()) < 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rmsnorm(dtype):
    rng = np.random.default_rng(4)
    M, H = 37, 640
    x = _rand(rng, (M, H), dtype, 3.0)
    g = _rand(rng, (H,), dtype)
    y = torch.empty((M, H), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    X.xp_rmsnorm(DT[dtype], to_device(x, dtype), 0, to_device(g, dtype), y, M, H, 1e-5)
    xf = rng.standard_normal((M, H)).astype(np.float32) * 2
    y2 = torch.empty_like(y)
    X.xp_rmsnorm(DT[dtype], torch.from_numpy(xf).cuda(), 1, to_device(g, dtype), y2, M, H, 1e-5)
    _sync()
    tol = 3e-3 if dtype == "bf16" else 1e-6
    ref = L.rmsnorm(to_f64(x, dtype), to_f64(g, dtype), 1e-5)
    assert rel_fro(to_f64(to_host_bits(y), dtype), ref) < tol
    ref2 = L.rmsnorm(xf.astype(np.float64), to_f64(g, dtype), 1e-5)
    assert rel_fro(to_f64(to_host_bits(y2), dtype), ref2) < tol


def _append_decode_tokens(inst, dpool, rng, kv):
    """Append random K/V of every decode request's new position on both sides."""
    wl, dt = inst.wl, inst.wl.dtype
    n = wl.n_decode * wl.n_kv_heads
    k = _rand(rng, (n, wl.head_dim), dt)
    v = _rand(rng, (n, wl.head_dim), dt)
    seq = np.arange(n, dtype=np.int32)
    pos = np.repeat(inst.dec_ctx, wl.n_kv_heads).astype(np.int32)
    table = inst.dec_pages.reshape(n, -1)
    X.xp_kv_append(DT[dt], dpool, inst.pool.n_pages, wl.page_size, wl.head_dim, to_device(table, "i32"),
                   table.shape[1], to_device(seq, "i32"), to_device(pos, "i32"), to_device(k, dt),
                   to_device(v, dt), n)
    k64, v64 = to_f64(k, dt), to_f64(v, dt)
    for t in range(n):
        kv.write(table[t], int(pos[t]), k64[t], v64[t])


def _append_chunk_tokens(inst, dpool, rng, kv):
    wl, dt = inst.wl, inst.wl.dtype
    n = wl.chunk_len * wl.hkv_loc
    k = _rand(rng, (n, wl.head_dim), dt)
    v = _rand(rng, (n, wl.head_dim), dt)
    seq = np.repeat(np.arange(wl.hkv_loc, dtype=np.int32), wl.chunk_len)
    pos = np.tile(wl.prior_len + np.arange(wl.chunk_len, dtype=np.int32), wl.hkv_loc)
    X.xp_kv_append(DT[dt], dpool, inst.pool.n_pages, wl.page_size, wl.head_dim, to_device(inst.pre_pages, "i32"),
                   inst.pre_pages.shape[1], to_device(seq, "i32"), to_device(pos, "i32"), to_device(k, dt),
                   to_device(v, dt), n)
    k64, v64 = to_f64(k, dt), to_f64(v, dt)
    for t in range(n):
        kv.write(inst.pre_pages[seq[t]], int(pos[t]), k64[t], v64[t])


@pytest.mark.parametrize("name", ["P1", "P2", "E1", "C1", "E3"])
def test_kv_append_and_gather_bit_exact(name):
    inst = make_instance(get_workload(name))
    wl, dt = inst.wl, inst.wl.dtype
    rng = np.random.default_rng(5)
    dpool = upload_pool(inst)
    kv = L.PagedKV(inst.pool, dt, wl.page_size, wl.head_dim)
    _append_decode_tokens(inst, dpool, rng, kv)
    _sync()
    host = to_host_bits(dpool)
    for p in range(inst.pool.n_pages):
        assert np.array_equal(host[p], kv.stored_page(p), equal_nan=True) if dt == "f32" else \
            np.array_equal(host[p], kv.stored_page(p)), p
    n = wl.n_decode * wl.n_kv_heads
    lens = np.repeat(inst.dec_ctx + 1, wl.n_kv_heads).astype(np.int32)
    max_len = int(lens.max())
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    ko = torch.zeros((n, max_len, wl.head_dim), dtype=tdt, device="cuda")
    vo = torch.zeros_like(ko)
    table = inst.dec_pages.reshape(n, -1)
    X.xp_kv_gather(DT[dt], dpool, inst.pool.n_pages, wl.page_size, wl.head_dim, to_device(table, "i32"),
                   table.shape[1], to_device(lens, "i32"), n, max_len, ko, vo)
    _sync()
    kh, vh = to_host_bits(ko), to_host_bits(vo)
    for t in range(n):
        K, V = kv.read(table[t], int(lens[t]))
        from oracle.numerics import encode
        assert np.array_equal(kh[t, :lens[t]], encode(K, dt)) and np.array_equal(vh[t, :lens[t]], encode(V, dt))


@pytest.mark.parametrize("name", ["P1", "P2", "P3", "E1", "C1", "E3"])
@pytest.mark.parametrize("pps", [0, 1, 5, 32, 64])
def test_decode_attention(name, pps):
    inst = make_instance(get_workload(name))
    wl, dt = inst.wl, inst.wl.dtype
    rng = np.random.default_rng(6)
    dpool = upload_pool(inst)
    kv = L.PagedKV(inst.pool, dt, wl.page_size, wl.head_dim)
    _append_decode_tokens(inst, dpool, rng, kv)
    q = _rand(rng, (wl.n_decode, wl.n_q_heads, wl.head_dim), dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.full((wl.n_decode, wl.n_q_heads * wl.head_dim), float("nan"), dtype=tdt, device="cuda")
    ws = torch.empty(X.xp_decode_workspace_size(wl.n_decode, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, inst.dec_max_blocks, pps),
                     dtype=torch.uint8, device="cuda")
    X.xp_decode_attention(DT[dt], to_device(q, dt), dpool, inst.pool.n_pages, wl.page_size,
                          to_device(inst.dec_pages, "i32"), inst.dec_max_blocks, to_device(inst.dec_ctx, "i32"),
                          wl.n_decode, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, out, wl.n_q_heads * wl.head_dim,
                          ws, pps)
    _sync()
    ref = L.decode_attention(to_f64(q, dt), kv, inst.dec_pages, inst.dec_ctx, wl.n_kv_heads)
    got = to_f64(to_host_bits(out), dt).reshape(ref.shape)
    assert np.isfinite(got).all()
    assert rel_fro(got, ref) < ATTN_TOL[dt]
    for i in range(wl.n_decode):      # per request as well (short contexts are not drowned out)
        assert rel_fro(got[i], ref[i]) < 2 * ATTN_TOL[dt], i


def test_decode_attention_long_contexts():
    """Identical inputs at 502, 8K, 32K and 49K cached tokens on the 32B head layout (the
    longest decode of the 32B batch takes the most key splits): each request within the
    attention bar on its own, in the split size the layer picks and in single-page splits."""
    inst = make_instance(get_workload("L1"))
    wl, dt = inst.wl, inst.wl.dtype
    rng = np.random.default_rng(8)
    dpool = upload_pool(inst)
    kv = L.PagedKV(inst.pool, dt, wl.page_size, wl.head_dim)
    _append_decode_tokens(inst, dpool, rng, kv)
    q = _rand(rng, (wl.n_decode, wl.n_q_heads, wl.head_dim), dt)
    ref = L.decode_attention(to_f64(q, dt), kv, inst.dec_pages, inst.dec_ctx, wl.n_kv_heads)
    errs = {}
    for pps in (0, 1):
        out = torch.full((wl.n_decode, wl.n_q_heads * wl.head_dim), float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        ws = torch.empty(X.xp_decode_workspace_size(wl.n_decode, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                                    inst.dec_max_blocks, pps), dtype=torch.uint8, device="cuda")
        X.xp_decode_attention(DT[dt], to_device(q, dt), dpool, inst.pool.n_pages, wl.page_size,
                              to_device(inst.dec_pages, "i32"), inst.dec_max_blocks,
                              to_device(inst.dec_ctx, "i32"), wl.n_decode, wl.n_q_heads, wl.n_kv_heads,
                              wl.head_dim, out, wl.n_q_heads * wl.head_dim, ws, pps)
        _sync()
        got = to_f64(to_host_bits(out), dt).reshape(ref.shape)
        assert np.isfinite(got).all()
        errs[pps] = [rel_fro(got[i], ref[i]) for i in range(wl.n_decode)]
    print(f"[decode long] per-request rel-Frobenius {dict(zip(inst.dec_ctx.tolist(), errs[0]))} "
          f"(single-page splits {errs[1]})", flush=True)
    for pps, e in errs.items():
        assert max(e) < ATTN_TOL[dt], (pps, e)


@pytest.mark.parametrize("name", ["P1", "P2", "P3", "P4", "P5", "P6", "P7", "P8", "P9", "P10", "E2", "C1", "E4", "E5"])
def test_prefill_attention(name):
    inst = make_instance(get_workload(name))
    wl, dt = inst.wl, inst.wl.dtype
    rng = np.random.default_rng(7)
    dpool = upload_pool(inst)
    kv = L.PagedKV(inst.pool, dt, wl.page_size, wl.head_dim)
    _append_chunk_tokens(inst, dpool, rng, kv)
    l, hq, d = wl.chunk_len, wl.hq_loc, wl.head_dim
    q = _rand(rng, (hq, l, d), dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    n_loc, off = wl.n_prefill_local, wl.local_row_offset
    out_l = torch.full((max(n_loc, 1), hq * d), float("nan"), dtype=tdt, device="cuda")
    out_p = torch.full((max(l - n_loc, 1), hq * d), float("nan"), dtype=tdt, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(X.xp_prefill_workspace_size(hq, wl.hkv_loc, d, wl.prior_len, l), 1), dtype=torch.uint8,
                     device="cuda")
    X.xp_prefill_attention(DT[dt], to_device(q, dt), dpool, inst.pool.n_pages, wl.page_size,
                           to_device(inst.pre_pages, "i32"), inst.pre_max_blocks, hq, wl.hkv_loc, d, wl.prior_len,
                           l, off, n_loc, out_l, hq * d, out_p, hq * d, ws, status)
    _sync()
    ref = L.prefill_attention(to_f64(q, dt).transpose(1, 0, 2), kv, inst.pre_pages, wl.prior_len, wl.group)
    ref = ref.reshape(l, hq * d)
    loc = [t for t in range(l) if off <= t < off + n_loc]
    peer = [t for t in range(l) if not (off <= t < off + n_loc)]
    got_l = to_f64(to_host_bits(out_l), dt)[:n_loc]
    got_p = to_f64(to_host_bits(out_p), dt)[:len(peer)]
    assert int(status.item()) == 0
    if loc:
        assert np.isfinite(got_l).all() and rel_fro(got_l, ref[loc]) < ATTN_TOL[dt]
    if peer:
        assert np.isfinite(got_p).all() and rel_fro(got_p, ref[peer]) < ATTN_TOL[dt]
    # every row, including the first chunk rows that see only a few keys
    full = np.zeros_like(ref)
    full[loc], full[peer] = got_l, got_p
    for t in sorted({0, min(1, l - 1), l // 2, l - 1}):
        assert rel_fro(full[t], ref[t]) < 2 * ATTN_TOL[dt], t


def test_prefill_out_of_range_page_is_flagged_not_dereferenced():
    """A page id outside the pool in one KV head's chunk table: the status bit is set, the
    query tiles whose staged key range covers that page come out as NaN on that head's query
    heads, and every other row (the earlier tile, the other KV head) is the oracle's."""
    inst = make_instance(get_workload("E2"))      # bf16, 8 q heads on 2 kv heads, 130 after 33
    wl, dt = inst.wl, inst.wl.dtype
    rng = np.random.default_rng(11)
    dpool = upload_pool(inst)
    kv = L.PagedKV(inst.pool, dt, wl.page_size, wl.head_dim)
    _append_chunk_tokens(inst, dpool, rng, kv)
    l, hq, hkv, d = wl.chunk_len, wl.hq_loc, wl.hkv_loc, wl.head_dim
    q = _rand(rng, (hq, l, d), dt)
    ref = L.prefill_attention(to_f64(q, dt).transpose(1, 0, 2), kv, inst.pre_pages, wl.prior_len, wl.group)
    ref = ref.reshape(l, hq * d)
    bad_pages = inst.pre_pages.copy()
    bad_pages[1, 7] = inst.pool.n_pages + 5       # kv head 1, keys 112..127
    tdt = torch.bfloat16
    out = torch.full((l, hq * d), 7.0, dtype=tdt, device="cuda")
    peer = torch.empty((1, hq * d), dtype=tdt, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(X.xp_prefill_workspace_size(hq, hkv, d, wl.prior_len, l), 1), dtype=torch.uint8,
                     device="cuda")
    pool0 = dpool.clone()
    X.xp_prefill_attention(DT[dt], to_device(q, dt), dpool, inst.pool.n_pages, wl.page_size,
                           to_device(bad_pages, "i32"), inst.pre_max_blocks, hq, hkv, d, wl.prior_len, l, 0, l,
                           out, hq * d, peer, hq * d, ws, status)
    _sync()
    assert int(status.item()) & X.XP_DEV_BAD_PAGE
    assert torch.equal(dpool.view(torch.int16), pool0.view(torch.int16))
    got = to_f64(to_host_bits(out), dt)
    g = wl.group
    head1 = slice(g * d, 2 * g * d)                # the query heads of kv head 1
    # tile 0 (queries 0..31) stages keys below 96 only; every later tile's range reaches 127
    assert np.isnan(got[32:, head1]).all()
    assert np.isfinite(got[:32, head1]).all() and rel_fro(got[:32, head1], ref[:32, head1]) < ATTN_TOL[dt]
    assert np.isfinite(got[:, :g * d]).all() and rel_fro(got[:, :g * d], ref[:, :g * d]) < ATTN_TOL[dt]


def test_decode_token_matches_prefill_row_on_gpu():
    # decode attention of a query at position c+t over the chunk's own table equals prefill row t
    inst = make_instance(get_workload("E2"))
    wl, dt = inst.wl, inst.wl.dtype
    rng = np.random.default_rng(8)
    dpool = upload_pool(inst)
    kv = L.PagedKV(inst.pool, dt, wl.page_size, wl.head_dim)
    _append_chunk_tokens(inst, dpool, rng, kv)
    l, hq, d, G = wl.chunk_len, wl.hq_loc, wl.head_dim, wl.group
    q = _rand(rng, (hq, l, d), dt)
    out_l = torch.empty((l, hq * d), dtype=torch.bfloat16, device="cuda")
    pws = torch.empty(max(X.xp_prefill_workspace_size(hq, wl.hkv_loc, d, wl.prior_len, l), 1), dtype=torch.uint8,
                      device="cuda")
    X.xp_prefill_attention(DT[dt], to_device(q, dt), dpool, inst.pool.n_pages, wl.page_size,
                           to_device(inst.pre_pages, "i32"), inst.pre_max_blocks, hq, wl.hkv_loc, d, wl.prior_len,
                           l, 0, l, out_l, hq * d, None, hq * d, pws)
    # the same queries as decode requests: request t has context prior + t on kv head g's table
    rows = [0, 5, l - 1]
    for g in range(wl.hkv_loc):
        qd = np.ascontiguousarray(q[g * G:(g + 1) * G].transpose(1, 0, 2)[rows])       # [n, G, d]
        tables = np.repeat(inst.pre_pages[g:g + 1][None], len(rows), axis=0)           # [n, 1, blocks]
        ctx = (wl.prior_len + np.array(rows)).astype(np.int32)
        out_d = torch.empty((len(rows), G * d), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(X.xp_decode_workspace_size(len(rows), G, 1, d, tables.shape[2], 4), dtype=torch.uint8,
                         device="cuda")
        X.xp_decode_attention(DT[dt], to_device(qd, dt), dpool, inst.pool.n_pages, wl.page_size,
                              to_device(tables, "i32"), tables.shape[2], to_device(ctx, "i32"), len(rows), G, 1, d,
                              out_d, G * d, ws, 4)
        _sync()
        a = to_f64(to_host_bits(out_d), dt)
        b = to_f64(to_host_bits(out_l), dt)[rows][:, g * G * d:(g + 1) * G * d]
        assert rel_fro(a, b) < 5e-3


def test_read_probe_reads_every_piece():
    # a thread writes the sink only when the XOR of the words it read equals 0x9e3779b9;
    # here each 16-byte piece is one thread's
    buf = torch.zeros(4096, dtype=torch.int32, device="cuda")
    buf[4093] = int(np.int32(np.uint32(0x9E3779B9).view(np.int32)))   # the last 16-byte piece
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    X.xp_probe_read(buf, buf.numel() * 4, sink)
    torch.cuda.synchronize()
    assert int(np.int32(sink.item()).view(np.uint32)) == 0x9E3779B9
    buf[4092] = 1                                                      # that piece's XOR changes
    sink.zero_()
    X.xp_probe_read(buf, buf.numel() * 4, sink)
    torch.cuda.synchronize()
    assert sink.item() == 0
    with pytest.raises(X.XpError):
        X.xp_probe_read(buf, 10, sink)
