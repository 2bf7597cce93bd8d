"""Pins of the oracle's attention (decode, prefill, paging) -- CPU only."""
import numpy as np
import pytest
import torch

from oracle import brute
from oracle import layer as L
from oracle.numerics import encode
from tests.helpers import ArrayPool, k_slots


def _rng(s):
    return np.random.default_rng(s)


def test_attend_matches_pure_python_brute_force():
    r = _rng(1)
    for nk in (1, 2, 7, 33):
        q = r.standard_normal((3, 8)); K = r.standard_normal((nk, 8)); V = r.standard_normal((nk, 8))
        o, p = L.attend(q, K, V)
        for h in range(3):
            ob = brute.brute_attention(list(q[h]), [list(k) for k in K], [list(v) for v in V])
            assert np.allclose(o[h], ob, atol=1e-13, rtol=0)


def test_attend_closed_forms():
    r = _rng(2)
    K = r.standard_normal((9, 16)); V = r.standard_normal((9, 16))
    o, p = L.attend(np.zeros((1, 16)), K, V)           # q = 0: uniform weights -> mean of V
    assert np.allclose(o[0], V.mean(axis=0), atol=1e-14)
    o, p = L.attend(r.standard_normal((2, 16)), K[:1], V[:1])   # one visible key -> v
    assert np.allclose(o, V[:1].repeat(2, axis=0), atol=0)
    o, p = L.attend(r.standard_normal((5, 16)) * 4, K, V)
    assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-12)


def test_attend_against_torch_sdpa_causal():
    # library routine: torch scaled_dot_product_attention in float64 with its own causal mask
    r = _rng(3)
    n, d = 37, 16
    q = r.standard_normal((n, d)); K = r.standard_normal((n, d)); V = r.standard_normal((n, d))
    mask = np.arange(n)[None, :] <= np.arange(n)[:, None]
    o, _ = L.attend(q, K, V, mask)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
        is_causal=True)[0, 0].numpy()
    assert np.allclose(o, ref, atol=1e-12)


def _build_pool(K_seq, V_seq, S, dtype, rnd, extra_pages=3):
    """Write contiguous per-head K/V [n, d] sequences into a shuffled pool with the ABI layout
    (plane 0 K in 16-byte chunks chunk-major over the slots: 4 fp32 per chunk here; plane 1
    dim-major V); unused slots NaN."""
    n_heads = len(K_seq)
    n, d = K_seq[0].shape
    nb = -(-n // S)
    n_pages = n_heads * nb + extra_pages
    perm = rnd.permutation(n_pages)
    pool = np.full((n_pages, 2, S * d), np.nan, dtype=np.float32)
    table = np.full((n_heads, nb), -1, dtype=np.int32)
    it = 0
    for h in range(n_heads):
        for b in range(nb):
            p = perm[it]; it += 1
            table[h, b] = p
            for s in range(S):
                pos = b * S + s
                if pos < n:
                    for j in range(d):
                        pool[p, 0, ((j // 4) * S + s) * 4 + j % 4] = K_seq[h][pos][j]
                    pool[p, 1, np.arange(d) * S + s] = V_seq[h][pos]
    return ArrayPool(pool), table


def test_paged_read_equals_contiguous_and_never_touches_tails():
    r = _rng(4)
    S, d = 16, 8
    for n in (1, 15, 16, 17, 50):
        Ks = [r.standard_normal((n, d)).astype(np.float32).astype(np.float64) for _ in range(2)]
        Vs = [r.standard_normal((n, d)).astype(np.float32).astype(np.float64) for _ in range(2)]
        pool, table = _build_pool(Ks, Vs, S, "f32", r)
        kv = L.PagedKV(pool, "f32", S, d)
        for h in range(2):
            K, V = kv.read(table[h], n)
            assert np.array_equal(K, Ks[h]) and np.array_equal(V, Vs[h])
            assert np.isfinite(K).all() and np.isfinite(V).all()


def test_decode_attention_paged_matches_brute_and_mha_special_case():
    r = _rng(5)
    S, d, Hq, Hkv = 16, 8, 4, 2
    ctx = np.array([0, 5, 16, 40])
    n_d = len(ctx)
    q = r.standard_normal((n_d, Hq, d))
    Ks = [[r.standard_normal((c + 1, d)).astype(np.float32).astype(np.float64) for _ in range(Hkv)] for c in ctx]
    Vs = [[r.standard_normal((c + 1, d)).astype(np.float32).astype(np.float64) for _ in range(Hkv)] for c in ctx]
    maxb = max(-(-(c + 1) // S) for c in ctx)
    pools, tables = [], np.full((n_d, Hkv, maxb), -1, dtype=np.int32)
    # one shared pool: concatenate requests' pages
    rows, off = [], 0
    for i in range(n_d):
        p, t = _build_pool(Ks[i], Vs[i], S, "f32", r, extra_pages=0)
        rows.append(p.array)
        tables[i, :, :t.shape[1]] = t + off
        off += p.array.shape[0]
    pool = ArrayPool(np.concatenate(rows))
    kv = L.PagedKV(pool, "f32", S, d)
    o = L.decode_attention(q, kv, tables, ctx, Hkv)
    for i in range(n_d):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            ob = brute.brute_attention(list(q[i, h]), [list(k) for k in Ks[i][g]], [list(v) for v in Vs[i][g]])
            assert np.allclose(o[i, h], ob, atol=1e-13)
    # G = 1 reduces to multi-head attention: read the same pages as Hq = Hkv heads
    o_mha = L.decode_attention(q[:, ::2].copy(), kv, tables, ctx, Hkv)
    assert np.allclose(o_mha, o[:, ::2], atol=0)


def test_prefill_attention_against_sdpa_with_prior_and_gqa():
    r = _rng(6)
    S, d, G = 16, 16, 3
    c, l = 21, 30
    n = c + l
    Ks = [r.standard_normal((n, d)).astype(np.float32).astype(np.float64)]
    Vs = [r.standard_normal((n, d)).astype(np.float32).astype(np.float64)]
    pool, table = _build_pool(Ks, Vs, S, "f32", r)
    kv = L.PagedKV(pool, "f32", S, d)
    q = r.standard_normal((l, G, d))
    o = L.prefill_attention(q, kv, table, c, G)
    # library: torch SDPA with an explicit boolean mask (query t sees keys <= c + t)
    mask = torch.from_numpy(np.arange(n)[None, :] <= (c + np.arange(l))[:, None])
    for h in range(G):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, h])[None, None], torch.from_numpy(Ks[0])[None, None],
            torch.from_numpy(Vs[0])[None, None], attn_mask=mask)[0, 0].numpy()
        assert np.allclose(o[:, h], ref, atol=1e-12)


def test_visible_pairs_equal_the_pages_workload_count():
    # V rows = one-hot key indicators: the output weights expose exactly which keys each
    # query saw; their count must be l c + l (l + 1) / 2 (ConfluxServe Eq. 9; Adaptive Context
    # Parallelism Eq. 1) and every weight positive.
    S = 16
    for c, l in ((0, 1), (0, 19), (13, 7), (32, 16)):
        n = c + l
        d = -(-n // 4) * 4          # whole 16-byte chunks of fp32 in the stored K plane
        r = _rng(c * 100 + l)
        Ks = [r.standard_normal((n, d)) * 0.1]
        Vs = [np.eye(n, d)]         # key j's V row is the indicator of column j
        pool, table = _build_pool(Ks, Vs, S, "f32", r)
        kv = L.PagedKV(pool, "f32", S, d)
        q = r.standard_normal((l, 1, d)) * 0.1
        o = L.prefill_attention(q, kv, table, c, 1)
        seen = (np.abs(o[:, 0]) > 0).sum()
        assert seen == l * c + l * (l + 1) // 2 == L.causal_pair_count(l, c)
        assert np.allclose(o[:, 0].sum(axis=-1), 1.0, atol=1e-6)
        # query t sees exactly keys 0..c+t
        for t in range(l):
            assert np.all(np.abs(o[t, 0, :c + t + 1]) > 0) and np.all(o[t, 0, c + t + 1:] == 0)


def test_decode_token_equals_prefill_row_over_same_kv():
    # a decode request with context c_i over the same KV as a chunk row at position c_i
    r = _rng(8)
    S, d, G = 16, 8, 2
    c, l = 10, 12
    n = c + l
    Ks = [r.standard_normal((n, d))]
    Vs = [r.standard_normal((n, d))]
    pool, table = _build_pool(Ks, Vs, S, "f32", r)
    kv = L.PagedKV(pool, "f32", S, d)
    q = r.standard_normal((l, G, d))
    o_pre = L.prefill_attention(q, kv, table, c, G)
    for t in range(l):
        o_dec = L.decode_attention(q[t:t + 1], kv, table[None], np.array([c + t]), 1)
        assert np.allclose(o_dec[0], o_pre[t], atol=1e-12)


def test_append_rounds_to_storage_and_roundtrips():
    r = _rng(9)
    S, d = 16, 8
    pool = ArrayPool(np.full((3, 2, S * d), 0x7FC0, dtype=np.uint16))
    kv = L.PagedKV(pool, "bf16", S, d)
    table = np.array([2, 0], dtype=np.int32)
    k = r.standard_normal(d); v = r.standard_normal(d)
    kv.write(table, 17, k, v)
    page = kv.stored_page(0)
    K = k_slots(page[0], S, d, "bf16"); V = page[1].reshape(d, S)
    ref_k = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref_v = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(K[1], ref_k) and np.array_equal(V[:, 1], ref_v)
    assert np.all(K[0] == 0x7FC0) and np.all(K[2:] == 0x7FC0)      # other slots untouched
    assert np.array_equal(kv.stored_page(2), pool.array[2])          # page 2 untouched
    Kr, Vr = kv.read(table, 18)
    assert np.array_equal(encode(Kr[17], "bf16"), ref_k)
