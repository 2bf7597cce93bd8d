"""Pure-Python loop formulation of a tiny layer step (test infrastructure).

A second, deliberately different formulation used only to pin ``oracle.layer``
on tiny inputs: scalar loops, ``math``/``cmath`` only, RoPE as multiplication
of (v_i + i*v_{i+d/2}) by exp(i*pos*theta_i), the pool read slot by slot.  It
covers the P = 1 case (no SP stand-in buffers).
"""
from __future__ import annotations

import cmath
import math

__all__ = ["read_stored", "brute_rmsnorm", "brute_rope", "brute_attention", "brute_layer"]


def read_stored(bits_or_float, dtype):
    """Scalar value of one stored element."""
    if dtype == "f32":
        return float(bits_or_float)
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits_or_float) << 16))[0]


def brute_rmsnorm(row, gamma, eps):
    ms = sum(v * v for v in row) / len(row)
    inv = 1.0 / math.sqrt(ms + eps)
    return [v * inv * g for v, g in zip(row, gamma)]


def brute_rope(vec, pos, base):
    d = len(vec)
    half = d // 2
    out = [0.0] * d
    for i in range(half):
        z = complex(vec[i], vec[i + half]) * cmath.exp(1j * pos * base ** (-2.0 * i / d))
        out[i], out[i + half] = z.real, z.imag
    return out


def brute_attention(q, keys, values):
    """One query over an explicit list of visible keys."""
    d = len(q)
    scores = [sum(a * b for a, b in zip(q, k)) / math.sqrt(d) for k in keys]
    mx = max(scores)
    w = [math.exp(s - mx) for s in scores]
    tot = sum(w)
    return [sum(w[j] * values[j][t] for j in range(len(keys))) / tot for t in range(d)]


def _matvec(W, x):
    """W given as rows [out][in]."""
    return [sum(a * b for a, b in zip(row, x)) for row in W]


def _read_page_slot(pool, page, slot, S, d, dtype):
    row = pool[[page]][0]
    E = 8 if dtype == "bf16" else 4          # elements per 16-byte chunk of the K plane
    k = [read_stored(row[0][((j // E) * S + slot) * E + j % E], dtype) for j in range(d)]
    v = [read_stored(row[1][j * S + slot], dtype) for j in range(d)]
    return k, v


def brute_layer(*, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, page_size, rms_eps, rope_base,
                dtype, x, weights, dec_ctx, dec_pages, chunk_len, prior_len, pre_pages, pool):
    """Tiny P = 1 layer step, row by row: returns out rows as lists (rows = [chunk || decode]).

    Appended K/V are rounded to the storage type through float32 (exact for f32 workloads;
    for bf16 workloads a caller compares with a tolerance)."""
    H, Hq, Hkv, d, S = hidden, n_q_heads, n_kv_heads, head_dim, page_size
    G = Hq // Hkv
    W = {k: [[read_stored(e, dtype) for e in row] for row in (v if v.ndim == 2 else [v])]
         for k, v in weights.items()}
    g_attn, g_ffn = W["g_attn"][0], W["g_ffn"][0]
    M = chunk_len + len(dec_ctx)
    X = [[read_stored(e, dtype) for e in x[m]] for m in range(M)]

    def project(m):
        hn = brute_rmsnorm(X[m], g_attn, rms_eps)
        qkv = _matvec(W["w_qkv"], hn)
        q = [qkv[h * d:(h + 1) * d] for h in range(Hq)]
        k = [qkv[(Hq + g) * d:(Hq + g + 1) * d] for g in range(Hkv)]
        v = [qkv[(Hq + Hkv + g) * d:(Hq + Hkv + g + 1) * d] for g in range(Hkv)]
        return q, k, v

    def store(val):
        import struct
        f = struct.unpack("<f", struct.pack("<f", val))[0]
        if dtype == "f32":
            return f
        raise NotImplementedError("brute_layer rounds only to f32")

    attn_rows = []
    chunk_k = [[None] * chunk_len for _ in range(Hkv)]
    chunk_v = [[None] * chunk_len for _ in range(Hkv)]
    chunk_q = []
    for t in range(chunk_len):
        q, k, v = project(t)
        pos = prior_len + t
        chunk_q.append([brute_rope(qh, pos, rope_base) for qh in q])
        for g in range(Hkv):
            chunk_k[g][t] = [store(e) for e in brute_rope(k[g], pos, rope_base)]
            chunk_v[g][t] = [store(e) for e in v[g]]
    prior = {}
    for g in range(Hkv):
        ks, vs = [], []
        for p in range(prior_len):
            kk, vv = _read_page_slot(pool, int(pre_pages[g][p // S]), p % S, S, d, dtype)
            ks.append(kk); vs.append(vv)
        prior[g] = (ks, vs)
    for t in range(chunk_len):
        row = []
        for h in range(Hq):
            g = h // G
            keys = prior[g][0] + chunk_k[g][:t + 1]
            vals = prior[g][1] + chunk_v[g][:t + 1]
            row += brute_attention(chunk_q[t][h], keys, vals)
        attn_rows.append(row)
    for i, c in enumerate(dec_ctx):
        m = chunk_len + i
        q, k, v = project(m)
        c = int(c)
        row = []
        for h in range(Hq):
            g = h // G
            keys, vals = [], []
            for p in range(c):
                kk, vv = _read_page_slot(pool, int(dec_pages[i][g][p // S]), p % S, S, d, dtype)
                keys.append(kk); vals.append(vv)
            keys.append([store(e) for e in brute_rope(k[g], c, rope_base)])
            vals.append([store(e) for e in v[g]])
            row += brute_attention(brute_rope(q[h], c, rope_base), keys, vals)
        attn_rows.append(row)
    outs = []
    for m in range(M):
        h1 = [a + b for a, b in zip(X[m], _matvec(W["w_o"], attn_rows[m]))]
        hn2 = brute_rmsnorm(h1, g_ffn, rms_eps)
        gate = _matvec(W["w_gate"], hn2)
        up = _matvec(W["w_up"], hn2)
        act = [(z / (1.0 + math.exp(-z))) * u for z, u in zip(gate, up)]
        outs.append([a + b for a, b in zip(h1, _matvec(W["w_down"], act))])
    return outs
