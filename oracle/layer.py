"""fp64 oracle of one GPU's share of a Conflux Parallelism layer (test infrastructure).

The method reaches exactly the plain per-row result of a pre-norm decoder
layer: dense operators apply the same weights to every token independently, so
co-batching the rank-local [prefill-chunk || decode] rows changes nothing per
row (ConfluxServe §4 and App. B, Table 7), and head-sharded (Ulysses) prefill
attention computes complete attention for each head it owns (ConfluxServe
App. A; Adaptive Context Parallelism §2.1: the result equals single-rank
causal attention).  So this module is that definition written out, in fp64,
with rounding only where the layer stores state in the workload's type: the
K/V it appends to the paged pool.

Readings of points the pages leave open:

* Block structure: two RMSNorms, two residual adds, no biases, SwiGLU FFN
  down(silu(gate) * up); no QK-norm.  Gains are inputs; eps is an input.
* RoPE: rotate-half pairing (i, i + d/2), theta_i = base^(-2i/d), positions are
  absolute; cached K is stored already rotated.
* Softmax scale 1/sqrt(d); causal mask inclusive (key j visible to the query at
  position i iff j <= i).
* A decode request with context c has c cached tokens; its new token sits at
  position c, is appended first and then attends c + 1 keys (Decode Token
  Parallelism §4.3: rotary embedding, append, then attention).
* GQA: q head h reads kv head floor(h / G); the SP rank r owns q heads
  [r*Hq/P, (r+1)*Hq/P) and kv heads [r*Hkv/P, (r+1)*Hkv/P).
* Local chunk rows are chunk rows [off, off + n_local); the other chunk rows
  arrive as the stand-in ``peer_qkv_in`` (already rotated, rank's heads only),
  and the local rows' other-head attention outputs as ``peer_attn_in``.
"""
from __future__ import annotations

import numpy as np

from .numerics import encode, round_f64, to_f64

__all__ = [
    "rmsnorm", "rope", "silu", "attend", "PagedKV", "decode_attention",
    "prefill_attention", "layer_forward", "layer_forward_chunks", "stack_forward", "causal_pair_count",
]


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma (pre-norm reading)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gamma


def rope(v: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE of v[n, heads, d] at absolute positions pos[n] (Decode Token
    Parallelism §4.3 applies it to the new token before the append)."""
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    half = d // 2
    theta = float(base) ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None, None] * theta[None, None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, mask: np.ndarray | None = None):
    """softmax(q K^T / sqrt(d) + M) V for q[nq, d], K/V[nk, d]; mask[nq, nk] True = visible
    (Adaptive Context Parallelism §2.1).  Returns (o[nq, d], p[nq, nk])."""
    d = q.shape[-1]
    s = (q @ K.T) / np.sqrt(d)
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=-1, keepdims=True)
    return p @ V, p


def causal_pair_count(chunk_len: int, prior_len: int) -> int:
    """Number of visible (query, key) pairs of a chunk of chunk_len queries after prior_len
    cached keys, counted from the mask the oracle applies."""
    t = np.arange(chunk_len)
    return int(np.sum(prior_len + t + 1))


def _k_chunk(dtype: str) -> int:
    """Elements of the storage type in one 16-byte chunk of the stored K plane."""
    return 8 if dtype == "bf16" else 4


class PagedKV:
    """Logical K/V view of the paged pool (ConfluxServe §4 KV residency; §7 KV-cache aliasing:
    one physical pool, a decode-local table and a head-sharded prefill table).

    ``pool[ids]`` returns stored rows [n, 2, S*d] in the C ABI's page format: plane 0 is K
    in 16-byte chunks of consecutive dims, chunk-major over the S slots ([d/E, S, E] with E
    the elements of 16 bytes: 8 bf16 or 4 fp32), plane 1 is V dim-major [d, S].  Writes (the appends of this step) are rounded to the storage
    type and kept in an overlay; the base pool is never modified.
    """

    def __init__(self, pool, dtype: str, page_size: int, head_dim: int):
        if head_dim % _k_chunk(dtype):
            raise ValueError(f"head_dim {head_dim} is not a whole number of 16-byte K chunks")
        self.pool = pool
        self.dtype = dtype
        self.S = page_size
        self.d = head_dim
        self.overlay: dict[int, tuple[np.ndarray, np.ndarray]] = {}

    def _load(self, ids: np.ndarray):
        S, d = self.S, self.d
        rows = to_f64(self.pool[np.asarray(ids, dtype=np.int64)], self.dtype)
        E = _k_chunk(self.dtype)
        K = rows[:, 0].reshape(len(ids), d // E, S, E).transpose(0, 2, 1, 3).reshape(len(ids), S, d).copy()
        V = rows[:, 1].reshape(len(ids), d, S).transpose(0, 2, 1).copy()
        for k, p in enumerate(ids):
            ov = self.overlay.get(int(p))
            if ov is not None:
                K[k], V[k] = ov
        return K, V

    def read(self, table_row: np.ndarray, n_pos: int):
        """K, V [n_pos, d] of positions 0..n_pos-1 through one block table row."""
        nb = -(-n_pos // self.S)
        ids = np.asarray(table_row[:nb], dtype=np.int64)
        if (ids < 0).any():
            raise IndexError("block table entry -1 inside the visible range")
        K, V = self._load(ids)
        return K.reshape(nb * self.S, self.d)[:n_pos], V.reshape(nb * self.S, self.d)[:n_pos]

    def write(self, table_row: np.ndarray, pos: int, k: np.ndarray, v: np.ndarray):
        """Append K/V of one token at absolute position pos (rounded to the storage type)."""
        p = int(table_row[pos // self.S])
        if p < 0:
            raise IndexError("append into a block table entry -1")
        if p not in self.overlay:
            K, V = self._load(np.array([p]))
            self.overlay[p] = (K[0], V[0])
        K, V = self.overlay[p]
        K[pos % self.S] = round_f64(k, self.dtype)
        V[pos % self.S] = round_f64(v, self.dtype)

    def stored_page(self, p: int) -> np.ndarray:
        """Page p in the storage format after this step's appends."""
        if int(p) not in self.overlay:
            return np.asarray(self.pool[np.array([p])])[0]
        K, V = self.overlay[int(p)]
        E = _k_chunk(self.dtype)
        k_plane = K.reshape(self.S, self.d // E, E).transpose(1, 0, 2).reshape(-1)
        return np.stack([encode(k_plane, self.dtype), encode(V.T.reshape(-1), self.dtype)])


def decode_attention(q: np.ndarray, kv: PagedKV, dec_pages: np.ndarray, dec_ctx: np.ndarray,
                     n_kv_heads: int, requests=None) -> np.ndarray:
    """Paged GQA decode attention (ConfluxServe §4: decode attention stays rank-local; each
    request reads only its own KV).  q[n_d, Hq, d] -> o[n_d, Hq, d]; request i attends the
    dec_ctx[i] + 1 keys at positions 0..dec_ctx[i]."""
    n_d, Hq, d = q.shape
    G = Hq // n_kv_heads
    o = np.full((n_d, Hq, d), np.nan)
    for i in (range(n_d) if requests is None else requests):
        n = int(dec_ctx[i]) + 1
        for g in range(n_kv_heads):
            K, V = kv.read(dec_pages[i, g], n)
            o[i, g * G:(g + 1) * G], _ = attend(q[i, g * G:(g + 1) * G], K, V)
    return o


def prefill_attention(q: np.ndarray, kv: PagedKV, pre_pages: np.ndarray, prior_len: int,
                      group: int, rows=None, block: int = 256) -> np.ndarray:
    """Causal chunked-prefill attention on one SP rank's head subset over the cached prior
    keys plus the chunk (ConfluxServe §4 and App. A: chunks reuse the head-sharded history;
    Adaptive Context Parallelism §2.1 for the mask).  q[l, hq_loc, d] -> o[l, hq_loc, d];
    chunk row t (position prior_len + t) sees keys 0..prior_len + t."""
    l, hq_loc, d = q.shape
    hkv_loc = hq_loc // group
    o = np.full((l, hq_loc, d), np.nan)
    rows = np.arange(l) if rows is None else np.asarray(sorted(rows), dtype=np.int64)
    if len(rows) == 0:
        return o
    n_keys = prior_len + int(rows.max()) + 1
    for g in range(hkv_loc):
        K, V = kv.read(pre_pages[g], n_keys)
        for b0 in range(0, len(rows), block):
            rb = rows[b0:b0 + block]
            nk = prior_len + int(rb.max()) + 1
            mask = np.arange(nk)[None, :] <= (prior_len + rb)[:, None]
            for h in range(g * group, (g + 1) * group):
                o[rb, h], _ = attend(q[rb, h], K[:nk], V[:nk], mask)
    return o


def layer_forward(*, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, page_size, rms_eps,
                  rope_base, dtype, x, weights, dec_ctx, dec_pages, chunk_len, prior_len,
                  sp_degree, sp_rank, n_prefill_local, local_row_offset, pre_pages,
                  peer_qkv_in, peer_attn_in, pool, rows=None, peer_rows=None, x_dtype=None) -> dict:
    """One layer step on one GPU, rows ordered [prefill-local || decode].

    Steps (ConfluxServe §4, Fig. 7: co-batched QKV, split attention, co-batched O-proj and
    FFN; Decode Token Parallelism §4.3 for the order inside the step):
      1. hn = RMSNorm(x) * g_attn;  [q | k | v] = hn W_qkv^T (head-major columns)
      2. RoPE on q, k at absolute positions; append K/V to the pages
         (decode: all kv heads; chunk: the rank's kv heads, local rows + peer rows)
      3. decode attention (all heads) and prefill attention (rank's heads)
      4. attn rows = decode || local prefill (own heads from 3, other heads from peer_attn_in)
      5. h1 = x + attn W_o^T;  a = silu(RMSNorm(h1) W_gate^T) * (RMSNorm(h1) W_up^T)
      6. out = h1 + a W_down^T
    ``rows`` limits steps 3-6 to a subset of output rows; ``peer_rows`` limits the exported
    peer attention rows.  Everything else is computed in full.  ``x`` is in the workload's
    storage format, or in ``x_dtype``'s ("f32": a stack's residual stream).
    """
    H, Hq, Hkv, d, S = hidden, n_q_heads, n_kv_heads, head_dim, page_size
    G = Hq // Hkv
    P, r = sp_degree, sp_rank
    hq_loc, hkv_loc = Hq // P, Hkv // P
    n_pl, off, l, c = n_prefill_local, local_row_offset, chunk_len, prior_len
    n_d = len(dec_ctx)
    M = n_pl + n_d
    W = {k: to_f64(v, dtype) for k, v in weights.items()}
    x64 = to_f64(x, x_dtype or dtype).reshape(M, H)
    kv = PagedKV(pool, dtype, S, d)

    # 1. norm + co-batched QKV projection over all M rows
    hn = rmsnorm(x64, W["g_attn"], rms_eps)
    qkv = hn @ W["w_qkv"].T
    q = qkv[:, :Hq * d].reshape(M, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(M, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(M, Hkv, d)

    # 2. RoPE at absolute positions, then the appends
    pos = np.concatenate([c + off + np.arange(n_pl), np.asarray(dec_ctx, dtype=np.int64)])
    q = rope(q, pos, rope_base)
    k = rope(k, pos, rope_base)
    for i in range(n_d):
        for g in range(Hkv):
            kv.write(dec_pages[i, g], int(dec_ctx[i]), k[n_pl + i, g], v[n_pl + i, g])

    own_q = np.arange(r * hq_loc, (r + 1) * hq_loc)
    own_kv = np.arange(r * hkv_loc, (r + 1) * hkv_loc)
    other_q = np.setdiff1d(np.arange(Hq), own_q)
    other_kv = np.setdiff1d(np.arange(Hkv), own_kv)
    peer = to_f64(peer_qkv_in, dtype).reshape(l - n_pl, (hq_loc + 2 * hkv_loc) * d) if l else None
    peer_chunk_rows = [t for t in range(l) if not (off <= t < off + n_pl)]
    q_pre = np.zeros((l, hq_loc, d))
    for t in range(l):
        if off <= t < off + n_pl:
            m = t - off
            q_pre[t] = q[m, own_q]
            kt, vt = k[m, own_kv], v[m, own_kv]
        else:
            pr = peer[_peer_index(t, off, n_pl)]
            q_pre[t] = pr[:hq_loc * d].reshape(hq_loc, d)
            kt = pr[hq_loc * d:(hq_loc + hkv_loc) * d].reshape(hkv_loc, d)
            vt = pr[(hq_loc + hkv_loc) * d:].reshape(hkv_loc, d)
        for gl in range(hkv_loc):
            kv.write(pre_pages[gl], c + t, kt[gl], vt[gl])

    # exported Q/K/V of the local rows on the heads other ranks own (stand-in for All-to-All #1)
    peer_qkv_out = np.concatenate([q[:n_pl][:, other_q].reshape(n_pl, len(other_q) * d),
                                   k[:n_pl][:, other_kv].reshape(n_pl, len(other_kv) * d),
                                   v[:n_pl][:, other_kv].reshape(n_pl, len(other_kv) * d)], axis=1)

    # 3. split attention
    rows = np.arange(M) if rows is None else np.asarray(sorted(set(int(i) for i in rows)), dtype=np.int64)
    dec_req = [int(i) - n_pl for i in rows if i >= n_pl]
    loc_rows = [int(i) for i in rows if i < n_pl]
    o_dec = decode_attention(q[n_pl:], kv, dec_pages, dec_ctx, Hkv, requests=dec_req)
    all_peer = np.array(peer_chunk_rows, dtype=np.int64)
    pr_sel = all_peer if peer_rows is None else all_peer[np.asarray(peer_rows, dtype=np.int64)]
    chunk_sel = sorted(set([off + m for m in loc_rows]) | set(int(t) for t in pr_sel))
    o_pre = prefill_attention(q_pre, kv, pre_pages, c, G, rows=chunk_sel) if l else np.zeros((0, hq_loc, d))

    # 4. reconverge: attention rows in [prefill-local || decode] order
    attn = np.full((M, Hq * d), np.nan)
    pa_in = to_f64(peer_attn_in, dtype).reshape(n_pl, (Hq - hq_loc) * d) if n_pl else None
    for m in loc_rows:
        a = np.empty((Hq, d))
        a[own_q] = o_pre[off + m]
        a[other_q] = pa_in[m].reshape(Hq - hq_loc, d)
        attn[m] = a.reshape(-1)
    for i in dec_req:
        attn[n_pl + i] = o_dec[i].reshape(-1)
    peer_attn_out = np.full((l - n_pl, hq_loc * d), np.nan)
    for t in pr_sel:
        peer_attn_out[_peer_index(int(t), off, n_pl)] = o_pre[t].reshape(-1)

    # 5-6. co-batched O-proj, FFN, residuals (only the requested rows)
    h1 = np.full((M, H), np.nan)
    act = np.full((M, ffn_dim), np.nan)
    out = np.full((M, H), np.nan)
    if len(rows):
        h1[rows] = x64[rows] + attn[rows] @ W["w_o"].T
        hn2 = rmsnorm(h1[rows], W["g_ffn"], rms_eps)
        act[rows] = silu(hn2 @ W["w_gate"].T) * (hn2 @ W["w_up"].T)
        out[rows] = h1[rows] + act[rows] @ W["w_down"].T
    return dict(out=out, h1=h1, act=act, attn=attn, q=q, k=k, v=v, q_pre=q_pre, positions=pos,
                peer_qkv_out=peer_qkv_out, peer_attn_out=peer_attn_out, kv=kv, rows=rows)


def layer_forward_chunks(*, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, page_size, rms_eps, rope_base,
                         dtype, x, weights, dec_ctx, dec_pages, chunks, pool, rows=None) -> dict:
    """One layer step whose prefill side is a set of chunks (ConfluxServe §6.2 Eq. 6 and §6.4:
    the scheduled prefills P are several requests' chunks), sp_degree 1.

    ``chunks`` is a list of (chunk_len, prior_len, table[Hkv, blocks]); rows are ordered
    [chunk 0 || chunk 1 || ... || decode].  Chunk j's row t is at position prior_j + t, its
    K/V go to every kv head through its own table, and it attends keys 0..prior_j + t of
    its own request.  Everything else is the step of ``layer_forward``.
    """
    H, Hq, Hkv, d = hidden, n_q_heads, n_kv_heads, head_dim
    G = Hq // Hkv
    n_d = len(dec_ctx)
    starts = np.cumsum([0] + [l for l, _, _ in chunks])
    n_pre = int(starts[-1])
    M = n_pre + n_d
    W = {k: to_f64(v, dtype) for k, v in weights.items()}
    x64 = to_f64(x, dtype).reshape(M, H)
    kv = PagedKV(pool, dtype, page_size, d)

    # co-batched norm + QKV over every row
    hn = rmsnorm(x64, W["g_attn"], rms_eps)
    qkv = hn @ W["w_qkv"].T
    q = qkv[:, :Hq * d].reshape(M, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(M, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(M, Hkv, d)

    # RoPE at absolute positions, then the appends
    pos = np.concatenate([c + np.arange(l) for l, c, _ in chunks] + [np.asarray(dec_ctx, dtype=np.int64)])
    q = rope(q, pos, rope_base)
    k = rope(k, pos, rope_base)
    for i in range(n_d):
        for g in range(Hkv):
            kv.write(dec_pages[i, g], int(dec_ctx[i]), k[n_pre + i, g], v[n_pre + i, g])
    for j, (l, c, table) in enumerate(chunks):
        for t in range(l):
            for g in range(Hkv):
                kv.write(table[g], c + t, k[starts[j] + t, g], v[starts[j] + t, g])

    # split attention: decodes, then each chunk over its own request's keys
    rows = np.arange(M) if rows is None else np.asarray(sorted(set(int(i) for i in rows)), dtype=np.int64)
    attn = np.full((M, Hq * d), np.nan)
    dec_req = [int(i) - n_pre for i in rows if i >= n_pre]
    o_dec = decode_attention(q[n_pre:], kv, dec_pages, dec_ctx, Hkv, requests=dec_req)
    for i in dec_req:
        attn[n_pre + i] = o_dec[i].reshape(-1)
    for j, (l, c, table) in enumerate(chunks):
        sel = [int(i) - int(starts[j]) for i in rows if starts[j] <= i < starts[j + 1]]
        if not sel:
            continue
        o = prefill_attention(q[starts[j]:starts[j + 1]], kv, table, c, G, rows=sel)
        for t in sel:
            attn[starts[j] + t] = o[t].reshape(-1)

    # co-batched O-proj, FFN and residuals on the requested rows
    h1 = np.full((M, H), np.nan)
    act = np.full((M, ffn_dim), np.nan)
    out = np.full((M, H), np.nan)
    if len(rows):
        h1[rows] = x64[rows] + attn[rows] @ W["w_o"].T
        hn2 = rmsnorm(h1[rows], W["g_ffn"], rms_eps)
        act[rows] = silu(hn2 @ W["w_gate"].T) * (hn2 @ W["w_up"].T)
        out[rows] = h1[rows] + act[rows] @ W["w_down"].T
    return dict(out=out, h1=h1, act=act, attn=attn, q=q, k=k, v=v, positions=pos, kv=kv, rows=rows)


def stack_forward(*, layers, x, dtype, **step) -> dict:
    """A stack of layer steps over one batch (ConfluxServe §4 Fig. 7 layer after layer),
    sp_degree 1.  ``layers``: per layer {"weights", "pool"}; every other argument is
    layer_forward's and serves every layer (tables, contexts, positions).  Layer 0 reads
    ``x`` in the workload's format; layer l > 0 reads layer l-1's output stored as
    float32 (the residual stream between layers is kept in fp32), so the only rounding
    between layers is that store.  Returns the last layer's output and every layer's
    result."""
    results = []
    cur, cur_dtype = x, None
    for layer in layers:
        r = layer_forward(x=cur, dtype=dtype, weights=layer["weights"], pool=layer["pool"], x_dtype=cur_dtype, **step)
        results.append(r)
        cur, cur_dtype = r["out"].astype(np.float32), "f32"
    return dict(out=results[-1]["out"], layers=results)


def _peer_index(t: int, off: int, n_pl: int) -> int:
    """Index of chunk row t among the peer rows (chunk rows in order, local block removed)."""
    return t if t < off else t - n_pl
