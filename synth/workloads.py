"""Seeded synthetic workloads for one GPU's share of a Conflux Parallelism layer.

Every tensor ``t`` of workload ``k`` is drawn from
``numpy.random.Generator(PCG64(SeedSequence([k, TENSOR_IDS[t]])))`` with
``standard_normal(dtype=float32)``, scaled in float32 and rounded
round-to-nearest-even to the workload's storage type (bf16 bit patterns held as
``uint16``, or float32).  Page tables are a seeded permutation of the pool.

Storage formats (these are the formats the C ABI consumes):

* activations / weights: row-major; weights are ``[out_features, in_features]``
  so a projection is ``y = x @ W.T``.
* KV pool: ``[n_pages, 2, page_size * head_dim]``.  Plane 0 holds K in 16-byte
  chunks of consecutive dims, chunk-major over the slots (with ``E`` elements per
  chunk, 8 for bf16 and 4 for float32, element ``((j // E) * page_size + s) * E +
  j % E`` is slot ``s``, dim ``j``); plane 1 holds V dim-major (element
  ``j * page_size + s``).  One page holds one KV head of one request.
* decode page table ``[n_decode, n_kv_heads, dec_max_blocks]`` int32 and prefill
  page table ``[n_kv_heads / sp_degree, pre_max_blocks]`` int32; block ``b``
  covers positions ``[b * page_size, (b + 1) * page_size)``; unused entries -1.

Slots that hold no valid cached token before the layer runs (including the
slots the layer itself appends to) are filled with NaN, so a kernel that reads
a slot it must not read, or skips an append, produces NaN.

Nothing here computes any part of the layer or of the dispatcher.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "TENSOR_IDS", "Workload", "Instance", "PagePool", "WaterfillCase",
    "WORKLOADS", "PARITY_WORKLOADS", "get_workload", "make_instance",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "storage_to_f64",
    "waterfill_cases", "make_latency_model", "SchedulerCase", "scheduler_case",
    "MultiChunkWorkload", "MultiChunkInstance", "make_multi_instance", "MULTI_CHUNK_WORKLOADS",
    "StackInstance", "make_stack_instance", "save_instance", "load_instance",
]

TENSOR_IDS = {
    "x": 0, "w_qkv": 1, "w_o": 2, "w_gate": 3, "w_up": 4, "w_down": 5,
    "kv": 6, "peer_qkv_in": 7, "peer_attn_in": 8, "dec_ctx": 9,
    "page_perm": 10, "kv_bank_idx": 11, "extra": 12, "sched_state": 13, "sched_queue": 14,
}

# Fixed draw granularity for the KV pool, so the drawn sequence is defined.
_KV_DRAW_PAGES = 1024


def _rng(seed_id: int, tensor: str, layer: int = 0) -> np.random.Generator:
    """Generator of one tensor; layer l > 0 of a stack draws its own (layer 0 is the
    single-layer draw)."""
    key = [seed_id, TENSOR_IDS[tensor]] + ([layer] if layer else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (NaN -> quiet NaN)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact value of a stored array as float64 (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _normal(seed_id: int, tensor: str, shape, scale: float, dtype: str, layer: int = 0) -> np.ndarray:
    v = _rng(seed_id, tensor, layer).standard_normal(size=int(np.prod(shape)), dtype=np.float32)
    if scale != 1.0:
        v *= np.float32(scale)
    v = v.reshape(shape)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


@dataclass(frozen=True)
class Workload:
    """One layer step on one GPU: shape, decode population and prefill chunk."""
    name: str
    seed_id: int
    dtype: str                      # "bf16" or "f32" (storage and operand type)
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    n_decode: int
    ctx: tuple                      # ("fixed", c) | ("uniform", lo, hi) | ("lognormal", mu, sigma, lo, hi)
    chunk_len: int
    prior_len: int
    sp_degree: int = 1
    sp_rank: int = 0
    page_size: int = 16
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    weight_std: float = 0.02
    kv_bank_pages: int = 0          # >0: pool pages are copies of a seeded bank of this many pages
    spare_pages: int = 0            # pool pages no table references (must stay untouched)
    description: str = ""

    @property
    def n_prefill_local(self) -> int:
        return self.chunk_len // self.sp_degree

    @property
    def local_row_offset(self) -> int:
        return self.sp_rank * self.n_prefill_local

    @property
    def n_rows(self) -> int:
        return self.n_prefill_local + self.n_decode

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def hq_loc(self) -> int:
        return self.n_q_heads // self.sp_degree

    @property
    def hkv_loc(self) -> int:
        return self.n_kv_heads // self.sp_degree

    @property
    def qkv_dim(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


class PagePool:
    """KV pool in the ABI storage format; ``pool[ids]`` returns rows.

    Either a materialised array, or a seeded bank of pages plus a per-page bank
    index (for pools too large to draw element by element).  ``valid_slots[p]``
    is the number of leading slots of page ``p`` that hold valid cached tokens;
    the other slots read as NaN.
    """

    def __init__(self, n_pages, row_shape, dtype, valid_slots, page_size, head_dim,
                 array=None, bank=None, bank_idx=None):
        self.n_pages = int(n_pages)
        self.row_shape = tuple(row_shape)
        self.dtype = dtype
        self.valid_slots = valid_slots
        self.page_size = page_size
        self.head_dim = head_dim
        self.array = array
        self.bank = bank
        self.bank_idx = bank_idx

    @property
    def np_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    @property
    def nbytes(self) -> int:
        return self.n_pages * int(np.prod(self.row_shape)) * np.dtype(self.np_dtype).itemsize

    def poisoned_pages(self) -> np.ndarray:
        return np.nonzero(self.valid_slots < self.page_size)[0].astype(np.int64)

    def _poison(self, rows: np.ndarray, ids: np.ndarray) -> np.ndarray:
        S, d = self.page_size, self.head_dim
        nan = np.uint16(0x7FC0) if self.dtype == "bf16" else np.float32(np.nan)
        for k, p in enumerate(ids):
            v = int(self.valid_slots[p])
            if v < S:
                E = 8 if self.dtype == "bf16" else 4
                rows[k, 0].reshape(d // E, S, E)[:, v:, :] = nan
                rows[k, 1].reshape(d, S)[:, v:] = nan
        return rows

    def __getitem__(self, ids):
        ids = np.atleast_1d(np.asarray(ids, dtype=np.int64))
        if self.array is not None:
            return self.array[ids]
        rows = self.bank[self.bank_idx[ids]].copy()
        return self._poison(rows, ids)


@dataclass
class Instance:
    """Drawn inputs of one workload, in storage format."""
    wl: Workload
    x: np.ndarray
    weights: dict
    dec_ctx: np.ndarray
    dec_pages: np.ndarray
    pre_pages: np.ndarray
    pool: PagePool
    peer_qkv_in: np.ndarray
    peer_attn_in: np.ndarray
    extra: dict = field(default_factory=dict)

    @property
    def dec_max_blocks(self) -> int:
        return int(self.dec_pages.shape[2]) if self.dec_pages.ndim == 3 else 0

    @property
    def pre_max_blocks(self) -> int:
        return int(self.pre_pages.shape[1]) if self.pre_pages.ndim == 2 else 0


def _draw_ctx(wl: Workload) -> np.ndarray:
    kind = wl.ctx[0]
    n = wl.n_decode
    if n == 0:
        return np.zeros(0, dtype=np.int32)
    if kind == "fixed":
        return np.full(n, int(wl.ctx[1]), dtype=np.int32)
    r = _rng(wl.seed_id, "dec_ctx")
    if kind == "uniform":
        return r.integers(int(wl.ctx[1]), int(wl.ctx[2]) + 1, size=n).astype(np.int32)
    if kind == "lognormal":
        mu, sigma, lo, hi = wl.ctx[1:]
        v = np.rint(r.lognormal(mu, sigma, size=n))
        return np.clip(v, lo, hi).astype(np.int32)
    if kind == "list":
        return np.asarray(wl.ctx[1], dtype=np.int32)
    raise ValueError(kind)


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def make_instance(wl: Workload, materialize_limit_bytes: int = 4 << 30) -> Instance:
    S, d, H = wl.page_size, wl.head_dim, wl.hidden
    Hq, Hkv, F = wl.n_q_heads, wl.n_kv_heads, wl.ffn_dim
    assert Hq % Hkv == 0 and Hq % wl.sp_degree == 0 and Hkv % wl.sp_degree == 0
    assert wl.chunk_len % wl.sp_degree == 0
    k = wl.seed_id
    dt = wl.dtype
    M = wl.n_rows

    x = _normal(k, "x", (M, H), 1.0, dt)
    ws = wl.weight_std
    weights = {
        "w_qkv": _normal(k, "w_qkv", (wl.qkv_dim, H), ws, dt),
        "w_o": _normal(k, "w_o", (H, Hq * d), ws, dt),
        "w_gate": _normal(k, "w_gate", (F, H), ws, dt),
        "w_up": _normal(k, "w_up", (F, H), ws, dt),
        "w_down": _normal(k, "w_down", (H, F), ws, dt),
    }
    one = f32_to_bf16_bits(np.ones(H, np.float32)) if dt == "bf16" else np.ones(H, np.float32)
    weights["g_attn"] = one.copy()
    weights["g_ffn"] = one.copy()

    ctx = _draw_ctx(wl)
    nb_dec = [_cdiv(int(c) + 1, S) for c in ctx]
    nb_pre = _cdiv(wl.prior_len + wl.chunk_len, S) if wl.chunk_len > 0 else 0
    n_used = sum(nb_dec) * Hkv + nb_pre * wl.hkv_loc
    n_pages = n_used + wl.spare_pages
    perm = _rng(k, "page_perm").permutation(n_pages).astype(np.int32)

    dec_max = max(nb_dec) if nb_dec else 0
    dec_pages = np.full((wl.n_decode, Hkv, max(dec_max, 1)), -1, dtype=np.int32)
    pre_pages = np.full((wl.hkv_loc, max(nb_pre, 1)), -1, dtype=np.int32)
    valid = np.full(n_pages, S, dtype=np.int32)
    it = 0
    for i, c in enumerate(ctx):
        for g in range(Hkv):
            for b in range(nb_dec[i]):
                p = int(perm[it]); it += 1
                dec_pages[i, g, b] = p
                valid[p] = min(max(int(c) - b * S, 0), S)
    for g in range(wl.hkv_loc):
        for b in range(nb_pre):
            p = int(perm[it]); it += 1
            pre_pages[g, b] = p
            valid[p] = min(max(wl.prior_len - b * S, 0), S)
    # spare pages keep valid = S (random content, never referenced)

    row_shape = (2, S * d)
    np_dt = np.uint16 if dt == "bf16" else np.float32
    if wl.kv_bank_pages > 0:
        nb = wl.kv_bank_pages
        bank = _draw_pages(k, "kv", nb, row_shape, dt)
        bank_idx = _rng(k, "kv_bank_idx").integers(0, nb, size=n_pages).astype(np.int64)
        pool = PagePool(n_pages, row_shape, dt, valid, S, d, bank=bank, bank_idx=bank_idx)
    else:
        nbytes = n_pages * 2 * S * d * np.dtype(np_dt).itemsize
        if nbytes > materialize_limit_bytes:
            raise ValueError(f"{wl.name}: pool of {nbytes / 2**30:.1f} GiB; set kv_bank_pages")
        arr = _draw_pages(k, "kv", n_pages, row_shape, dt)
        pool = PagePool(n_pages, row_shape, dt, valid, S, d, array=arr)
        ids = pool.poisoned_pages()
        if len(ids):
            arr[ids] = pool._poison(arr[ids].copy(), ids)

    n_peer_rows = wl.chunk_len - wl.n_prefill_local
    peer_qkv_in = _normal(k, "peer_qkv_in", (n_peer_rows, (wl.hq_loc + 2 * wl.hkv_loc) * d), 1.0, dt)
    peer_attn_in = _normal(k, "peer_attn_in", (wl.n_prefill_local, (Hq - wl.hq_loc) * d), 1.0, dt)
    return Instance(wl, x, weights, ctx, dec_pages, pre_pages, pool, peer_qkv_in, peer_attn_in)


def _draw_pages(seed_id, tensor, n_pages, row_shape, dt, layer=0):
    r = _rng(seed_id, tensor, layer)
    per = int(np.prod(row_shape))
    out = np.empty((n_pages,) + tuple(row_shape), dtype=np.uint16 if dt == "bf16" else np.float32)
    flat = out.reshape(n_pages, per)
    for p0 in range(0, n_pages, _KV_DRAW_PAGES):
        p1 = min(n_pages, p0 + _KV_DRAW_PAGES)
        v = r.standard_normal(size=(p1 - p0) * per, dtype=np.float32).reshape(p1 - p0, per)
        flat[p0:p1] = f32_to_bf16_bits(v) if dt == "bf16" else v
    return out


# ---------------------------------------------------------------------------
# The workloads.  C1..C5 are the layer shapes the measurements are quoted on;
# "-full" are the whole-prompt-as-one-chunk readings of C3 and C5; P*/E* are
# small parity and edge-case workloads the oracle finishes in seconds.
# ---------------------------------------------------------------------------

_LN_MU = math.log(6346.0)
_LN_SIGMA = math.log(26114.0 / 6346.0) / 1.6448536269514722

WORKLOADS = {
    "C1": Workload("C1", 1, "f32", 256, 4, 2, 64, 512, n_decode=4, ctx=("uniform", 1, 256),
                   chunk_len=64, prior_len=128,
                   description="tiny fp32 layer: 64-token chunk after 128 cached, 4 decodes"),
    "C2": Workload("C2", 2, "bf16", 4096, 32, 8, 128, 14336, n_decode=16, ctx=("fixed", 8192),
                   chunk_len=1024, prior_len=0,
                   description="Llama-3.1-8B layer: 16 decodes at 8192 + 1024-token chunk"),
    "C3": Workload("C3", 3, "bf16", 5120, 40, 8, 128, 17408, n_decode=24, ctx=("fixed", 8192),
                   chunk_len=2048, prior_len=6144, sp_degree=4, sp_rank=0,
                   description="Qwen3-14B layer: 24 decodes at 8192 + SP4 share of a 2048 chunk after 6144"),
    "C3-full": Workload("C3-full", 31, "bf16", 5120, 40, 8, 128, 17408, n_decode=24, ctx=("fixed", 8192),
                        chunk_len=32768, prior_len=0, sp_degree=4, sp_rank=0,
                        description="Qwen3-14B layer: 24 decodes + SP4 share of a whole 32768 prompt"),
    "C4": Workload("C4", 4, "bf16", 4096, 32, 8, 128, 14336, n_decode=128, ctx=("fixed", 32768),
                   chunk_len=0, prior_len=0, kv_bank_pages=16384,
                   description="decode-heavy Llama-3.1-8B layer: 128 decodes at 32768, no prefill"),
    "D1": Workload("D1", 6, "bf16", 4096, 32, 8, 128, 14336, n_decode=16, ctx=("fixed", 1024),
                   chunk_len=0, prior_len=0,
                   description="small Llama-3.1-8B decode step: 16 decodes at 1024, no prefill"),
    "C5": Workload("C5", 5, "bf16", 5120, 64, 8, 128, 25600, n_decode=32,
                   ctx=("lognormal", _LN_MU, _LN_SIGMA, 1, 65536),
                   chunk_len=4096, prior_len=12288, sp_degree=8, sp_rank=0,
                   description="Qwen3-32B layer: 32 lognormal decodes + SP8 share of a 4096 chunk after 12288"),
    "C5-full": Workload("C5-full", 51, "bf16", 5120, 64, 8, 128, 25600, n_decode=32,
                        ctx=("lognormal", _LN_MU, _LN_SIGMA, 1, 65536),
                        chunk_len=65536, prior_len=0, sp_degree=8, sp_rank=0,
                        description="Qwen3-32B layer: 32 decodes + SP8 share of a whole 65536 prompt"),
}

PARITY_WORKLOADS = {
    # bf16, G=5, SP2 on rank 1 (non-zero row offset), ragged chunk/page/tile tails
    "P1": Workload("P1", 101, "bf16", 640, 10, 2, 128, 1408, n_decode=7, ctx=("uniform", 0, 700),
                   chunk_len=200, prior_len=75, sp_degree=2, sp_rank=1, spare_pages=3,
                   description="small bf16 layer, SP2 rank 1, ragged tails"),
    # bf16, G=4, P=1, chunk starting at 0, decodes of various lengths incl. ctx 0
    "P2": Workload("P2", 102, "bf16", 512, 8, 2, 128, 1024, n_decode=5, ctx=("list", [0, 1, 15, 16, 300]),
                   chunk_len=97, prior_len=0,
                   description="small bf16 layer, decode contexts at page edges"),
    # bf16, G=8 with one kv head per rank (the C5 head layout), SP8
    "P3": Workload("P3", 103, "bf16", 1024, 64, 8, 128, 2048, n_decode=3, ctx=("uniform", 100, 900),
                   chunk_len=256, prior_len=130, sp_degree=8, sp_rank=0,
                   description="small bf16 layer, 8 q heads on one kv head per rank"),
    # long prior context: many key splits per query tile (the merge path), G=8 on one kv head, rank 1
    "P4": Workload("P4", 104, "bf16", 1024, 16, 2, 128, 2048, n_decode=2, ctx=("list", [37, 2500]),
                   chunk_len=320, prior_len=2000, sp_degree=2, sp_rank=1,
                   description="small bf16 layer, 2000 prior keys, SP2 rank 1"),
    # the 8B head layout (G = 4 on 8 kv heads): grids of at most one workgroup per CU
    # whose work units span 16 or more key blocks (one wave per SIMD); ragged chunk,
    # prior not a multiple of the 32-key block
    "P5": Workload("P5", 105, "bf16", 512, 32, 8, 128, 1024, n_decode=0, ctx=("fixed", 0),
                   chunk_len=900, prior_len=300, description="prefill only, 8B heads, 900 after 300"),
    # the same with the key range split three ways (19-block units, not a multiple of
    # the pipelined loop's three-block stages) and merged
    "P6": Workload("P6", 106, "bf16", 512, 32, 8, 128, 1024, n_decode=0, ctx=("fixed", 0),
                   chunk_len=300, prior_len=1500, description="prefill only, 8B heads, 300 after 1500"),
    # long decode contexts on the 32B head layout (64 q / 8 kv heads): the shortest and
    # longest requests of the 32B decode batch (502 and 48957 cached tokens) and the 8K and
    # 32K contexts of the 8B batches, for decode-attention parity on identical inputs
    "L1": Workload("L1", 121, "bf16", 1024, 64, 8, 128, 2048, n_decode=4, ctx=("list", [502, 8192, 32768, 48957]),
                   chunk_len=0, prior_len=0, description="decode only, 32B heads, 502 / 8K / 32K / 49K contexts"),
    # decode only
    "E1": Workload("E1", 111, "bf16", 512, 8, 2, 128, 1024, n_decode=9, ctx=("uniform", 1, 2000),
                   chunk_len=0, prior_len=0, description="decode only"),
    # prefill only
    "E2": Workload("E2", 112, "bf16", 512, 8, 2, 128, 1024, n_decode=0, ctx=("fixed", 0),
                   chunk_len=130, prior_len=33, description="prefill only"),
    # single decode row, fp32
    "E3": Workload("E3", 113, "f32", 256, 4, 2, 64, 512, n_decode=1, ctx=("fixed", 40),
                   chunk_len=0, prior_len=0, description="one fp32 decode row"),
    # bf16 with d = 64 and three query heads per kv head: the pipelined prefill loop's
    # d = 64 form, ragged chunk and prior
    "P7": Workload("P7", 107, "bf16", 512, 12, 4, 64, 1024, n_decode=0, ctx=("fixed", 0),
                   chunk_len=150, prior_len=90, description="prefill only, bf16, d = 64, G = 3"),
    # twelve query heads per kv head: each kv head takes two workgroups of eight waves,
    # the second with four heads, so four of its waves only take the stage barriers
    "P8": Workload("P8", 108, "bf16", 512, 24, 2, 128, 1024, n_decode=0, ctx=("fixed", 0),
                   chunk_len=100, prior_len=300, description="prefill only, bf16, G = 12"),
    # a three-token chunk after 1000 cached tokens: one mostly empty query tile whose key
    # range is cut into splits, merged by the combine
    "P9": Workload("P9", 109, "bf16", 512, 16, 2, 128, 1024, n_decode=0, ctx=("fixed", 0),
                   chunk_len=3, prior_len=1000, description="prefill only, bf16, 3 after 1000"),
    # d = 64 on the 8B head layout (P5's grid): in bf16 the block-pipelined loop with
    # units of up to 38 key blocks; in fp32 a workgroup holds two waves per query head
    # (two key sets, 32-bit operands only)
    "P10": Workload("P10", 110, "bf16", 512, 32, 8, 64, 1024, n_decode=0, ctx=("fixed", 0),
                    chunk_len=900, prior_len=300, description="prefill only, bf16, d = 64, long units"),
    "E5": Workload("E5", 115, "f32", 512, 32, 8, 64, 1024, n_decode=0, ctx=("fixed", 0),
                   chunk_len=900, prior_len=300, description="prefill only, fp32, two key sets"),
    # fp32 with SP2
    "E4": Workload("E4", 114, "f32", 256, 4, 2, 64, 512, n_decode=3, ctx=("uniform", 0, 100),
                   chunk_len=34, prior_len=17, sp_degree=2, sp_rank=1, description="fp32, SP2 rank 1"),
}


def get_workload(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    return PARITY_WORKLOADS[name]


# ---------------------------------------------------------------------------
# Waterfill (host dispatch) inputs.
# ---------------------------------------------------------------------------

@dataclass
class WaterfillCase:
    name: str
    n_decode_tokens: list          # n_d^r per rank
    decode_ctx_sum: list           # sum of decode contexts resident on rank r
    existing_assign: list          # n_p^r(A_p) before this request
    selected: list                 # [(len, ctx)] of chunks already selected this iteration
    candidate: Optional[tuple]     # (m_remaining, c_processed) or None
    fixed_target: int              # >= 0: use as n_target; -1: search
    tbt_slo: float
    quantum: int
    level_hi: int                  # search range upper bound when no candidate (else 0 = derive)
    model: dict                    # latency-model coefficients (see make_latency_model)
    source: str = ""


def make_latency_model(gamma=2.0 ** -17, gamma0=2.0 ** -12, a_d=2.0 ** -27, a_d0=2.0 ** -13,
                       a_p=2.0 ** -31, a_p0=2.0 ** -13, a_comm=2.0 ** -20, a_comm0=2.0 ** -14,
                       alpha=1.125, beta=1.25, n_layers=64) -> dict:
    """Synthetic coefficients (dyadic, so model evaluations are exact in fp64)."""
    return dict(gamma=gamma, gamma0=gamma0, a_d=a_d, a_d0=a_d0, a_p=a_p, a_p0=a_p0,
                a_comm=a_comm, a_comm0=a_comm0, alpha=alpha, beta=beta, n_layers=n_layers)


def waterfill_cases() -> list:
    cases = []
    m0 = make_latency_model()
    # C5's dispatch exercise: 4 simulated ranks holding the 32 lognormal decodes
    # in request order with token loads 4/4/12/12; candidate = the 65536-token
    # prompt after 12288 processed tokens.
    ctx = _draw_ctx(WORKLOADS["C5"]).astype(np.int64)
    split = [4, 4, 12, 12]
    sums, o = [], 0
    for n in split:
        sums.append(int(ctx[o:o + n].sum()))
        o += n
    cases.append(WaterfillCase("C5-4rank", split, sums, [0, 0, 0, 0], [], (65536 - 12288, 12288),
                               -1, 0.100, 16, 0, m0, source="C5 decode population on 4 simulated ranks"))
    # the same with a 4096-token candidate (the C5 chunk as the remaining length)
    cases.append(WaterfillCase("C5-4rank-m4096", split, sums, [0, 0, 0, 0], [], (4096, 12288),
                               -1, 0.100, 16, 0, m0))
    # reference budget B0 (no candidate) on the same state
    cases.append(WaterfillCase("C5-4rank-B0", split, sums, [0, 0, 0, 0], [], None,
                               -1, 0.100, 16, 1 << 16, m0))
    return cases


@dataclass
class SchedulerCase:
    """Decode state of one XP instance and a pending prefill queue (host values)."""
    name: str
    n_decode_tokens: list
    decode_ctx_sum: list
    kv_used: list
    kv_capacity: list
    m_remaining: list
    c_processed: list
    deadlines: list
    now: float
    tau: float
    quantum: int
    eta: float
    headroom: int
    model: dict


# Mooncake-Toolagent prompt lengths (P50 6,346, P95 26,114 tokens), the stand-in for the
# pages' traces: lognormal with mu = ln 6346 and sigma = ln(26114 / 6346) / 1.644854.
_PROMPT_MU, _PROMPT_SIGMA = float(np.log(6346.0)), float(np.log(26114.0 / 6346.0) / 1.644854)


def scheduler_case(depth: int, n_ranks: int = 8, seed: int = 0, kv_capacity: int = 1_600_000,
                   tau: float = 0.100, quantum: int = 16, eta: float = 0.8, headroom: int = 4096) -> SchedulerCase:
    """A scheduling iteration on ``n_ranks`` ranks with ``depth`` pending prefills.

    Each rank holds 4..32 resident decodes whose contexts are drawn from the prompt
    distribution; its KV use is their sum, against ``kv_capacity`` tokens (about
    200 GB of 128 KiB-per-token KV, an 8B model on one MI355X).  Pending requests
    draw a prompt from the same distribution; a quarter already have part of it
    cached (c > 0).  They arrived in the last 2 s and their TTFT deadline is
    arrival + 0.5 s + 0.1 ms per prompt token.  The latency model has the magnitudes of
    an 8B layer on one MI355X (32 layers; about 0.5 us per shared-linear token, 1 ns per
    decode context token, 60 ps per prefill attention pair), in dyadic coefficients.
    """
    rs = _rng(seed, "sched_state")
    nd = rs.integers(4, 33, size=n_ranks)
    ctx = [np.clip(np.rint(rs.lognormal(_PROMPT_MU, _PROMPT_SIGMA, size=int(n))), 1, 65536).astype(np.int64)
           for n in nd]
    ctx_sum = [int(c.sum()) for c in ctx]
    rq = _rng(seed, "sched_queue")
    prompt = np.clip(np.rint(rq.lognormal(_PROMPT_MU, _PROMPT_SIGMA, size=depth)), 16, 65536).astype(np.int64)
    partial = rq.random(depth) < 0.25
    done = np.where(partial, np.floor(prompt * rq.uniform(0.1, 0.9, size=depth)), 0).astype(np.int64)
    now = 100.0
    arrival = now - rq.uniform(0.0, 2.0, size=depth)
    deadline = arrival + 0.5 + 1e-4 * prompt
    return SchedulerCase(f"sched-N{n_ranks}-R{depth}-s{seed}", [int(v) for v in nd], ctx_sum, list(ctx_sum),
                         [kv_capacity] * n_ranks, [int(v) for v in prompt - done], [int(v) for v in done],
                         [float(v) for v in deadline], now, tau, quantum, eta, headroom,
                         make_latency_model(gamma=2.0 ** -21, gamma0=2.0 ** -15, a_d=2.0 ** -30, a_d0=2.0 ** -16,
                                            a_p=2.0 ** -34, a_p0=2.0 ** -16, a_comm=2.0 ** -24,
                                            a_comm0=2.0 ** -16, n_layers=32))


# ---------------------------------------------------------------------------
# Multi-chunk steps: several prefill requests in one step (sp_degree 1).
# ---------------------------------------------------------------------------

@dataclass
class MultiChunkWorkload:
    """A layer step whose prefill side is a list of chunks [(chunk_len, prior_len)], each
    a different request with its own cached context, plus a decode population."""
    name: str
    seed_id: int
    dtype: str
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    n_decode: int
    ctx: tuple
    chunks: list
    page_size: int = 16
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    weight_std: float = 0.02
    description: str = ""

    @property
    def n_prefill_rows(self) -> int:
        return sum(l for l, _ in self.chunks)

    @property
    def n_rows(self) -> int:
        return self.n_prefill_rows + self.n_decode

    @property
    def qkv_dim(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclass
class MultiChunkInstance:
    wl: MultiChunkWorkload
    x: np.ndarray
    weights: dict
    dec_ctx: np.ndarray
    dec_pages: np.ndarray
    chunk_pages: list              # per chunk: [Hkv, blocks] int32
    pool: PagePool


def make_multi_instance(wl: MultiChunkWorkload) -> MultiChunkInstance:
    """Inputs of a multi-chunk step: rows [chunk 0 || chunk 1 || ... || decode].  Every
    chunk's table covers its prior context and the chunk on all kv heads; slots that hold
    no cached token (including the ones the step appends to) are NaN."""
    S, d, H = wl.page_size, wl.head_dim, wl.hidden
    Hq, Hkv, F = wl.n_q_heads, wl.n_kv_heads, wl.ffn_dim
    k, dt = wl.seed_id, wl.dtype
    x = _normal(k, "x", (wl.n_rows, H), 1.0, dt)
    ws = wl.weight_std
    weights = {
        "w_qkv": _normal(k, "w_qkv", (wl.qkv_dim, H), ws, dt),
        "w_o": _normal(k, "w_o", (H, Hq * d), ws, dt),
        "w_gate": _normal(k, "w_gate", (F, H), ws, dt),
        "w_up": _normal(k, "w_up", (F, H), ws, dt),
        "w_down": _normal(k, "w_down", (H, F), ws, dt),
    }
    one = f32_to_bf16_bits(np.ones(H, np.float32)) if dt == "bf16" else np.ones(H, np.float32)
    weights["g_attn"] = one.copy()
    weights["g_ffn"] = one.copy()
    ctx = _draw_ctx(wl)
    nb_dec = [_cdiv(int(c) + 1, S) for c in ctx]
    nb_ch = [_cdiv(c + l, S) for l, c in wl.chunks]
    n_pages = (sum(nb_dec) + sum(nb_ch)) * Hkv
    perm = _rng(k, "page_perm").permutation(n_pages).astype(np.int32)
    dec_pages = np.full((wl.n_decode, Hkv, max(max(nb_dec, default=1), 1)), -1, dtype=np.int32)
    valid = np.full(n_pages, S, dtype=np.int32)
    it = 0
    for i, c in enumerate(ctx):
        for g in range(Hkv):
            for b in range(nb_dec[i]):
                p = int(perm[it]); it += 1
                dec_pages[i, g, b] = p
                valid[p] = min(max(int(c) - b * S, 0), S)
    chunk_pages = []
    for (l, c), nb in zip(wl.chunks, nb_ch):
        t = np.full((Hkv, nb), -1, dtype=np.int32)
        for g in range(Hkv):
            for b in range(nb):
                p = int(perm[it]); it += 1
                t[g, b] = p
                valid[p] = min(max(c - b * S, 0), S)
        chunk_pages.append(t)
    arr = _draw_pages(k, "kv", n_pages, (2, S * d), dt)
    pool = PagePool(n_pages, (2, S * d), dt, valid, S, d, array=arr)
    ids = pool.poisoned_pages()
    if len(ids):
        arr[ids] = pool._poison(arr[ids].copy(), ids)
    return MultiChunkInstance(wl, x, weights, ctx, dec_pages, chunk_pages, pool)


MULTI_CHUNK_WORKLOADS = {
    # four requests' chunks in one step, bf16, ragged lengths, one starting at position 0
    "M1": MultiChunkWorkload("M1", 121, "bf16", 512, 8, 2, 128, 1024, n_decode=5, ctx=("uniform", 0, 600),
                             chunks=[(97, 0), (64, 130), (33, 17), (150, 400)],
                             description="small bf16 layer, 4 chunks + 5 decodes"),
    # fp32, with a one-token chunk and no decode shorter than a page
    "M2": MultiChunkWorkload("M2", 122, "f32", 256, 4, 2, 64, 512, n_decode=3, ctx=("uniform", 20, 90),
                             chunks=[(20, 5), (1, 0), (40, 100)],
                             description="tiny fp32 layer, 3 chunks incl. a 1-token chunk"),
    # prefill only: three chunks, no decode
    "M3": MultiChunkWorkload("M3", 123, "bf16", 512, 8, 2, 128, 1024, n_decode=0, ctx=("fixed", 0),
                             chunks=[(70, 33), (16, 0), (129, 250)],
                             description="small bf16 layer, 3 chunks, no decode"),
    # ten chunks: more than one grouped prefill launch (eight chunks per launch)
    "M4": MultiChunkWorkload("M4", 124, "bf16", 512, 8, 2, 128, 1024, n_decode=2, ctx=("uniform", 10, 300),
                             chunks=[(17, 0), (40, 3), (5, 60), (64, 16), (33, 200), (1, 7), (90, 0), (12, 500),
                                     (48, 31), (20, 100)],
                             description="small bf16 layer, 10 chunks + 2 decodes"),
    # the 8B step of the layer benchmark with its 1024 prefill rows from four requests
    "C2x4": MultiChunkWorkload("C2x4", 24, "bf16", 4096, 32, 8, 128, 14336, n_decode=16, ctx=("fixed", 8192),
                               chunks=[(256, 0), (256, 2048), (256, 4096), (256, 8192)],
                               description="Llama-3.1-8B layer: 16 decodes at 8192 + four 256-token chunks "
                                           "after 0/2048/4096/8192 cached tokens"),
}


# ---------------------------------------------------------------------------
# Layer stacks: one batch (x, decode contexts, page tables) through n layers, each
# with its own weights and its own KV pool laid out by the same tables.
# ---------------------------------------------------------------------------

@dataclass
class StackInstance:
    base: Instance                 # the batch and layer 0 (the single-layer draw)
    layers: list                   # per layer: {"weights": dict, "pool": PagePool}

    @property
    def wl(self) -> Workload:
        return self.base.wl


def make_stack_instance(wl: Workload, n_layers: int) -> StackInstance:
    """Layer 0 is make_instance(wl); layer l > 0 draws its weights and its pool pages
    from its own generators, with the same valid slots (NaN past each page's cached
    tokens) and, for banked pools, the same bank indices."""
    assert wl.sp_degree == 1 and n_layers >= 1
    base = make_instance(wl)
    k, dt = wl.seed_id, wl.dtype
    H, d, F, S = wl.hidden, wl.head_dim, wl.ffn_dim, wl.page_size
    layers = [{"weights": base.weights, "pool": base.pool}]
    for l in range(1, n_layers):
        ws = wl.weight_std
        w = {
            "w_qkv": _normal(k, "w_qkv", (wl.qkv_dim, H), ws, dt, l),
            "w_o": _normal(k, "w_o", (H, wl.n_q_heads * d), ws, dt, l),
            "w_gate": _normal(k, "w_gate", (F, H), ws, dt, l),
            "w_up": _normal(k, "w_up", (F, H), ws, dt, l),
            "w_down": _normal(k, "w_down", (H, F), ws, dt, l),
            "g_attn": base.weights["g_attn"].copy(),
            "g_ffn": base.weights["g_ffn"].copy(),
        }
        bp = base.pool
        if bp.bank is not None:
            bank = _draw_pages(k, "kv", bp.bank.shape[0], bp.row_shape, dt, l)
            pool = PagePool(bp.n_pages, bp.row_shape, dt, bp.valid_slots, S, d, bank=bank, bank_idx=bp.bank_idx)
        else:
            arr = _draw_pages(k, "kv", bp.n_pages, bp.row_shape, dt, l)
            pool = PagePool(bp.n_pages, bp.row_shape, dt, bp.valid_slots, S, d, array=arr)
            ids = pool.poisoned_pages()
            if len(ids):
                arr[ids] = pool._poison(arr[ids].copy(), ids)
        layers.append({"weights": w, "pool": pool})
    return StackInstance(base, layers)


# ---------------------------------------------------------------------------
# A drawn instance stored as plain .npy arrays plus a JSON description (no
# pickling), so another process can map the same inputs instead of drawing them
# again.
# ---------------------------------------------------------------------------

def save_instance(inst: Instance, path: str) -> None:
    import json
    import os
    os.makedirs(path, exist_ok=True)
    arrays = {"x": inst.x, "dec_ctx": inst.dec_ctx, "dec_pages": inst.dec_pages, "pre_pages": inst.pre_pages,
              "peer_qkv_in": inst.peer_qkv_in, "peer_attn_in": inst.peer_attn_in,
              "valid_slots": inst.pool.valid_slots}
    arrays.update({"w." + k: v for k, v in inst.weights.items()})
    pool = inst.pool
    if pool.array is not None:
        arrays["pool"] = pool.array
    else:
        arrays["bank"], arrays["bank_idx"] = pool.bank, pool.bank_idx
    for k, v in arrays.items():
        np.save(os.path.join(path, k + ".npy"), np.ascontiguousarray(v), allow_pickle=False)
    meta = {"workload": inst.wl.name, "n_pages": pool.n_pages, "row_shape": list(pool.row_shape),
            "dtype": pool.dtype, "page_size": pool.page_size, "head_dim": pool.head_dim,
            "weights": sorted(inst.weights), "arrays": sorted(arrays)}
    with open(os.path.join(path, "instance.json"), "w") as f:
        json.dump(meta, f)


def load_instance(path: str) -> Instance:
    """The instance save_instance stored (arrays memory-mapped read-only)."""
    import json
    import os
    meta = json.load(open(os.path.join(path, "instance.json")))
    a = {k: np.load(os.path.join(path, k + ".npy"), mmap_mode="r", allow_pickle=False) for k in meta["arrays"]}
    pool = PagePool(meta["n_pages"], tuple(meta["row_shape"]), meta["dtype"], np.asarray(a["valid_slots"]),
                    meta["page_size"], meta["head_dim"], array=a.get("pool"), bank=a.get("bank"),
                    bank_idx=a.get("bank_idx"))
    weights = {k: a["w." + k] for k in meta["weights"]}
    return Instance(get_workload(meta["workload"]), a["x"], weights, np.asarray(a["dec_ctx"]),
                    np.asarray(a["dec_pages"]), np.asarray(a["pre_pages"]), pool, a["peer_qkv_in"],
                    a["peer_attn_in"])
