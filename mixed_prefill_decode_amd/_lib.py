"""ctypes binding of libxp.so: the same entry points as include/xp.h, argument
marshalling only (device buffers are passed as torch tensors or raw addresses).

Every call raises ``XpError`` when the library returns a negative status.  The
library must be built (``python -m mixed_prefill_decode_amd.build``); there is
no fallback path.
"""
from __future__ import annotations

import atexit
import ctypes as C
import os
import weakref

import numpy as np

__all__ = ["XpError", "lib", "close_all", "XP_F32", "XP_BF16", "XP_EPI_F32", "XP_EPI_ADD_T", "XP_EPI_ADD_F32",
           "XP_EPI_SWIGLU", "XP_DEV_BAD_PAGE", "LayerShape", "LayerWeights", "KvPages", "BatchDesc",
           "WsLayout", "LatencyModel", "Ctx", "EXPORTED", "Chunk", "chunk_array",
           "xp_ctx_create", "xp_layer_workspace_layout", "xp_layer_forward", "xp_validate_batch",
           "xp_layer_workspace_layout_chunks", "xp_layer_forward_chunks", "xp_validate_chunks",
           "xp_stack_forward", "xp_stack_graph_create", "xp_graph_launch", "xp_graph_destroy", "Graph",
           "weights_array", "pools_array",
           "xp_layer_read_status", "xp_rmsnorm", "xp_gemm_workspace_size", "xp_gemm_tile", "xp_gemm", "xp_kv_append",
           "xp_kv_gather",
           "xp_decode_workspace_size", "xp_decode_attention", "xp_decode_attention_static", "XP_DECODE_STATIC_SCRATCH_BYTES",
           "xp_prefill_workspace_size", "xp_prefill_attention",
           "xp_probe_hw_ids", "xp_probe_read", "xp_calibrate_decode_cus", "xp_probe_read_curve", "CuCurve",
           "XP_SPLIT_SERIALIZED", "XP_SPLIT_UNMASKED", "STAGES", "XP_STAGE_COUNT",
           "xp_waterfill", "xp_iteration_latency", "xp_admission", "xp_decode_placement", "xp_schedule",
           "ScheduleCall", "WaterfillCall", "xp_fit_affine", "xp_fit_latency_model", "XP_SCHED_DONE", "XP_SCHED_BUDGET", "XP_SCHED_NO_HOST", "xp_build_info", "xp_last_error"]

XP_F32, XP_BF16 = 0, 1
XP_EPI_F32, XP_EPI_ADD_T, XP_EPI_ADD_F32, XP_EPI_SWIGLU = 0, 1, 2, 3
XP_DEV_BAD_PAGE = 1
XP_SPLIT_SERIALIZED, XP_SPLIT_UNMASKED = 0, -1
XP_SCHED_DONE, XP_SCHED_BUDGET, XP_SCHED_NO_HOST = 0, 1, 2
# layer stages of xp_ctx_stage_timing, in XP_STAGE_* order
STAGES = ("norm1", "qkv", "rope_append", "decode", "prefill", "o", "norm2", "gate_up", "down")
XP_STAGE_COUNT = len(STAGES)
STATUS_NAMES = {0: "XP_OK", -1: "XP_EINVAL", -2: "XP_ESHAPE", -3: "XP_EPAGE", -4: "XP_EHIP",
                -5: "XP_EUNSUPPORTED", -6: "XP_EWORKSPACE"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxp.so")

# every symbol include/xp.h declares
EXPORTED = ["xp_last_error", "xp_build_info", "xp_ctx_create", "xp_ctx_destroy", "xp_ctx_cu_masks",
            "xp_ctx_streams", "xp_ctx_stage_timing", "xp_ctx_stage_time",
            "xp_layer_workspace_layout", "xp_layer_forward", "xp_validate_batch", "xp_layer_read_status",
            "xp_layer_workspace_layout_chunks", "xp_layer_forward_chunks", "xp_validate_chunks",
            "xp_stack_forward", "xp_stack_graph_create", "xp_graph_launch", "xp_graph_destroy",
            "xp_rmsnorm", "xp_gemm_workspace_size", "xp_gemm_tile", "xp_gemm", "xp_kv_append", "xp_kv_gather",
            "xp_decode_workspace_size",
            "xp_decode_attention", "xp_decode_attention_static", "xp_prefill_workspace_size", "xp_prefill_attention", "xp_probe_hw_ids",
            "xp_probe_read", "xp_calibrate_decode_cus", "xp_probe_read_curve", "xp_waterfill",
            "xp_iteration_latency", "xp_fit_affine", "xp_fit_latency_model", "xp_admission",
            "xp_decode_placement", "xp_schedule"]


class XpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class LayerShape(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("ffn_dim", C.c_int32), ("page_size", C.c_int32),
                ("rms_eps", C.c_float), ("rope_base", C.c_double), ("dtype", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_ffn")]


class KvPages(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("n_pages", C.c_int32)]


class BatchDesc(C.Structure):
    _fields_ = [("x", C.c_void_p), ("n_prefill_local", C.c_int32), ("n_decode", C.c_int32),
                ("dec_ctx", C.c_void_p), ("dec_pages", C.c_void_p), ("dec_max_blocks", C.c_int32),
                ("chunk_len", C.c_int32), ("prior_len", C.c_int32), ("sp_degree", C.c_int32),
                ("sp_rank", C.c_int32), ("local_row_offset", C.c_int32), ("pre_pages", C.c_void_p),
                ("pre_max_blocks", C.c_int32), ("peer_qkv_in", C.c_void_p), ("peer_qkv_out", C.c_void_p),
                ("peer_attn_in", C.c_void_p), ("peer_attn_out", C.c_void_p), ("dec_ctx_host", C.c_void_p),
                ("dec_pages_host", C.c_void_p), ("pre_pages_host", C.c_void_p)]


class Chunk(C.Structure):
    _fields_ = [("chunk_len", C.c_int32), ("prior_len", C.c_int32), ("pre_pages", C.c_void_p),
                ("pre_max_blocks", C.c_int32), ("pre_pages_host", C.c_void_p)]


class WsLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("status", "hn", "qkv", "q_dec", "q_pre", "attn", "dec_ml",
                                          "dec_o", "pre_part", "gemm_part", "h1", "act", "total")] + \
               [("dec_splits", C.c_int32), ("dec_pages_per_split", C.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


XP_CU_CURVE_MAX = 64


class CuCurve(C.Structure):
    _fields_ = [("n_cus", C.c_int32), ("us_all", C.c_double), ("n_points", C.c_int32),
                ("cus", C.c_int32 * XP_CU_CURVE_MAX), ("us", C.c_double * XP_CU_CURVE_MAX)]

    def as_dict(self):
        return {"n_cus": self.n_cus, "us_all": self.us_all,
                "points": {int(self.cus[i]): float(self.us[i]) for i in range(self.n_points)}}


class LatencyModel(C.Structure):
    _fields_ = [(n, C.c_double) for n in ("gamma", "gamma0", "a_d", "a_d0", "a_p", "a_p0", "a_comm",
                                          "a_comm0", "alpha", "beta")] + [("n_layers", C.c_int32)]


class WaterfillIn(C.Structure):
    _fields_ = [("n_ranks", C.c_int32), ("n_decode_tokens", C.c_void_p), ("decode_ctx_sum", C.c_void_p),
                ("existing_assign", C.c_void_p), ("n_selected", C.c_int32), ("sel_len", C.c_void_p),
                ("sel_ctx", C.c_void_p), ("has_candidate", C.c_int32), ("m_remaining", C.c_int32),
                ("c_processed", C.c_int64), ("fixed_target", C.c_int32), ("level_hi", C.c_int32),
                ("quantum", C.c_int32), ("tbt_slo", C.c_double), ("model", C.POINTER(LatencyModel))]


class WaterfillOut(C.Structure):
    _fields_ = [("n_target", C.c_int32), ("budget", C.c_int64), ("chunk_len", C.c_int32),
                ("assign", C.c_void_p)]


class Samples(C.Structure):
    _fields_ = [("n", C.c_int32), ("x", C.c_void_p), ("t", C.c_void_p)]


class MixedSamples(C.Structure):
    _fields_ = [("n", C.c_int32), ("gemm_x", C.c_void_p), ("decode_x", C.c_void_p), ("prefill_x", C.c_void_p),
                ("comm_x", C.c_void_p), ("t", C.c_void_p)]


class DecodeState(C.Structure):
    _fields_ = [("n_ranks", C.c_int32), ("n_decode_tokens", C.c_void_p), ("decode_ctx_sum", C.c_void_p),
                ("kv_used", C.c_void_p), ("kv_capacity", C.c_void_p)]


class PrefillQueue(C.Structure):
    _fields_ = [("n", C.c_int32), ("m_remaining", C.c_void_p), ("c_processed", C.c_void_p),
                ("deadline", C.c_void_p)]


class SchedParams(C.Structure):
    _fields_ = [("now", C.c_double), ("tbt_slo", C.c_double), ("quantum", C.c_int32),
                ("kv_util_threshold", C.c_double), ("kv_headroom", C.c_int64),
                ("model", C.POINTER(LatencyModel))]


class ScheduleOut(C.Structure):
    _fields_ = [("ref_budget", C.c_int64), ("n_admitted", C.c_int32), ("n_selected", C.c_int32),
                ("stop", C.c_int32), ("order", C.c_void_p), ("chunk_len", C.c_void_p),
                ("decode_rank", C.c_void_p), ("prefill_assign", C.c_void_p), ("request_assign", C.c_void_p)]


_LIB = None
_vp, _i32, _sz, _f32, _f64 = C.c_void_p, C.c_int32, C.c_size_t, C.c_float, C.c_double


def _declare(L):
    S = _i32
    sig = {
        "xp_last_error": (C.c_char_p, []),
        "xp_build_info": (C.c_char_p, []),
        "xp_ctx_create": (S, [C.POINTER(_vp), _i32, _i32, _i32]),
        "xp_ctx_destroy": (S, [_vp]),
        "xp_ctx_cu_masks": (S, [_vp, _vp, _vp, _vp]),
        "xp_ctx_streams": (S, [_vp, C.POINTER(_vp), C.POINTER(_vp)]),
        "xp_ctx_stage_timing": (S, [_vp, _i32]),
        "xp_ctx_stage_time": (S, [_vp, _i32, C.POINTER(_i32), C.POINTER(C.c_double)]),
        "xp_layer_workspace_layout": (S, [_vp, C.POINTER(LayerShape), C.POINTER(BatchDesc), C.POINTER(WsLayout)]),
        "xp_layer_forward": (S, [_vp, C.POINTER(LayerShape), C.POINTER(BatchDesc), C.POINTER(LayerWeights),
                                 C.POINTER(KvPages), _vp, _vp, _sz, _vp]),
        "xp_layer_workspace_layout_chunks": (S, [_vp, C.POINTER(LayerShape), C.POINTER(BatchDesc), _i32,
                                                 C.POINTER(Chunk), C.POINTER(WsLayout)]),
        "xp_layer_forward_chunks": (S, [_vp, C.POINTER(LayerShape), C.POINTER(BatchDesc), _i32, C.POINTER(Chunk),
                                        C.POINTER(LayerWeights), C.POINTER(KvPages), _vp, _vp, _sz, _vp]),
        "xp_validate_chunks": (S, [C.POINTER(LayerShape), C.POINTER(BatchDesc), _i32, C.POINTER(Chunk), _i32, _vp,
                                   _vp, _vp]),
        "xp_stack_forward": (S, [_vp, C.POINTER(LayerShape), C.POINTER(BatchDesc), _i32, C.POINTER(LayerWeights),
                                 C.POINTER(KvPages), _vp, _vp, _sz, _vp]),
        "xp_stack_graph_create": (S, [_vp, C.POINTER(LayerShape), C.POINTER(BatchDesc), _i32,
                                      C.POINTER(LayerWeights), C.POINTER(KvPages), _vp, _vp, _sz, _vp,
                                      C.POINTER(_vp)]),
        "xp_graph_launch": (S, [_vp, _vp]),
        "xp_graph_destroy": (S, [_vp]),
        "xp_validate_batch": (S, [C.POINTER(LayerShape), C.POINTER(BatchDesc), _i32, _vp, _vp, _vp]),
        "xp_layer_read_status": (S, [_vp, C.POINTER(WsLayout), _vp, _vp]),
        "xp_rmsnorm": (S, [_i32, _vp, _i32, _vp, _vp, _i32, _i32, _f32, _vp]),
        "xp_gemm_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
        "xp_gemm_tile": (S, [_i32, _i32, _i32, _i32, _i32, C.POINTER(_i32), C.POINTER(_i32), C.POINTER(_i32)]),
        "xp_gemm": (S, [_i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
        "xp_kv_append": (S, [_i32, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp]),
        "xp_kv_gather": (S, [_i32, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _vp]),
        "xp_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
        "xp_decode_attention": (S, [_i32, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp,
                                    _i32, _vp, _i32, _vp]),
        "xp_decode_attention_static": (S, [_i32, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp,
                                           _i32, _i32, _vp]),
        "xp_prefill_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
        "xp_prefill_attention": (S, [_i32, _vp, _vp, _i32, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _i32, _vp, _i32, _vp, _i32, _vp, _i32, _vp, _vp]),
        "xp_probe_hw_ids": (S, [_i32, _vp, _vp]),
        "xp_probe_read": (S, [_vp, _sz, _vp, _vp]),
        "xp_calibrate_decode_cus": (S, [_i32, _i32, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                        _vp, _i32, _vp, _i32, _f64, _i32, _i32, _i32, C.POINTER(_i32),
                                        C.POINTER(CuCurve)]),
        "xp_probe_read_curve": (S, [_i32, _vp, _sz, _vp, _i32, _i32, C.POINTER(CuCurve)]),
        "xp_waterfill": (S, [C.POINTER(WaterfillIn), C.POINTER(WaterfillOut)]),
        "xp_iteration_latency": (S, [C.POINTER(LatencyModel), _i32, _vp, _vp, _vp, _i32, _vp, _vp,
                                     C.POINTER(_f64)]),
        "xp_fit_affine": (S, [C.POINTER(Samples), C.POINTER(_f64), C.POINTER(_f64)]),
        "xp_fit_latency_model": (S, [C.POINTER(Samples)] * 4 + [C.POINTER(MixedSamples), _i32, _f64,
                                                                C.POINTER(LatencyModel)]),
        "xp_admission": (S, [C.POINTER(PrefillQueue), C.c_int64, _f64, _f64, _vp, C.POINTER(_i32)]),
        "xp_decode_placement": (S, [C.POINTER(DecodeState), C.c_int64, _f64, C.c_int64, C.POINTER(_i32)]),
        "xp_schedule": (S, [C.POINTER(DecodeState), C.POINTER(PrefillQueue), C.POINTER(SchedParams),
                            C.POINTER(ScheduleOut)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


# Contexts and captured graphs still open.  They own HIP streams, events and graphs,
# which are destroyed at interpreter exit by an atexit hook (registered when the
# library is loaded, so it runs while the HIP runtime is still up) rather than left
# to garbage collection during interpreter teardown or to the runtime's own
# finalizers: graphs first, then the contexts whose streams they were captured on.
_LIVE_GRAPHS = weakref.WeakSet()
_LIVE_CTXS = weakref.WeakSet()


def close_all():
    """Destroys every open Graph, then every open Ctx (safe to call more than once)."""
    for g in list(_LIVE_GRAPHS):
        try:
            g.close()
        except Exception:
            pass
    for c in list(_LIVE_CTXS):
        try:
            c.close()
        except Exception:
            pass


def lib():
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise XpError(-4, f"{LIB_PATH} is missing: build it with `python -m mixed_prefill_decode_amd.build`")
        L = C.CDLL(LIB_PATH)
        _declare(L)
        _LIB = L
        atexit.register(close_all)
    return _LIB


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(type(x))


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int):
    if st != 0:
        raise XpError(st, lib().xp_last_error().decode())


def xp_last_error() -> str:
    return lib().xp_last_error().decode()


def xp_build_info() -> str:
    return lib().xp_build_info().decode()


class Ctx:
    """Owns an xp_ctx (two attention streams + fork/join events)."""

    def __init__(self, device: int = 0, decode_cus: int = 0, pages_per_split: int = 0):
        h = _vp()
        _check(lib().xp_ctx_create(C.byref(h), device, decode_cus, pages_per_split))
        self.handle = h
        self.device, self.decode_cus = device, decode_cus
        _LIVE_CTXS.add(self)

    def cu_masks(self):
        dec = (C.c_uint32 * 8)()
        pre = (C.c_uint32 * 8)()
        n = _i32()
        _check(lib().xp_ctx_cu_masks(self.handle, dec, pre, C.byref(n)))
        return list(dec), list(pre), n.value

    def streams(self):
        """(decode stream, prefill stream) raw handles; 0 in serialized mode."""
        d, p = _vp(), _vp()
        _check(lib().xp_ctx_streams(self.handle, C.byref(d), C.byref(p)))
        return d.value or 0, p.value or 0

    def stage_timing(self, capacity: int):
        """Times the next `capacity` eager runs of every layer stage (0 stops)."""
        _check(lib().xp_ctx_stage_timing(self.handle, capacity))

    def stage_times(self) -> dict:
        """{stage name: (runs, total milliseconds)} of the runs timed so far (waits for them)."""
        out = {}
        for k, name in enumerate(STAGES):
            n, ms = _i32(), C.c_double()
            _check(lib().xp_ctx_stage_time(self.handle, k, C.byref(n), C.byref(ms)))
            out[name] = (n.value, ms.value)
        return out

    def close(self):
        if getattr(self, "handle", None):
            h, self.handle = self.handle, None
            _LIVE_CTXS.discard(self)
            lib().xp_ctx_destroy(h)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def xp_ctx_create(device=0, decode_cus=0, pages_per_split=0) -> Ctx:
    return Ctx(device, decode_cus, pages_per_split)


def xp_layer_workspace_layout(ctx, shape: LayerShape, desc: BatchDesc) -> WsLayout:
    L = WsLayout()
    _check(lib().xp_layer_workspace_layout(ctx.handle if ctx else None, C.byref(shape), C.byref(desc), C.byref(L)))
    return L


def xp_layer_forward(ctx, shape, desc, weights, kv, out, workspace, workspace_bytes, stream=None):
    _check(lib().xp_layer_forward(ctx.handle, C.byref(shape), C.byref(desc), C.byref(weights), C.byref(kv),
                                  _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)))


def xp_layer_workspace_layout_chunks(ctx, shape, desc, chunks) -> WsLayout:
    """``chunks``: a ctypes array of Chunk (see chunk_array)."""
    out = WsLayout()
    _check(lib().xp_layer_workspace_layout_chunks(ctx.handle if ctx is not None else None, C.byref(shape),
                                                  C.byref(desc), len(chunks), chunks, C.byref(out)))
    return out


def xp_layer_forward_chunks(ctx, shape, desc, chunks, weights, kv, out, workspace, workspace_bytes, stream=None):
    _check(lib().xp_layer_forward_chunks(ctx.handle, C.byref(shape), C.byref(desc), len(chunks), chunks,
                                         C.byref(weights), C.byref(kv), _ptr(out), _ptr(workspace), workspace_bytes,
                                         _stream(stream)))


def weights_array(weights):
    """ctypes array of LayerWeights, one per layer of a stack."""
    arr = (LayerWeights * len(weights))()
    for l, w in enumerate(weights):
        arr[l] = w
    return arr


def pools_array(pools):
    """ctypes array of KvPages from [(pool tensor, n_pages)], one per layer of a stack."""
    arr = (KvPages * len(pools))()
    for l, (p, n) in enumerate(pools):
        arr[l] = KvPages(_ptr(p), int(n))
    return arr


def xp_stack_forward(ctx, shape, desc, weights, pools, out, workspace, workspace_bytes, stream=None):
    """``weights``/``pools``: ctypes arrays of one LayerWeights / KvPages per layer."""
    if len(weights) != len(pools):
        raise ValueError("one weight set and one pool per layer")
    _check(lib().xp_stack_forward(ctx.handle, C.byref(shape), C.byref(desc), len(weights), weights, pools,
                                  _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)))


class Graph:
    """A captured stack (xp_stack_graph_create); ``launch`` replays it, ``close`` frees it."""

    def __init__(self, handle):
        self.handle = handle
        _LIVE_GRAPHS.add(self)

    def launch(self, stream=None):
        xp_graph_launch(self, stream)

    def close(self):
        if getattr(self, "handle", None):
            h, self.handle = self.handle, None
            _LIVE_GRAPHS.discard(self)
            _check(lib().xp_graph_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def xp_stack_graph_create(ctx, shape, desc, weights, pools, out, workspace, workspace_bytes, stream) -> Graph:
    if len(weights) != len(pools):
        raise ValueError("one weight set and one pool per layer")
    h = _vp()
    _check(lib().xp_stack_graph_create(ctx.handle, C.byref(shape), C.byref(desc), len(weights), weights, pools,
                                       _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream), C.byref(h)))
    return Graph(h)


def xp_graph_launch(graph, stream=None):
    _check(lib().xp_graph_launch(graph.handle, _stream(stream)))


def xp_graph_destroy(graph):
    graph.close()


def chunk_array(chunks, host_tables=None):
    """ctypes array of Chunk from [(chunk_len, prior_len, table tensor [Hkv, blocks])];
    ``host_tables``: optional host copies of the tables (validated before launch)."""
    arr = (Chunk * max(1, len(chunks)))()
    keep = []
    for j, (l, c, t) in enumerate(chunks):
        h = None
        if host_tables is not None:
            h = np.ascontiguousarray(host_tables[j], dtype=np.int32)
            keep.append(h)
        arr[j] = Chunk(int(l), int(c), _ptr(t), int(t.shape[-1]), _ptr(h))
    out = arr if chunks else (Chunk * 0)()
    out._host = keep          # the host copies live as long as the array
    return out


def xp_validate_chunks(shape, desc, chunks, n_pages, dec_ctx_host, dec_pages_host, chunk_tables_host):
    """``chunks``: a ctypes Chunk array; ``chunk_tables_host``: the chunks' host tables in list order."""
    flat = np.ascontiguousarray(np.concatenate([np.asarray(t, dtype=np.int32).reshape(-1) for t in chunk_tables_host])
                                if len(chunk_tables_host) else np.zeros(1, np.int32), dtype=np.int32)
    arrs = [None if a is None else np.ascontiguousarray(a, dtype=np.int32) for a in (dec_ctx_host, dec_pages_host)]
    return lib().xp_validate_chunks(C.byref(shape), C.byref(desc), len(chunks), chunks, n_pages,
                                    *[_ptr(a) for a in arrs], _ptr(flat))


def xp_validate_batch(shape, desc, n_pages, dec_ctx_host, dec_pages_host, pre_pages_host):
    arrs = [None if a is None else np.ascontiguousarray(a, dtype=np.int32)
            for a in (dec_ctx_host, dec_pages_host, pre_pages_host)]
    return lib().xp_validate_batch(C.byref(shape), C.byref(desc), n_pages, *[_ptr(a) for a in arrs])


def xp_layer_read_status(workspace, layout: WsLayout, stream=None) -> int:
    v = C.c_uint32()
    _check(lib().xp_layer_read_status(_ptr(workspace), C.byref(layout), C.byref(v), _stream(stream)))
    return v.value


def xp_rmsnorm(dtype, x, x_is_f32, gamma, y, M, H, eps, stream=None):
    _check(lib().xp_rmsnorm(dtype, _ptr(x), int(x_is_f32), _ptr(gamma), _ptr(y), M, H, eps, _stream(stream)))


def xp_gemm_workspace_size(dtype, epilogue, M, N, K) -> int:
    return int(lib().xp_gemm_workspace_size(dtype, epilogue, M, N, K))


def xp_gemm_tile(dtype, epilogue, M, N, K) -> tuple:
    """(rows, columns, K splits) of the work unit xp_gemm would use for this product."""
    bm, bn, sp = _i32(), _i32(), _i32()
    _check(lib().xp_gemm_tile(dtype, epilogue, M, N, K, C.byref(bm), C.byref(bn), C.byref(sp)))
    return bm.value, bn.value, sp.value


def xp_gemm(dtype, epilogue, A, B, B2, R, Cout, M, N, K, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().xp_gemm(dtype, epilogue, _ptr(A), _ptr(B), _ptr(B2), _ptr(R), _ptr(Cout), M, N, K,
                         _ptr(workspace), workspace_bytes, _stream(stream)))


def xp_kv_append(dtype, pool, n_pages, page_size, head_dim, table, table_stride, seq, pos, k, v, n, stream=None):
    _check(lib().xp_kv_append(dtype, _ptr(pool), n_pages, page_size, head_dim, _ptr(table), table_stride,
                              _ptr(seq), _ptr(pos), _ptr(k), _ptr(v), n, _stream(stream)))


def xp_kv_gather(dtype, pool, n_pages, page_size, head_dim, table, table_stride, lens, n_seq, max_len, k_out,
                 v_out, stream=None):
    _check(lib().xp_kv_gather(dtype, _ptr(pool), n_pages, page_size, head_dim, _ptr(table), table_stride,
                              _ptr(lens), n_seq, max_len, _ptr(k_out), _ptr(v_out), _stream(stream)))


def xp_decode_workspace_size(n_decode, n_q_heads, n_kv_heads, head_dim, dec_max_blocks, pages_per_split) -> int:
    return int(lib().xp_decode_workspace_size(n_decode, n_q_heads, n_kv_heads, head_dim, dec_max_blocks,
                                              pages_per_split))


def xp_decode_attention(dtype, q, pool, n_pages, page_size, dec_pages, dec_max_blocks, dec_ctx, n_decode,
                        n_q_heads, n_kv_heads, head_dim, out, out_stride, workspace, pages_per_split,
                        stream=None):
    _check(lib().xp_decode_attention(dtype, _ptr(q), _ptr(pool), n_pages, page_size, _ptr(dec_pages),
                                     dec_max_blocks, _ptr(dec_ctx), n_decode, n_q_heads, n_kv_heads, head_dim,
                                     _ptr(out), out_stride, _ptr(workspace), pages_per_split, _stream(stream)))


def xp_decode_attention_static(dtype, q, pool, n_pages, page_size, dec_pages, dec_max_blocks, dec_ctx, n_decode,
                               n_q_heads, n_kv_heads, head_dim, out, out_stride, pages_per_split, stream=None):
    _check(lib().xp_decode_attention_static(dtype, _ptr(q), _ptr(pool), n_pages, page_size, _ptr(dec_pages),
                                            dec_max_blocks, _ptr(dec_ctx), n_decode, n_q_heads, n_kv_heads,
                                            head_dim, _ptr(out), out_stride, pages_per_split, _stream(stream)))


XP_DECODE_STATIC_SCRATCH_BYTES = 64 << 20


def xp_prefill_workspace_size(hq, hkv, head_dim, prior_len, chunk_len, plan_cus=0) -> int:
    return int(lib().xp_prefill_workspace_size(hq, hkv, head_dim, prior_len, chunk_len, plan_cus))


def xp_prefill_attention(dtype, q, pool, n_pages, page_size, pre_pages, pre_max_blocks, hq, hkv, head_dim,
                         prior_len, chunk_len, off, n_local, out_local, out_local_stride, out_peer,
                         out_peer_stride, workspace=None, status=None, stream=None, plan_cus=0):
    _check(lib().xp_prefill_attention(dtype, _ptr(q), _ptr(pool), n_pages, page_size, _ptr(pre_pages),
                                      pre_max_blocks, hq, hkv, head_dim, prior_len, chunk_len, off, n_local,
                                      _ptr(out_local), out_local_stride, _ptr(out_peer), out_peer_stride,
                                      _ptr(workspace), plan_cus, _ptr(status), _stream(stream)))


def xp_probe_hw_ids(n_blocks, out, stream=None):
    _check(lib().xp_probe_hw_ids(n_blocks, _ptr(out), _stream(stream)))


def xp_probe_read(src, nbytes, sink, stream=None):
    _check(lib().xp_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)))


def xp_calibrate_decode_cus(device, dtype, q, pool, n_pages, page_size, dec_pages, dec_max_blocks, dec_ctx,
                            n_decode, n_q_heads, n_kv_heads, head_dim, out, out_stride, workspace,
                            pages_per_split=0, keep_fraction=0.9, cu_step=32, repeats=10, stop_at_rule=True):
    """(decode_cus, curve dict): the pages' decode-CU rule measured on this device."""
    k = _i32()
    cv = CuCurve()
    _check(lib().xp_calibrate_decode_cus(device, dtype, _ptr(q), _ptr(pool), n_pages, page_size, _ptr(dec_pages),
                                         dec_max_blocks, _ptr(dec_ctx), n_decode, n_q_heads, n_kv_heads, head_dim,
                                         _ptr(out), out_stride, _ptr(workspace), pages_per_split,
                                         float(keep_fraction), cu_step, repeats, int(bool(stop_at_rule)),
                                         C.byref(k), C.byref(cv)))
    return k.value, cv.as_dict()


def xp_probe_read_curve(device, src, nbytes, sink, cu_step=32, repeats=5) -> dict:
    cv = CuCurve()
    _check(lib().xp_probe_read_curve(device, _ptr(src), nbytes, _ptr(sink), cu_step, repeats, C.byref(cv)))
    return cv.as_dict()


def _model(d: dict) -> LatencyModel:
    return LatencyModel(*[float(d[k]) for k in ("gamma", "gamma0", "a_d", "a_d0", "a_p", "a_p0", "a_comm",
                                                "a_comm0", "alpha", "beta")], int(d["n_layers"]))


class WaterfillCall:
    """One xp_waterfill call with its arguments marshalled once: ``call()`` runs the
    dispatcher on them (so a caller can time the native call alone), ``result()``
    decodes the last call's outputs."""

    def __init__(self, *, tau, n_decode_tokens, decode_ctx_sum, existing=None, selected=(), candidate=None,
                 quantum=1, model, fixed_target=-1, level_hi=0):
        N = len(n_decode_tokens)
        self._arrs = (np.ascontiguousarray(n_decode_tokens, dtype=np.int32),
                      np.ascontiguousarray(decode_ctx_sum, dtype=np.int64),
                      None if existing is None else np.ascontiguousarray(existing, dtype=np.int32),
                      np.ascontiguousarray([s[0] for s in selected] or [0], dtype=np.int32),
                      np.ascontiguousarray([s[1] for s in selected] or [0], dtype=np.int64))
        nd, cs, ex, sl, sc = self._arrs
        self._m = _model(model)
        self.inp = WaterfillIn(N, _ptr(nd), _ptr(cs), _ptr(ex), len(selected), _ptr(sl), _ptr(sc),
                               1 if candidate is not None else 0, int(candidate[0]) if candidate else 0,
                               int(candidate[1]) if candidate else 0, int(fixed_target), int(level_hi), int(quantum),
                               float(tau), C.pointer(self._m))
        self.assign = np.zeros(N, dtype=np.int32)
        self.out = WaterfillOut(0, 0, 0, _ptr(self.assign))
        self._fn = lib().xp_waterfill
        self._args = (C.byref(self.inp), C.byref(self.out))

    def call(self):
        _check(self._fn(*self._args))
        return self

    def result(self) -> dict:
        o = self.out
        return dict(n_target=o.n_target, budget=o.budget, chunk_len=o.chunk_len, assign=self.assign.tolist())


def xp_waterfill(**kw) -> dict:
    """Algorithm 2 (keyword arguments as WaterfillCall)."""
    return WaterfillCall(**kw).call().result()


def xp_iteration_latency(model: dict, n_decode_tokens, decode_ctx_sum, n_prefill_tokens, chunks) -> float:
    N = len(n_decode_tokens)
    nd = np.ascontiguousarray(n_decode_tokens, dtype=np.int32)
    cs = np.ascontiguousarray(decode_ctx_sum, dtype=np.int64)
    npf = np.ascontiguousarray(n_prefill_tokens, dtype=np.int32)
    cl = np.ascontiguousarray([c[0] for c in chunks] or [0], dtype=np.int32)
    cc = np.ascontiguousarray([c[1] for c in chunks] or [0], dtype=np.int64)
    m = _model(model)
    t = _f64()
    _check(lib().xp_iteration_latency(C.byref(m), N, _ptr(nd), _ptr(cs), _ptr(npf), len(chunks), _ptr(cl),
                                      _ptr(cc), C.byref(t)))
    return t.value


_STOP_NAMES = {XP_SCHED_DONE: "done", XP_SCHED_BUDGET: "budget", XP_SCHED_NO_HOST: "no_host"}


def _queue(m_remaining, c_processed, deadlines):
    m = np.ascontiguousarray(m_remaining, dtype=np.int32)
    c = np.ascontiguousarray(c_processed, dtype=np.int64)
    d = np.ascontiguousarray(deadlines, dtype=np.float64)
    return PrefillQueue(len(m), _ptr(m), _ptr(c), _ptr(d)), (m, c, d)


def _state(n_decode_tokens, decode_ctx_sum, kv_used, kv_capacity):
    arrs = (np.ascontiguousarray(n_decode_tokens, dtype=np.int32),
            np.ascontiguousarray(decode_ctx_sum, dtype=np.int64),
            np.ascontiguousarray(kv_used, dtype=np.int64), np.ascontiguousarray(kv_capacity, dtype=np.int64))
    return DecodeState(len(arrs[0]), *[_ptr(a) for a in arrs]), arrs


def xp_admission(m_remaining, deadlines, ref_budget, now, tau, c_processed=None):
    """(admitted in EDF order, removed in SJF order) -- Algorithm 4."""
    q, keep = _queue(m_remaining, [0] * len(m_remaining) if c_processed is None else c_processed, deadlines)
    order = np.zeros(max(1, q.n), dtype=np.int32)
    n_adm = _i32()
    _check(lib().xp_admission(C.byref(q), int(ref_budget), float(now), float(tau), _ptr(order), C.byref(n_adm)))
    o = order[:q.n].tolist()
    return o[:n_adm.value], o[n_adm.value:]


def xp_decode_placement(decode_ctx_sum, kv_used, kv_capacity, need, eta, headroom, n_decode_tokens=None):
    """Host rank of a request with ``need`` KV tokens, or None (Infeasible) -- Algorithm 3."""
    nd = [0] * len(kv_used) if n_decode_tokens is None else n_decode_tokens
    st, keep = _state(nd, decode_ctx_sum, kv_used, kv_capacity)
    g = _i32()
    _check(lib().xp_decode_placement(C.byref(st), int(need), float(eta), int(headroom), C.byref(g)))
    return None if g.value < 0 else g.value


class ScheduleCall:
    """One xp_schedule call with its arguments marshalled once: ``call()`` runs the
    scheduler on them (so a caller can time the native call alone), ``result()``
    decodes the last call's outputs."""

    def __init__(self, *, n_decode_tokens, decode_ctx_sum, kv_used, kv_capacity, m_remaining, c_processed,
                 deadlines, now, tau, quantum, eta, headroom, model):
        self.state, self._keep_s = _state(n_decode_tokens, decode_ctx_sum, kv_used, kv_capacity)
        self.queue, self._keep_q = _queue(m_remaining, c_processed, deadlines)
        N, R = self.state.n_ranks, self.queue.n
        self._model = _model(model)
        self.params = SchedParams(float(now), float(tau), int(quantum), float(eta), int(headroom),
                                  C.pointer(self._model))
        self.order = np.zeros(max(1, R), dtype=np.int32)
        self.chunk = np.zeros(max(1, R), dtype=np.int32)
        self.host = np.zeros(max(1, R), dtype=np.int32)
        self.a_p = np.zeros(N, dtype=np.int32)
        self.req = np.zeros((max(1, R), N), dtype=np.int32)
        self.out = ScheduleOut(0, 0, 0, 0, _ptr(self.order), _ptr(self.chunk), _ptr(self.host), _ptr(self.a_p),
                               _ptr(self.req))
        self._fn = lib().xp_schedule
        self._args = (C.byref(self.state), C.byref(self.queue), C.byref(self.params), C.byref(self.out))

    def call(self):
        _check(self._fn(*self._args))
        return self

    def result(self) -> dict:
        R, o = self.queue.n, self.out
        return dict(ref_budget=o.ref_budget, n_admitted=o.n_admitted, order=self.order[:R].tolist(),
                    n_selected=o.n_selected, stop=_STOP_NAMES[o.stop], chunk_len=self.chunk[:R].tolist(),
                    decode_rank=self.host[:R].tolist(), prefill_assign=self.a_p.tolist(),
                    request_assign=self.req[:R].tolist())


def xp_schedule(**kw) -> dict:
    """One iteration of the SLO-aware scheduler (Algorithm 1); keyword arguments as
    ScheduleCall."""
    return ScheduleCall(**kw).call().result()


def _samples(x, t):
    xa = np.ascontiguousarray(x, dtype=np.float64)
    ta = np.ascontiguousarray(t, dtype=np.float64)
    if xa.shape != ta.shape:
        raise ValueError("x and t differ in length")
    return Samples(len(xa), _ptr(xa), _ptr(ta)), (xa, ta)


def xp_fit_affine(x, t) -> tuple:
    """(slope, intercept) of t ~ slope x + intercept on relative error (App. D base functions)."""
    s, keep = _samples(x, t)
    a, b = _f64(), _f64()
    _check(lib().xp_fit_affine(C.byref(s), C.byref(a), C.byref(b)))
    return a.value, b.value


def xp_fit_latency_model(gemm, decode, prefill, comm, mixed, n_layers=1, ab_max=3.0) -> dict:
    """The latency model from isolated profiles ((x, t) pairs) and heterogeneous iterations
    [(gemm_x, decode_x, prefill_x, comm_x, t)]."""
    parts = [_samples(*p) for p in (gemm, decode, prefill, comm)]
    cols = [np.ascontiguousarray([m[k] for m in mixed], dtype=np.float64) for k in range(5)]
    ms = MixedSamples(len(mixed), *[_ptr(c) for c in cols])
    out = LatencyModel()
    _check(lib().xp_fit_latency_model(*[C.byref(p[0]) for p in parts], C.byref(ms), int(n_layers), float(ab_max),
                                      C.byref(out)))
    return {f: getattr(out, f) for f, _ in LatencyModel._fields_}
