#!/usr/bin/env python3
"""Benchmark of one GPU's share of a Conflux Parallelism layer step on MI355X.

A timed step is one pass of the whole hot path over one batch: the waterfill
dispatch of the iteration's chunk (host) and one xp_layer_forward (co-batched
RMSNorm + QKV GEMM, RoPE + paged K/V append, decode attention || prefill
attention on a CU partition, O-proj, RMSNorm, gate/up + SwiGLU, down), inputs
resident in HBM.  Prints one JSON line (metric, value, roofline of the dominant
kernel, the fp64 oracle timed on the host as a baseline) on stdout; details go
to stderr.  The dominant kernel is the one with the longest launches inside the
step, timed by the library's stage events over a second pass of the same steps
(`stages_us`); standalone loops of each kernel are reported beside it (`kernels`).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload C5]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import shutil
import sys
import tempfile
import time

import numpy as np

METRIC = "mixed-layer tokens/s; decode-attn HBM GB/s and GEMM MFMA util as % of peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="C5")
    p.add_argument("--decode-cus", type=int, default=None,
                   help="CUs for decode attention (default: the fastest of serialized, unmasked and a sweep of "
                        "partitions that includes the pages' 90%% rule; 0 = serialized, -1 = unmasked)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=25.0)
    p.add_argument("--kernel-only", choices=["none", "qkv", "o", "gate_up", "down", "decode_attn", "prefill_attn", "read",
                                             "copy"], default="none",
                   help="only launch one kernel repeatedly (for counter runs)")
    p.add_argument("--no-kernel-loops", action="store_true",
                   help="skip the standalone per-kernel timing loops (a kernel trace then holds only the "
                        "step's own launches)")
    p.add_argument("--extra-decode", default="C4",
                   help="also time this workload's decode attention alone (its KV pool is built on the device); "
                        "'none' to skip")
    p.add_argument("--no-split-sweep", action="store_true",
                   help="time the step serialized only (no split-attention probes)")
    p.add_argument("--instance-cache", default=None, help="internal: directory of a saved input instance")
    p.add_argument("--repeats", type=int, default=20, help="launches per kernel timing")
    p.add_argument("--estimator", action="store_true",
                   help="fit the iteration-latency estimator on this GPU from isolated profiles and report its "
                        "error on random heterogeneous batches, instead of the layer benchmark")
    p.add_argument("--estimator-decode-cus", type=int, default=128,
                   help="decode CUs of the concurrent split attention the estimator models")
    p.add_argument("--estimator-batches", type=int, default=200)
    p.add_argument("--estimator-out", default=None, help="write every profiled and evaluated batch here (JSON)")
    p.add_argument("--stack", type=int, default=0,
                   help="run the workload's batch through this many layers (each with its own weights and KV "
                        "pool) eagerly and as piecewise graph launches, instead of the layer benchmark")
    p.add_argument("--probe", default=None,
                   help="internal: time one split-attention mode in this fresh process ('rule' = the pages' "
                        "decode-CU calibration, or a decode CU count) and print it as one JSON line")
    return p.parse_args()


class Timer:
    """HIP-event timing on torch's current stream.  The GPU's clock drops after a few
    milliseconds idle and takes most of a 20-step window to recover (measured: the
    first window after a 50 ms gap is ~9% slow), so n untimed calls run first."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, n):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        for _ in range(n):
            fn()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / n * 1e-3  # seconds per launch


def decode_bytes(inst) -> int:
    """Algorithmic bytes of decode attention: every K/V element of the visible context once
    (for all G heads of a group), q in, o out, the table entries read."""
    wl = inst.wl
    eb = 2 if wl.dtype == "bf16" else 4
    keys = int(np.sum(inst.dec_ctx.astype(np.int64) + 1))
    kv = keys * 2 * wl.n_kv_heads * wl.head_dim * eb
    qo = 2 * wl.n_decode * wl.n_q_heads * wl.head_dim * eb
    tbl = int(np.sum(-(-(inst.dec_ctx.astype(np.int64) + 1) // wl.page_size))) * wl.n_kv_heads * 4
    return kv + qo + tbl


def prefill_flops(wl) -> int:
    pairs = wl.chunk_len * wl.prior_len + wl.chunk_len * (wl.chunk_len + 1) // 2
    return 4 * wl.head_dim * wl.hq_loc * pairs


def gemm_list(wl):
    M, H, F, d = wl.n_rows, wl.hidden, wl.ffn_dim, wl.head_dim
    return {"qkv": (M, (wl.n_q_heads + 2 * wl.n_kv_heads) * d, H), "o": (M, H, wl.n_q_heads * d),
            "gate_up": (M, 2 * F, H), "down": (M, H, F)}


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
# the sources each measured kernel is built from: a traffic record counts only while they
# hash to the value recorded with it
KERNEL_SOURCES = {
    "gemm": ("mixed_prefill_decode_amd/csrc/gemm_core.h", "mixed_prefill_decode_amd/csrc/gemm.hip",
             "mixed_prefill_decode_amd/csrc/xp_device.h"),
    "decode_attn": ("mixed_prefill_decode_amd/csrc/decode_attn.hip", "mixed_prefill_decode_amd/csrc/xp_device.h"),
    "prefill_attn": ("mixed_prefill_decode_amd/csrc/prefill_attn.hip", "mixed_prefill_decode_amd/csrc/gemm_core.h",
                     "mixed_prefill_decode_amd/csrc/xp_device.h"),
}
KERNEL_NAMES = {
    "qkv": "gemm_kernel<bf16,F32 or RoPE/append epilogue> (QKV projection)", "o": "gemm_kernel<bf16,AddT> (O projection + residual)",
    "gate_up": "gemm_kernel<bf16,SwiGLU> (gate/up projection)",
    "down": "gemm_kernel<bf16,AddF32> (down projection + residual)",
    "decode_attn": "decode_split_kernel + decode_combine_kernel (paged GQA decode attention)",
    "prefill_attn": "prefill_kernel (+ prefill_combine_kernel) (causal chunked-prefill attention)",
}
# the attention kernels' co-resident forms, which the step runs when decode and prefill
# attention share every CU
CORES_KERNEL_NAMES = {
    "decode_attn": "decode_split_cores_kernel + decode_combine_kernel (paged GQA decode attention, co-resident form)",
    "prefill_attn": "prefill_cores_kernel (+ prefill_combine_kernel) (causal chunked-prefill attention, co-resident form)",
}
# layer stages (xp_ctx_stage_timing) -> the kernel figures above they time inside the step
STAGE_KERNELS = {"qkv": "qkv", "o": "o", "gate_up": "gate_up", "down": "down", "decode": "decode_attn",
                 "prefill": "prefill_attn"}


def sources_hash(kernel: str) -> str:
    key = "gemm" if kernel in ("qkv", "o", "gate_up", "down") else kernel
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for f in KERNEL_SOURCES[key]:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` on `workload` from a committed counter summary
    (profiles/*_traffic.md: FETCH_SIZE and WRITE_SIZE scaled by what the same counters
    read for a copy kernel), or None when there is none for this pair or the kernel's
    sources changed since it was taken."""
    import glob
    try:
        want = sources_hash(kernel)
    except OSError:
        return None
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_traffic.md"))):
        try:
            text = open(path).read()
            rec = json.loads(text[text.index("```json") + 7:text.index("```", text.index("```json") + 7)])
        except (OSError, ValueError):
            continue
        if rec.get("workload") == workload and rec.get("kernel") == kernel and rec.get("src_sha256_16") == want:
            return rec["traffic_bytes"]
    return None


def cpu_baseline(inst, budget_s: float) -> dict:
    """The fp64 oracle (as it stands) on the host: full layer steps until the budget is used."""
    from oracle import layer as L
    from tests.helpers import oracle_kwargs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    t0 = time.perf_counter()
    n = 0
    while True:
        L.layer_forward(**oracle_kwargs(inst))
        n += 1
        if time.perf_counter() - t0 > budget_s / 2 or n >= 3:
            break
    dt = (time.perf_counter() - t0) / n
    return {"value": round(inst.wl.n_rows / dt, 2), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} full {inst.wl.name} layer step(s) of {inst.wl.n_rows} rows in fp64 on the host "
                      f"({dt:.2f} s each)"}


class EstimatorRig:
    """Device buffers for timing Llama-3.1-8B layer steps of arbitrary batch mixes: random
    bf16 weights, a random KV pool large enough for 128 decodes at 16K context plus a
    10K-token chunk after 16K cached tokens, and page tables cut from one random
    permutation of the pool."""

    H, HQ, HKV, D, F, PAGE = 4096, 32, 8, 128, 14336, 16
    MAX_ROWS = 10240 + 128

    def __init__(self, X, torch, ctx):
        self.X, self.torch, self.ctx = X, torch, ctx
        g = torch.Generator(device="cuda")
        g.manual_seed(1234)
        H, HQ, HKV, D, F = self.H, self.HQ, self.HKV, self.D, self.F

        def rnd(*shape, scale=1.0):
            out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
            flat = out.view(-1)
            step = 1 << 28
            for o in range(0, flat.numel(), step):
                n = min(step, flat.numel() - o)
                flat[o:o + n] = (torch.randn(n, generator=g, device="cuda") * scale).to(torch.bfloat16)
            return out

        self.w = {"w_qkv": rnd((HQ + 2 * HKV) * D, H, scale=0.02), "w_o": rnd(H, HQ * D, scale=0.02),
                  "w_gate": rnd(F, H, scale=0.02), "w_up": rnd(F, H, scale=0.02), "w_down": rnd(H, F, scale=0.02),
                  "g_attn": torch.ones(H, dtype=torch.bfloat16, device="cuda"),
                  "g_ffn": torch.ones(H, dtype=torch.bfloat16, device="cuda")}
        self.n_pages = 128 * HKV * (16384 // self.PAGE + 1) + HKV * ((16384 + 10240) // self.PAGE + 1) + 1024
        self.pool = rnd(self.n_pages, 2, self.PAGE * D)
        self.perm = torch.randperm(self.n_pages, generator=g, device="cuda").to(torch.int32)
        self.x = rnd(self.MAX_ROWS, H)
        self.q = rnd(self.MAX_ROWS, HQ * D)
        self.out = torch.empty(self.MAX_ROWS, HQ * D, dtype=torch.bfloat16, device="cuda")
        self.shape = X.layer_shape(hidden=H, n_q_heads=HQ, n_kv_heads=HKV, head_dim=D, ffn_dim=F)
        self.weights = X.layer_weights(self.w)

    def tables(self, dec_ctx, chunk, prior):
        t, HKV, P = self.torch, self.HKV, self.PAGE
        n_d = len(dec_ctx)
        dmb = max([(c + 1 + P - 1) // P for c in dec_ctx], default=0)
        pmb = (prior + chunk + P - 1) // P if chunk else 0
        nd_pages = n_d * HKV * dmb
        dec_pages = self.perm[:nd_pages].view(n_d, HKV, dmb) if n_d else None
        pre_pages = self.perm[nd_pages:nd_pages + HKV * pmb].view(HKV, pmb) if chunk else None
        ctx = t.tensor(dec_ctx, dtype=t.int32, device="cuda") if n_d else None
        return ctx, dec_pages, dmb, pre_pages, pmb

    def layer_step(self, dec_ctx, chunk, prior):
        X = self.X
        ctx_t, dec_pages, _, pre_pages, _ = self.tables(dec_ctx, chunk, prior)
        M = chunk + len(dec_ctx)
        desc = X.batch_desc(x=self.x[:M], n_prefill_local=chunk, n_decode=len(dec_ctx), dec_ctx=ctx_t,
                            dec_pages=dec_pages, chunk_len=chunk, prior_len=prior, pre_pages=pre_pages)
        return X.LayerStep(self.ctx, self.shape, desc, self.weights, self.pool, self.n_pages,
                           keep=(ctx_t, dec_pages, pre_pages))

    def decode_call(self, dec_ctx):
        X, t = self.X, self.torch
        ctx_t, dec_pages, dmb, _, _ = self.tables(dec_ctx, 0, 0)
        n_d = len(dec_ctx)
        ws = t.empty(max(256, X.xp_decode_workspace_size(n_d, self.HQ, self.HKV, self.D, dmb, 0)),
                     dtype=t.uint8, device="cuda")
        keep = (ctx_t, dec_pages, ws)
        return lambda: X.xp_decode_attention(X.XP_BF16, self.q, self.pool, self.n_pages, self.PAGE, dec_pages,
                                             dmb, ctx_t, n_d, self.HQ, self.HKV, self.D, self.out, self.HQ * self.D,
                                             ws, 0) or keep

    def prefill_call(self, chunk, prior):
        X, t = self.X, self.torch
        _, _, _, pre_pages, pmb = self.tables([], chunk, prior)
        ws = t.empty(max(256, X.xp_prefill_workspace_size(self.HQ, self.HKV, self.D, prior, chunk)),
                     dtype=t.uint8, device="cuda")
        keep = (pre_pages, ws)
        return lambda: X.xp_prefill_attention(X.XP_BF16, self.q, self.pool, self.n_pages, self.PAGE, pre_pages,
                                              pmb, self.HQ, self.HKV, self.D, prior, chunk, 0, chunk, self.out,
                                              self.HQ * self.D, None, self.HQ * self.D, ws) or keep


def _mixed_batch(rnd):
    """A heterogeneous batch as the pages sample them for estimator accuracy (§8.5): a
    prefill chunk of 32-10K tokens (log-uniform) after 0-16K cached tokens, and 1-128
    decodes with contexts of 1K-16K tokens."""
    chunk = int(round(math.exp(rnd.uniform(math.log(32), math.log(10240)))))
    prior = rnd.randint(0, 16384)
    dec = [rnd.randint(1024, 16384) for _ in range(rnd.randint(1, 128))]
    return chunk, prior, dec


def multi_chunk_mode(args, X, torch, timer):
    """Several prefill requests in one step (xp_layer_forward_chunks): the step time in
    serialized split attention, and each chunk's prefill attention standalone."""
    from synth import MULTI_CHUNK_WORKLOADS, make_multi_instance
    from synth.device import make_chunked_step
    wl = MULTI_CHUNK_WORKLOADS[args.workload]
    t0 = time.time()
    inst = make_multi_instance(wl)
    ctx = X.Ctx(0, 0, 0)
    step = make_chunked_step(inst, ctx)
    log(f"[bench] {wl.name}: {wl.description}; rows {wl.n_rows}; inputs ready in {time.time() - t0:.1f} s")
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.2:
        step.run()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t1 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step.run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    ms = ev0.elapsed_time(ev1) / args.steps
    assert step.status() == 0
    lay = step.layout
    ws = int(step.workspace.data_ptr())
    hq, d = wl.n_q_heads, wl.head_dim
    out = torch.empty((max(l for l, _ in wl.chunks), hq * d), dtype=torch.bfloat16, device="cuda")
    pre, q_off = [], 0
    for (l, c), t in zip(wl.chunks, step.tables):
        pws = torch.empty(max(256, X.xp_prefill_workspace_size(hq, wl.n_kv_heads, d, c, l)), dtype=torch.uint8,
                          device="cuda")
        tt = timer(lambda: X.xp_prefill_attention(X.XP_BF16, ws + lay.q_pre + q_off, step.pool, inst.pool.n_pages,
                                                  wl.page_size, t, int(t.shape[1]), hq, wl.n_kv_heads, d, c, l, 0, l,
                                                  out, hq * d, None, hq * d, pws), args.repeats)
        fl = 4 * d * hq * (l * c + l * (l + 1) // 2)
        pre.append({"chunk": l, "prior": c, "us": round(tt * 1e6, 2), "TFLOPs": round(fl / tt / 1e12, 1)})
        q_off += l * hq * d * 2
    line = {"metric": METRIC, "value": round(wl.n_rows * args.steps / wall, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded, random-init weights)",
            "config": {"workload": f"{wl.name}: {wl.description}", "rows": wl.n_rows, "chunks": wl.chunks,
                       "decodes": wl.n_decode, "split_attention": "serialized"},
            "kernels": {"prefill_attn_chunks": pre}}
    log(f"[bench] layer {ms * 1e3:.1f} us/step; prefill chunks {json.dumps(pre)}")
    print(json.dumps(line), flush=True)
    ctx.close()


def stack_mode(args, X, torch):
    """One batch through a stack of layers (xp_stack_forward), eager and as piecewise graph
    launches (xp_stack_graph_create: the shared-linear segments in graphs, the attention
    region eager between them, ConfluxServe §6.1 Fig. 10).  Reports GPU time per step and
    per layer, and the host time to enqueue a step."""
    from synth import get_workload, make_stack_instance
    from synth.device import make_stack_step
    wl = get_workload(args.workload)
    t0 = time.time()
    sinst = make_stack_instance(wl, args.stack)
    decode_cus = args.decode_cus or 0
    ctx = X.Ctx(0, decode_cus, 0)
    step = make_stack_step(sinst, ctx)
    s = torch.cuda.current_stream()
    log(f"[bench] {wl.name} x {args.stack} layers: {wl.description}; inputs ready in {time.time() - t0:.1f} s")
    graph = step.capture(s)
    res = {}
    for name, fn in (("eager", lambda: step.run(s)), ("graph", lambda: graph.launch(s))):
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < 0.2:
            fn()
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t1 = time.perf_counter()
        ev0.record()
        for _ in range(args.steps):
            fn()
        enq = time.perf_counter() - t1
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t1
        us = ev0.elapsed_time(ev1) / args.steps * 1e3
        res[name] = {"us_per_step": round(us, 1), "us_per_layer": round(us / args.stack, 1),
                     "host_enqueue_us_per_step": round(enq / args.steps * 1e6, 1),
                     "tokens_per_s": round(wl.n_rows * args.steps / wall, 1)}
        log(f"[bench] {name}: {json.dumps(res[name])}")
    assert step.status() == 0
    graph.close()
    line = {"metric": METRIC, "value": res["graph"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["graph"]["us_per_step"] / 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
            "data": "synthetic (seeded, random-init weights)",
            "config": {"workload": f"{wl.name}: {wl.description}", "rows": wl.n_rows, "layers": args.stack,
                       "decode_cus": decode_cus, "timed": "graph launches (eager alongside)"},
            "stack": res}
    print(json.dumps(line), flush=True)
    ctx.close()


def estimator_mode(args, X, torch, timer):
    """Fit the latency model (ConfluxServe §6.2, App. D) from isolated profiles of this
    build's kernels, calibrate alpha and beta on heterogeneous layer steps, then report
    its mean absolute percentage error on fresh random heterogeneous batches (§8.5)."""
    import random
    t0 = time.time()
    ctx = X.Ctx(0, args.estimator_decode_cus, 0)
    rig = EstimatorRig(X, torch, ctx)
    log(f"[estimator] rig ready in {time.time() - t0:.1f} s: {rig.n_pages} pages, "
        f"decode CUs {args.estimator_decode_cus}")
    rec = {"gemm": [], "decode": [], "prefill": [], "mixed": [], "eval": []}
    n_rep = 8
    # shared linear region: decode-only steps of n rows with one-page contexts, minus the
    # standalone decode attention of the same rows
    for n in (16, 32, 48, 64, 96, 128, 192, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192,
              10368):
        dec = [15] * n
        step = rig.layer_step(dec, 0, 0)
        t_layer = timer(step.run, n_rep)
        t_dec = timer(rig.decode_call(dec), n_rep)
        assert step.status() == 0
        rec["gemm"].append((n, t_layer - t_dec))
    log(f"[estimator] shared-linear profile: {[(n, round(t * 1e6, 1)) for n, t in rec['gemm']]}")
    rnd = random.Random(7)
    for _ in range(32):
        dec = [rnd.randint(1024, 16384) for _ in range(rnd.randint(1, 128))]
        rec["decode"].append((sum(dec), timer(rig.decode_call(dec), n_rep)))
    for _ in range(32):
        chunk, prior = int(round(math.exp(rnd.uniform(math.log(32), math.log(10240))))), rnd.randint(0, 16384)
        w = chunk * prior + chunk * (chunk + 1) // 2
        rec["prefill"].append((w, timer(rig.prefill_call(chunk, prior), n_rep)))
    log(f"[estimator] attention profiles done ({time.time() - t0:.0f} s)")

    def run_mixed(rnd, n):
        out = []
        for _ in range(n):
            chunk, prior, dec = _mixed_batch(rnd)
            step = rig.layer_step(dec, chunk, prior)
            t = timer(step.run, n_rep)
            assert step.status() == 0
            out.append((chunk, prior, dec, t))
        return out

    def reduce(b):
        chunk, prior, dec, t = b
        return (chunk + len(dec), float(sum(dec)), float(chunk * prior + chunk * (chunk + 1) // 2), float(chunk), t)

    mixed = run_mixed(random.Random(11), 60)
    rec["mixed"] = [reduce(b) for b in mixed]
    model = X.xp_fit_latency_model(tuple(zip(*rec["gemm"])), tuple(zip(*rec["decode"])),
                                   tuple(zip(*rec["prefill"])), ([], []), rec["mixed"], n_layers=1, ab_max=4.0)
    log(f"[estimator] fitted {json.dumps(model)} ({time.time() - t0:.0f} s)")
    ev = run_mixed(random.Random(12), args.estimator_batches)

    def predict(b):
        chunk, prior, dec, _ = b
        return X.xp_iteration_latency(model, [len(dec)], [sum(dec)], [chunk], [(chunk, prior)])

    errs = [abs(predict(b) - b[3]) / b[3] for b in ev]
    cal = [abs(predict(b) - b[3]) / b[3] for b in mixed]
    rec["eval"] = [(b[0], b[1], len(b[2]), sum(b[2]), b[3], predict(b)) for b in ev]
    # the fitted model fed to the dispatcher: the TBT-safe chunk for the 8B decode batch
    # of the layer benchmark (16 decodes at 8192) under a 32-layer, 100 ms iteration
    m32 = dict(model, n_layers=32)
    wf = X.xp_waterfill(tau=0.100, n_decode_tokens=[16], decode_ctx_sum=[16 * 8192], candidate=(65536, 0),
                        model=m32)
    srt = sorted(errs)
    res = {"estimator": {
        "model": model, "mode": f"split attention on {args.estimator_decode_cus} decode CUs",
        "profiles": {k: len(rec[k]) for k in ("gemm", "decode", "prefill", "mixed")},
        "calibration_mape": round(sum(cal) / len(cal), 4), "eval_batches": len(ev),
        "eval_mape": round(sum(errs) / len(errs), 4), "eval_p50": round(srt[len(srt) // 2], 4),
        "eval_p90": round(srt[int(len(srt) * 0.9)], 4), "eval_max": round(srt[-1], 4),
        "dispatch_example": {"decodes": 16, "ctx": 8192, "tau_s": 0.100, "layers": 32,
                             "chunk_len": wf["chunk_len"], "n_target": wf["n_target"]},
        "seconds": round(time.time() - t0, 1)}}
    if args.estimator_out:
        with open(args.estimator_out, "w") as f:
            json.dump(dict(res, records=rec), f)
    print(json.dumps(res), flush=True)
    ctx.close()


def scheduler_timing(X, repeats: int = 100) -> dict:
    """Host time of one SLO-aware scheduling iteration (admission, ordering, one dispatch
    per chosen chunk, decode placement) on 8 simulated ranks, at the pending-queue depths
    the pages report (ConfluxServe §8.5, Table 5): mean and standard deviation over
    ``repeats`` calls of the native entry point, arguments marshalled once."""
    import dataclasses
    import statistics
    from synth import scheduler_case
    out = {"unit": "us", "ranks": 8, "repeats": repeats, "depths": {}}
    # one dispatch (Algorithm 2) on the same 8-rank state: a 4096-token candidate
    c = dataclasses.asdict(scheduler_case(10))
    wf = X.WaterfillCall(tau=c["tau"], n_decode_tokens=c["n_decode_tokens"], decode_ctx_sum=c["decode_ctx_sum"],
                         candidate=(4096, 0), quantum=c["quantum"], model=c["model"])
    for _ in range(10):
        wf.call()
    ts = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        wf.call()
        ts.append(time.perf_counter() - t0)
    out["waterfill_dispatch"] = {"mean": round(statistics.mean(ts) * 1e6, 2), "std": round(statistics.stdev(ts) * 1e6, 2),
                                 "chunk_len": wf.result()["chunk_len"]}
    for depth in (10, 50, 100, 500):
        c = dataclasses.asdict(scheduler_case(depth))
        c.pop("name")
        call = X.ScheduleCall(**c)
        for _ in range(10):
            call.call()
        ts = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            call.call()
            ts.append(time.perf_counter() - t0)
        r = call.result()
        out["depths"][depth] = {"mean": round(statistics.mean(ts) * 1e6, 1),
                                "std": round(statistics.stdev(ts) * 1e6, 1), "chunks": r["n_selected"],
                                "admitted": r["n_admitted"], "tokens": sum(r["prefill_assign"])}
    return out


def calibrate_decode_cus(X, torch, step, inst, dev, n_cus, repeats) -> tuple[int, dict]:
    """The pages' decode-CU rule, measured by the library (xp_calibrate_decode_cus): the
    fewest CUs, in steps of 32 (every shader engine of the 8 XCDs gains one), whose
    standalone decode-attention bandwidth is >= 90% of the all-CU figure."""
    wl = inst.wl
    lay = step.layout
    q = int(step.workspace.data_ptr()) + lay.q_dec
    dws = torch.empty(X.xp_decode_workspace_size(wl.n_decode, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, inst.dec_max_blocks,
                                                 lay.dec_pages_per_split), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.n_decode, wl.n_q_heads * wl.head_dim), dtype=torch.bfloat16, device="cuda")
    nbytes = decode_bytes(inst)
    k, curve = X.xp_calibrate_decode_cus(0, X.XP_BF16, q, dev.pool, inst.pool.n_pages, wl.page_size, dev.dec_pages,
                                         inst.dec_max_blocks, dev.dec_ctx, wl.n_decode, wl.n_q_heads,
                                         wl.n_kv_heads, wl.head_dim, out, wl.n_q_heads * wl.head_dim, dws,
                                         lay.dec_pages_per_split, keep_fraction=0.9, cu_step=32, repeats=repeats,
                                         stop_at_rule=False)
    torch.cuda.synchronize()
    gbs = {c: round(nbytes / (us * 1e-6) / 1e9, 1) for c, us in curve["points"].items()}
    return k, {"full_GBs": round(nbytes / (curve["us_all"] * 1e-6) / 1e9, 1), "curve_GBs": gbs}


def read_curve(X, torch, repeats) -> dict:
    """The streaming-read probe's bandwidth against the CUs it may use (xp_probe_read_curve
    over 2 GiB, 8x the Infinity Cache): the most HBM bandwidth a partition of k CUs can
    reach, the ceiling of the decode side of a CU partition."""
    big = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    c = X.xp_probe_read_curve(0, big, big.numel(), sink, cu_step=32, repeats=repeats)
    torch.cuda.synchronize()
    del big
    gb = (1 << 31) / 1e9
    return {"full_GBs": round(gb / (c["us_all"] * 1e-6), 1),
            "curve_GBs": {k: round(gb / (us * 1e-6), 1) for k, us in c["points"].items()}}


def kernel_calls(X, torch, inst, step, dev, plan_cus=0):
    """Launchers of the step's kernels on their own, through the C ABI, on the step's
    workspace (torch's current stream): name -> (call, algorithmic work, unit).  The
    prefill attention plans its key splits for plan_cus CUs (0: all of them), as the
    step's context does."""
    wl = inst.wl
    lay, ws, w = step.layout, int(step.workspace.data_ptr()), dev.weights
    M, H, F = wl.n_rows, wl.hidden, wl.ffn_dim
    gl = gemm_list(wl)
    gp, gpb = ws + lay.gemm_part, lay.h1 - lay.gemm_part     # the layer's GEMM split partials
    calls = {
        "qkv": lambda: X.xp_gemm(X.XP_BF16, X.XP_EPI_F32, ws + lay.hn, w["w_qkv"], None, None, ws + lay.qkv,
                                 M, gl["qkv"][1], H, gp, gpb),
        "o": lambda: X.xp_gemm(X.XP_BF16, X.XP_EPI_ADD_T, ws + lay.attn, w["w_o"], None, dev.x, ws + lay.h1,
                               M, H, gl["o"][2], gp, gpb),
        "gate_up": lambda: X.xp_gemm(X.XP_BF16, X.XP_EPI_SWIGLU, ws + lay.hn, w["w_gate"], w["w_up"], None,
                                     ws + lay.act, M, F, H, gp, gpb),
        "down": lambda: X.xp_gemm(X.XP_BF16, X.XP_EPI_ADD_F32, ws + lay.act, w["w_down"], None, ws + lay.h1,
                                  step.out, M, H, F, gp, gpb),
    }
    out = {k: (fn, 2.0 * gl[k][0] * gl[k][1] * gl[k][2], "flop") for k, fn in calls.items()}
    if wl.n_decode:
        dws = torch.empty(X.xp_decode_workspace_size(wl.n_decode, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                                     inst.dec_max_blocks, lay.dec_pages_per_split),
                          dtype=torch.uint8, device="cuda")
        dout = torch.empty((wl.n_decode, wl.n_q_heads * wl.head_dim), dtype=torch.bfloat16, device="cuda")

        def dec(stream=None):
            X.xp_decode_attention(X.XP_BF16, ws + lay.q_dec, dev.pool, inst.pool.n_pages, wl.page_size,
                                  dev.dec_pages, inst.dec_max_blocks, dev.dec_ctx, wl.n_decode, wl.n_q_heads,
                                  wl.n_kv_heads, wl.head_dim, dout, wl.n_q_heads * wl.head_dim, dws,
                                  lay.dec_pages_per_split, stream)
        dec._keep = (dws, dout)
        out["decode_attn"] = (dec, float(decode_bytes(inst)), "byte")
    if wl.chunk_len:
        hq, d = wl.hq_loc, wl.head_dim
        pout = torch.empty((wl.chunk_len, hq * d), dtype=torch.bfloat16, device="cuda")

        def pre(stream=None):
            X.xp_prefill_attention(X.XP_BF16, ws + lay.q_pre, dev.pool, inst.pool.n_pages, wl.page_size,
                                   dev.pre_pages, inst.pre_max_blocks, hq, wl.hkv_loc, d, wl.prior_len,
                                   wl.chunk_len, 0, wl.chunk_len, pout, hq * d, None, hq * d, ws + lay.pre_part,
                                   None, stream, plan_cus=plan_cus)
        pre._keep = (pout,)
        out["prefill_attn"] = (pre, float(prefill_flops(wl)), "flop")
    return out


def kernel_figures(name, seconds, work, unit) -> dict:
    r = {"us": round(seconds * 1e6, 2)}
    if unit == "byte":
        r.update(GBs=round(work / seconds / 1e9, 1), hbm_frac=round(work / seconds / 1e9 / PEAK_HBM_GBS, 4),
                 bytes=int(work))
    else:
        r.update(TFLOPs=round(work / seconds / 1e12, 1),
                 mfma_frac=round(work / seconds / 1e12 / PEAK_BF16_TFLOPS, 4), flops=work)
    return r


def window_times(X, torch, inst, step, dev, ctx, repeats) -> dict:
    """Decode and prefill attention inside the split region of a CU-partitioned (or
    unmasked) context, from the layer step itself: the library's stage events time each
    of the two on its own stream while the other one runs (the figures the pages'
    overlap rule is about: decode's bandwidth and prefill's MFMA rate while the other
    runs).  Both start at the step's fork, so the region lasts as long as the longer."""
    wl = inst.wl
    calls = kernel_calls(X, torch, inst, step, dev)
    _, dbytes, _ = calls["decode_attn"]
    _, pflops, _ = calls["prefill_attn"]
    for _ in range(repeats):
        step.run()
    torch.cuda.synchronize()
    ctx.stage_timing(repeats)
    for _ in range(repeats):
        step.run()
    torch.cuda.synchronize()
    st = ctx.stage_times()
    ctx.stage_timing(0)
    td = st["decode"][1] / max(st["decode"][0], 1) * 1e-3
    tp = st["prefill"][1] / max(st["prefill"][0], 1) * 1e-3
    return {"window_us": round(max(td, tp) * 1e6, 1), "decode_us": round(td * 1e6, 1),
            "decode_GBs": round(dbytes / td / 1e9, 1), "decode_hbm_frac": round(dbytes / td / 1e9 / PEAK_HBM_GBS, 4),
            "prefill_us": round(tp * 1e6, 1), "prefill_TFLOPs": round(pflops / tp / 1e12, 1),
            "prefill_mfma_frac": round(pflops / tp / 1e12 / PEAK_BF16_TFLOPS, 4)}


def extra_decode(X, torch, name, timer, repeats) -> dict:
    """Decode attention of another workload alone (its KV pool built on the device), for
    the HBM-bound figure on a decode-heavy batch."""
    from synth import get_workload, make_instance
    from synth.device import to_device, upload_pool
    wl = get_workload(name)
    inst = make_instance(wl)
    pool = upload_pool(inst)
    dec_pages, dec_ctx = to_device(inst.dec_pages, "i32"), to_device(inst.dec_ctx, "i32")
    q = (torch.randn((wl.n_decode, wl.n_q_heads * wl.head_dim), device="cuda")).to(torch.bfloat16)
    out = torch.empty_like(q)
    ws = torch.empty(X.xp_decode_workspace_size(wl.n_decode, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                                inst.dec_max_blocks, 0), dtype=torch.uint8, device="cuda")
    fn = lambda: X.xp_decode_attention(X.XP_BF16, q, pool, inst.pool.n_pages, wl.page_size, dec_pages,
                                       inst.dec_max_blocks, dec_ctx, wl.n_decode, wl.n_q_heads, wl.n_kv_heads,
                                       wl.head_dim, out, wl.n_q_heads * wl.head_dim, ws, 0)
    t = timer(fn, repeats)
    r = kernel_figures("decode_attn", t, float(decode_bytes(inst)), "byte")
    r["workload"] = f"{wl.name}: {wl.description}"
    del pool
    torch.cuda.empty_cache()
    return r


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU's share of the layer; this build has no "
                                   "multi-GPU path (run with --gpus 1)", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import mixed_prefill_decode_amd as X
    from synth import get_workload, load_instance, make_instance, save_instance
    from synth.device import make_step, upload

    torch.cuda.init()
    # Everything runs on a non-blocking stream: the context's CU-masked side
    # streams are blocking HIP streams, which the null stream would otherwise
    # wait on at every launch.
    torch.cuda.set_stream(torch.cuda.Stream())
    if args.estimator:
        return estimator_mode(args, X, torch, Timer(torch))
    if args.stack > 0:
        return stack_mode(args, X, torch)
    from synth import MULTI_CHUNK_WORKLOADS
    if args.workload in MULTI_CHUNK_WORKLOADS:
        return multi_chunk_mode(args, X, torch, Timer(torch))
    props = torch.cuda.get_device_properties(0)
    n_cus = props.multi_processor_count
    wl = get_workload(args.workload)
    t0 = time.time()
    inst = load_instance(args.instance_cache) if args.instance_cache else make_instance(wl)
    dev = upload(inst)
    log(f"[bench] {wl.name}: {wl.description}; rows {wl.n_rows}; pool {inst.pool.nbytes / 2**30:.2f} GiB; "
        f"inputs ready in {time.time() - t0:.1f} s on {props.name} ({n_cus} CUs)")
    timer = Timer(torch)

    # the iteration's dispatch: the chunk the waterfill gives this rank at the batch's level
    model = dict(gamma=2.0 ** -17, gamma0=2.0 ** -12, a_d=2.0 ** -27, a_d0=2.0 ** -13, a_p=2.0 ** -31,
                 a_p0=2.0 ** -13, a_comm=2.0 ** -20, a_comm0=2.0 ** -14, alpha=1.125, beta=1.25, n_layers=32)
    ctx_sum = int(np.sum(inst.dec_ctx.astype(np.int64)))
    wf_args = dict(tau=0.05, n_decode_tokens=[wl.n_decode], decode_ctx_sum=[ctx_sum],
                   candidate=(wl.n_prefill_local, wl.prior_len), model=model, fixed_target=wl.n_rows)

    if args.probe is not None:
        return probe_mode(args, X, torch, inst, dev, timer, n_cus)

    ctx0 = X.Ctx(0, 0, 0)
    step0, _ = make_step(inst, ctx0, dev)

    if args.kernel_only != "none":
        return kernel_only(args, X, torch, inst, step0, dev, timer)

    step0.run()
    torch.cuda.synchronize()
    # Split-attention mode.  The pages size the decode partition by their rule (the
    # fewest CUs that keep 90% of decode's standalone bandwidth).  The step is timed
    # serialized, with the two attention kernels concurrent on all CUs (no masks), on
    # a sweep of partitions and on the rule's; the timed steps use the fastest and
    # every figure is reported.  Each mode is timed in a fresh process whose first
    # streams are that context's (a context created after others in one process can
    # be slowed as a whole: its queues may share a hardware pipe with the main
    # stream's), so this process creates no masked context before the chosen one;
    # the probes map this process's inputs instead of drawing them again.
    seg = {}
    step, k, timed_mode = step0, 0, "serialized"
    cache = None
    try:
        if args.decode_cus is not None:
            k = args.decode_cus
            if k != 0:
                step, _ = make_step(inst, X.Ctx(0, k, 0), dev)
                timed_mode = "unmasked" if k < 0 else "partitioned"
        elif wl.n_decode and wl.chunk_len and not args.no_split_sweep:
            cache = tempfile.mkdtemp(prefix="xp_bench_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
            save_instance(inst, cache)
            rule = run_probe(args, "rule", cache)
            k_rule = rule["rule_decode_cus"]
            seg["rule_decode_cus"] = k_rule
            seg["calibration"] = rule["calibration"]
            seg["read_probe_curve"] = rule["read_curve"]
            seg["serialized_layer_us"] = round(timer(step0.run, args.repeats) * 1e6, 1)
            sweep, windows = {}, {}
            best = (seg["serialized_layer_us"], 0)
            for kk in sorted({-1, 64, 80, 96, 112, 128, 160, k_rule}):
                r = run_probe(args, str(kk), cache)
                t = r["layer_us"]
                sweep["unmasked" if kk < 0 else kk] = t
                windows["unmasked" if kk < 0 else kk] = r["window"]
                if t < best[0]:
                    best = (t, kk)
            seg["rule_layer_us"] = sweep[k_rule]
            seg["unmasked_layer_us"] = sweep["unmasked"]
            seg["partition_layer_us"] = {kk: v for kk, v in sweep.items() if kk != "unmasked"}
            seg["window"] = windows
            k = best[1]
            if k != 0:
                step, _ = make_step(inst, X.Ctx(0, k, 0), dev)
            timed_mode = "serialized" if k == 0 else "unmasked" if k < 0 else "partitioned"
            seg["decode_cus"] = k
            seg["timed_mode"] = timed_mode
    finally:
        if cache:
            shutil.rmtree(cache, ignore_errors=True)

    def one_step():
        r = X.xp_waterfill(**wf_args)
        assert r["chunk_len"] == wl.n_prefill_local
        step.run()

    # untimed steps until the clock has settled (not part of the W warmup steps)
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.2:
        step.run()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        one_step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    tokens_per_s = wl.n_rows * args.steps / wall
    assert step.status() == 0
    # The same steps again with the library's stage events (xp_ctx_stage_timing: HIP
    # events around each stage on the stream it runs on): the per-launch durations of the
    # kernels inside the step.  The events add a few microseconds between kernels (about
    # 5% of a C5 step), so this pass is not the one the step rate comes from.
    step.ctx.stage_timing(args.steps)
    ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev2.record()
    for _ in range(args.steps):
        one_step()
    ev3.record()
    torch.cuda.synchronize()
    stages = {name: round(t / n * 1e3, 2) for name, (n, t) in step.ctx.stage_times().items() if n}
    stages["step_with_events"] = round(ev2.elapsed_time(ev3) / args.steps * 1e3, 2)
    step.ctx.stage_timing(0)

    # per-kernel measurements (standalone, all CUs, HIP events on the launch stream)
    kern = {}
    calls = kernel_calls(X, torch, inst, step0, dev)
    for name, (fn, work, unit) in ([] if args.no_kernel_loops else calls.items()):
        kern[name] = kernel_figures(name, timer(fn, args.repeats), work, unit)
        if name in ("qkv", "o", "gate_up", "down"):
            m_, n_, k_ = gemm_list(wl)[name]
            kern[name]["weight_GBs"] = round(n_ * k_ * 2 / (kern[name]["us"] * 1e-6) / 1e9, 1)
    if "decode_attn" in kern:
        # measured streaming-read ceiling: one read of 2 GiB (8x the Infinity Cache)
        big = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        ceiling = big.numel() / timer(lambda: X.xp_probe_read(big, big.numel(), sink), 5) / 1e9
        del big
        kern["decode_attn"]["read_ceiling_GBs"] = round(ceiling, 1)
        kern["decode_attn"]["ceiling_frac"] = round(kern["decode_attn"]["GBs"] / ceiling, 4)

    if "serialized_layer_us" in seg and "decode_attn" in kern:
        # the attention segment alone: decode then prefill each on the whole GPU
        # (standalone kernel times above), the contention-free bound max(T_D, T_P), and
        # the overlapped modes' segment time, i.e. their layer time less the layer's
        # non-attention part (serialized layer time - T_D - T_P)
        td, tp = kern["decode_attn"]["us"], kern["prefill_attn"]["us"]
        rest = seg["serialized_layer_us"] - (td + tp)
        seg["attention_segment_us"] = {
            "serialized": round(td + tp, 1), "bound": round(max(td, tp), 1),
            "unmasked": round(seg["unmasked_layer_us"] - rest, 1),
            "partitions": {kk: round(v - rest, 1) for kk, v in seg["partition_layer_us"].items()}}

    # the roofline of the kernel that takes the most time in this workload's timed steps,
    # from its launches inside them (the stage events); the standalone loops above are
    # reported beside it
    in_step = {kn: stages[sn] for sn, kn in STAGE_KERNELS.items() if sn in stages and kn in calls}
    if not in_step:
        in_step = {kn: kern[kn]["us"] for kn in kern}
    dom = max(in_step, key=in_step.get)
    fn, work, unit = calls[dom]
    t_dom = in_step[dom] * 1e-6
    traffic = recorded_traffic(wl.name, dom)
    kname = CORES_KERNEL_NAMES.get(dom, KERNEL_NAMES[dom]) if timed_mode == "unmasked" else KERNEL_NAMES[dom]
    if unit == "byte":
        roofline = {"bound": "hbm", "achieved": round(work / t_dom / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(work / t_dom / 1e9 / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "kernel": kname, "bytes_per_launch": work, "launch_us": round(t_dom * 1e6, 2)}
    else:
        roofline = {"bound": "mfma", "achieved": round(work / t_dom / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(work / t_dom / 1e12 / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                    "kernel": kname, "flops_per_launch": work, "launch_us": round(t_dom * 1e6, 2)}
    log(f"[bench] layer {ms * 1e3:.1f} us/step, {tokens_per_s:.0f} tokens/s; kernels {json.dumps(kern)}")
    log(f"[bench] split attention {json.dumps(seg)}")

    extra = None
    if args.extra_decode != "none" and args.extra_decode != wl.name:
        extra = extra_decode(X, torch, args.extra_decode, timer, args.repeats)
        log(f"[bench] extra decode {json.dumps(extra)}")

    sched = scheduler_timing(X)
    log(f"[bench] scheduler {json.dumps(sched)}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inst, args.cpu_budget_s)
        log(f"[bench] cpu baseline {cpu}")
    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded, random-init weights)",
        "config": {"workload": f"{wl.name}: {wl.description}", "rows": wl.n_rows, "hidden": wl.hidden,
                   "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
                   "ffn": wl.ffn_dim, "decodes": wl.n_decode, "decode_ctx": wl.ctx[1] if wl.ctx[0] == "fixed" else list(wl.ctx),
                   "chunk": wl.chunk_len, "prior": wl.prior_len, "sp_degree": wl.sp_degree,
                   "decode_cus": k, "split_attention": timed_mode if wl.n_decode and wl.chunk_len else None,
                   "page_size": wl.page_size},
        "roofline": roofline, "cpu_baseline": cpu, "stages_us": stages, "kernels": kern, "extra_decode": extra,
        "split_attention": seg, "scheduler": sched,
    }
    print(json.dumps(line), flush=True)


def run_probe(args, what: str, cache: str) -> dict:
    """Runs this script with --probe in a child process (on the saved inputs) and
    returns its JSON line."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", args.workload, "--repeats", str(args.repeats),
           "--probe", what, "--instance-cache", cache]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"probe {what} failed ({r.returncode}):\n{r.stderr[-2000:]}")
    out = json.loads(r.stdout.strip().splitlines()[-1])
    log(f"[bench] probe {what}: {json.dumps(out)}")
    return out


def probe_mode(args, X, torch, inst, dev, timer, n_cus):
    """One split-attention mode in this fresh process: its context is the first one made."""
    from synth.device import make_step
    if args.probe == "rule":
        ctx0 = X.Ctx(0, 0, 0)
        step0, _ = make_step(inst, ctx0, dev)
        step0.run()
        torch.cuda.synchronize()
        k_rule, calib = calibrate_decode_cus(X, torch, step0, inst, dev, n_cus, args.repeats)
        rc = read_curve(X, torch, 5)
        print(json.dumps({"rule_decode_cus": k_rule, "calibration": calib, "read_curve": rc}), flush=True)
        ctx0.close()
        return
    k = int(args.probe)
    ctx = X.Ctx(0, k, 0)
    step, _ = make_step(inst, ctx, dev)
    for _ in range(3):
        step.run()
    torch.cuda.synchronize()
    t = timer(step.run, args.repeats)
    assert step.status() == 0
    win = window_times(X, torch, inst, step, dev, ctx, args.repeats)
    print(json.dumps({"decode_cus": k, "layer_us": round(t * 1e6, 1), "window": win}), flush=True)
    ctx.close()


def kernel_only(args, X, torch, inst, step, dev, timer):
    """Launch only one kernel repeatedly (input of counter-collection runs)."""
    step.run()
    torch.cuda.synchronize()
    if args.kernel_only == "copy":
        # a plain elementwise kernel (16-byte loads and stores per lane), not the runtime's
        # blit, whose counter readings differ from one runtime to the next
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)   # 1 GiB
        dst = torch.empty_like(src)
        fn = lambda: torch.mul(src, 1.0, out=dst)
        log("[bench] copy kernel: 1 GiB read + 1 GiB written per launch")
    elif args.kernel_only == "read":
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)   # 1 GiB
        sink = torch.empty(1 << 16, dtype=torch.float32, device="cuda")
        fn = lambda: X.xp_probe_read(src, src.numel() * 4, sink)
        log("[bench] read probe: 1 GiB read per launch")
    else:
        calls = kernel_calls(X, torch, inst, step, dev)
        if args.kernel_only not in calls:
            raise SystemExit(f"--kernel-only {args.kernel_only}: not part of {inst.wl.name}")
        fn = calls[args.kernel_only][0]
    t = timer(fn, args.repeats)
    torch.cuda.synchronize()
    log(f"[bench] {args.kernel_only}: {t * 1e6:.2f} us per launch over {args.repeats} launches")
    print(json.dumps({"kernel_only": args.kernel_only, "us": round(t * 1e6, 3), "repeats": args.repeats,
                      "src_sha256_16": sources_hash(args.kernel_only) if args.kernel_only not in ("copy", "read") else None}))


if __name__ == "__main__":
    main()
