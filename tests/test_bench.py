"""bench.py's host-side arithmetic and records (no GPU): the algorithmic work the roofline
divides by, the committed HBM-traffic records it reads, and its one-GPU guard."""
import glob
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from synth import PARITY_WORKLOADS, WORKLOADS, get_workload, make_instance

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _records():
    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
        text = open(path).read()
        if "```json" not in text:
            continue
        i = text.index("```json") + 7
        out.append((os.path.basename(path), json.loads(text[i:text.index("```", i)])))
    return out


@pytest.mark.parametrize("name", ["P1", "P4", "E2"])
def test_prefill_flops_count_the_causal_pairs(name):
    """4 d (Hq/P) per (query, key) pair the inclusive causal mask keeps (ConfluxServe Eq. 9),
    counted here by enumeration."""
    wl = get_workload(name)
    c, n = wl.prior_len, wl.chunk_len
    pairs = sum(1 for t in range(n) for k in range(c + n) if k <= c + t)
    assert bench.prefill_flops(wl) == 4 * wl.head_dim * wl.hq_loc * pairs


def test_prefill_flops_of_the_32b_chunk():
    # 4096 queries after 12288 cached keys, 8 heads of d = 128 on this rank
    assert bench.prefill_flops(get_workload("C5")) == 4 * 128 * 8 * (4096 * 12288 + 4096 * 4097 // 2)


@pytest.mark.parametrize("name", ["P2", "E1"])
def test_decode_bytes_read_each_visible_key_once(name):
    """Every K and V element of each request's c + 1 keys once for all heads of its group,
    q in and o out, and one table entry per visible page and kv head."""
    inst = make_instance(get_workload(name))
    wl = inst.wl
    eb = 2 if wl.dtype == "bf16" else 4
    want = 0
    for c in inst.dec_ctx.tolist():
        want += (c + 1) * 2 * wl.n_kv_heads * wl.head_dim * eb           # K and V
        want += 2 * wl.n_q_heads * wl.head_dim * eb                     # q in, o out
        want += len(range(0, c + 1, wl.page_size)) * wl.n_kv_heads * 4   # table entries
    assert bench.decode_bytes(inst) == want


def test_gemm_shapes_follow_the_layer():
    wl = get_workload("C5")
    g = bench.gemm_list(wl)
    assert g["qkv"] == (544, (64 + 16) * 128, 5120)
    assert g["o"] == (544, 5120, 64 * 128)
    assert g["gate_up"] == (544, 2 * 25600, 5120)
    assert g["down"] == (544, 5120, 25600)


def test_traffic_records_are_consistent():
    """Each committed record: scaled bytes = FETCH x read factor + WRITE x write factor (KiB),
    factors near the 2.0 / 1.0 a plain copy reads, a known kernel and workload, and the
    kernel's current sources (a record taken on other sources is not reported)."""
    recs = _records()
    assert recs, "no traffic records"
    names = set(WORKLOADS) | set(PARITY_WORKLOADS)
    for path, r in recs:
        scaled = (r["fetch_kib"] * r["fetch_factor"] + r["write_kib"] * r["write_factor"]) * 1024
        assert abs(scaled - r["traffic_bytes"]) <= 1e-6 * r["traffic_bytes"] + 1024, path
        assert 1.9 < r["fetch_factor"] < 2.1 and 0.95 < r["write_factor"] < 1.05, path
        assert r["workload"] in names, path
        assert r["src_sha256_16"] == bench.sources_hash(r["kernel"]), (
            f"{path} was taken on other {r['kernel']} sources: take its counters again")
        assert bench.recorded_traffic(r["workload"], r["kernel"]) == r["traffic_bytes"], path


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
