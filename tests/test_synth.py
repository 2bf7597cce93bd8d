"""The seeded input generators: determinism, table validity, NaN poisoning -- CPU only."""
import numpy as np

from tests.helpers import k_slots
from synth import (PARITY_WORKLOADS, WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, get_workload,
                   make_instance, waterfill_cases)


def test_generation_is_deterministic():
    a = make_instance(get_workload("P1"))
    b = make_instance(get_workload("P1"))
    assert np.array_equal(a.x, b.x) and np.array_equal(a.dec_pages, b.dec_pages)
    assert np.array_equal(a.pool.array, b.pool.array, equal_nan=True)
    for k in a.weights:
        assert np.array_equal(a.weights[k], b.weights[k])


def test_page_tables_cover_exactly_the_needed_blocks():
    for name in ("P1", "P2", "P3", "E1", "E2", "C1"):
        inst = make_instance(get_workload(name))
        wl, S = inst.wl, inst.wl.page_size
        used = []
        for i, c in enumerate(inst.dec_ctx):
            nb = -(-(int(c) + 1) // S)
            assert (inst.dec_pages[i, :, :nb] >= 0).all() and (inst.dec_pages[i, :, nb:] == -1).all()
            used += list(inst.dec_pages[i, :, :nb].ravel())
        if wl.chunk_len:
            nb = -(-(wl.prior_len + wl.chunk_len) // S)
            assert inst.pre_pages.shape == (wl.hkv_loc, nb) and (inst.pre_pages >= 0).all()
            used += list(inst.pre_pages.ravel())
        assert len(used) == len(set(used)), "a page is shared"
        assert max(used) < inst.pool.n_pages


def test_unwritten_slots_are_nan_and_cached_slots_finite():
    inst = make_instance(get_workload("P2"))
    S, d = inst.wl.page_size, inst.wl.head_dim
    for i, c in enumerate(inst.dec_ctx):
        for g in range(inst.wl.n_kv_heads):
            for pos in range(-(-(int(c) + 1) // S) * S):
                row = inst.pool[[inst.dec_pages[i, g, pos // S]]][0]
                k = bf16_bits_to_f32(k_slots(row[0], S, d, "bf16")[pos % S])
                v = bf16_bits_to_f32(row[1].reshape(d, S)[:, pos % S])
                assert np.isfinite(k).all() == (pos < c) and np.isfinite(v).all() == (pos < c)


def test_bank_pool_reads_like_a_materialised_pool():
    from dataclasses import replace
    wl = replace(get_workload("E1"), kv_bank_pages=5)
    inst = make_instance(wl)
    ids = np.arange(inst.pool.n_pages)
    rows = inst.pool[ids]
    assert np.array_equal(rows[~np.isin(ids, inst.pool.poisoned_pages())],
                          inst.pool.bank[inst.pool.bank_idx[ids]][~np.isin(ids, inst.pool.poisoned_pages())])


def test_bf16_conversion_roundtrip():
    v = np.array([1.0, -2.5, 3.14159, 1e-3, 65504.0], dtype=np.float32)
    assert np.allclose(bf16_bits_to_f32(f32_to_bf16_bits(v)), v, rtol=2 ** -8)


def test_workload_shapes_are_consistent():
    for wl in list(WORKLOADS.values()) + list(PARITY_WORKLOADS.values()):
        assert wl.n_q_heads % wl.n_kv_heads == 0
        assert wl.n_q_heads % wl.sp_degree == 0 and wl.n_kv_heads % wl.sp_degree == 0
        assert wl.hq_loc % wl.group == 0
        assert wl.chunk_len % wl.sp_degree == 0
    assert WORKLOADS["C2"].n_rows == 1040 and WORKLOADS["C3"].n_rows == 536
    assert WORKLOADS["C4"].n_rows == 128 and WORKLOADS["C5"].n_rows == 544
    assert len(waterfill_cases()) >= 3


def test_saved_instance_maps_back_identically(tmp_path):
    from synth import load_instance, save_instance
    inst = make_instance(get_workload("P1"))
    save_instance(inst, str(tmp_path))
    back = load_instance(str(tmp_path))
    assert back.wl == inst.wl
    for a, b in ((back.x, inst.x), (back.dec_ctx, inst.dec_ctx), (back.dec_pages, inst.dec_pages),
                 (back.pre_pages, inst.pre_pages), (back.peer_qkv_in, inst.peer_qkv_in),
                 (back.peer_attn_in, inst.peer_attn_in), (back.pool.array, inst.pool.array),
                 (back.pool.valid_slots, inst.pool.valid_slots)):
        assert np.array_equal(np.asarray(a), np.asarray(b))
    assert all(np.array_equal(back.weights[k], inst.weights[k]) for k in inst.weights)
