"""Pins of oracle.layer.stack_forward (a layer stack over one batch, ConfluxServe §4
Fig. 7 layer after layer) -- CPU only.

Pinned by: a one-layer stack is the layer step itself; a layer whose output and down
projections are zero is the identity on the residual stream, so a stack ending in one
returns the previous layer's output as stored (float32) bit for bit; an fp32 copy of
a bf16 input gives the same step; each layer appends only to its own pool.
"""
import numpy as np

from oracle import layer as L
from synth import get_workload, make_stack_instance
from tests.helpers import oracle_kwargs, stack_oracle_kwargs


def test_one_layer_stack_is_the_layer_step():
    s = make_stack_instance(get_workload("P2"), 1)
    one = L.layer_forward(**oracle_kwargs(s.base))
    st = L.stack_forward(**stack_oracle_kwargs(s))
    assert np.array_equal(st["out"], one["out"])


def test_zero_output_projections_make_an_identity_layer():
    s = make_stack_instance(get_workload("P2"), 2)
    w1 = dict(s.layers[1]["weights"])
    w1["w_o"] = np.zeros_like(w1["w_o"])
    w1["w_down"] = np.zeros_like(w1["w_down"])
    s.layers[1] = {"weights": w1, "pool": s.layers[1]["pool"]}
    st = L.stack_forward(**stack_oracle_kwargs(s))
    first = L.layer_forward(**oracle_kwargs(s.base))["out"]
    assert np.array_equal(st["out"], first.astype(np.float32).astype(np.float64))
    assert np.array_equal(st["layers"][0]["out"], first)


def test_fp32_input_of_bf16_values_gives_the_same_step():
    s = make_stack_instance(get_workload("P2"), 1)
    kw = oracle_kwargs(s.base)
    a = L.layer_forward(**kw)
    x32 = (s.base.x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    b = L.layer_forward(**dict(kw, x=x32, x_dtype="f32"))
    assert np.array_equal(a["out"], b["out"])


def test_each_layer_appends_to_its_own_pool():
    s = make_stack_instance(get_workload("P2"), 2)
    st = L.stack_forward(**stack_oracle_kwargs(s))
    kv0, kv1 = st["layers"][0]["kv"], st["layers"][1]["kv"]
    assert kv0.pool is s.layers[0]["pool"] and kv1.pool is s.layers[1]["pool"]
    assert set(kv0.overlay) == set(kv1.overlay) and kv0.overlay
    # same slots, different appended values (different weights and inputs)
    p = sorted(kv0.overlay)[0]
    assert not np.array_equal(kv0.stored_page(p), kv1.stored_page(p))
