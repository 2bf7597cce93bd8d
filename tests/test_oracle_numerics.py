"""Pins of oracle.numerics (storage rounding) and the elementwise pieces -- CPU only."""
import numpy as np
import torch

from oracle import layer as L
from oracle.numerics import encode, round_f64, to_f64


def _torch_bf16_bits(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_library_conversion():
    r = np.random.default_rng(0)
    v = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40, 2.0 ** -133]])
    # exact ties at the bf16 rounding point: 1 + 2^-8 (ties to even -> 1), 1 + 3*2^-8 -> 1 + 2^-6
    v = np.concatenate([v, [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]])
    ours = encode(round_f64(v, "bf16"), "bf16")
    assert np.array_equal(ours, _torch_bf16_bits(v))
    assert np.array_equal(to_f64(ours, "bf16"), round_f64(v, "bf16"))


def test_f32_rounding_is_ieee_rne():
    r = np.random.default_rng(1)
    v = r.standard_normal(1000) * 1e3
    assert np.array_equal(round_f64(v, "f32"), v.astype(np.float32).astype(np.float64))


def test_rope_properties():
    r = np.random.default_rng(2)
    v = r.standard_normal((5, 3, 64))
    assert np.array_equal(L.rope(v, np.zeros(5), 10000.0), v)                       # identity at 0
    pos = r.integers(0, 70000, 5)
    w = L.rope(v, pos, 10000.0)
    assert np.allclose(np.linalg.norm(w, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-13)
    # <R(q, m), R(k, n)> depends only on m - n
    q, k = r.standard_normal((1, 1, 64)), r.standard_normal((1, 1, 64))
    dots = [np.sum(L.rope(q, np.array([m + s]), 1e4) * L.rope(k, np.array([7 + s]), 1e4))
            for m, s in ((20, 0), (20, 1000), (20, 54321))]
    assert np.allclose(dots, dots[0], rtol=1e-9)
    # pairing is (i, i + d/2): a vector living in dims {0, 32} rotates within them
    e = np.zeros((1, 1, 64)); e[0, 0, 0] = 1.0
    out = L.rope(e, np.array([1]), 10000.0)[0, 0]
    assert np.isclose(out[0], np.cos(1.0)) and np.isclose(out[32], np.sin(1.0))
    assert np.count_nonzero(out) == 2


def test_rmsnorm_and_silu():
    r = np.random.default_rng(3)
    x = r.standard_normal((4, 256)) * 7
    y = L.rmsnorm(x, np.ones(256), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-14)
    assert np.allclose(L.rmsnorm(3.5 * x, np.ones(256), 0.0), y, atol=1e-14)        # scale-free
    g = r.standard_normal(256)
    assert np.allclose(L.rmsnorm(x, g, 1e-5), L.rmsnorm(x, np.ones(256), 1e-5) * g)
    z = r.standard_normal(1000) * 20
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    assert np.allclose(L.silu(z), ref, atol=1e-14, rtol=1e-14)
    assert L.silu(np.array([0.0]))[0] == 0.0
