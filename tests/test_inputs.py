"""The seeded generator: distributions, shapes and determinism (CPU only)."""
import numpy as np

import kda_inputs as ki


def test_configs_shapes():
    c = ki.headline_configs()
    assert c[0].total_tokens == 256 and c[0].dtype == "f32" and c[0].d_k == 64
    assert c[1].total_tokens == 4 * 4096 and c[1].n_heads == 16
    assert c[2].total_tokens == 65536 and c[2].n_heads == 32 and c[2].s0_std == 0.02
    assert c[4].total_tokens == 1 << 20 and c[4].window == 8192
    L = np.array(c[3].lengths)
    assert len(L) == 64 and L.min() >= 512 and L.max() <= 16384
    assert np.all(L % 16 != 0)
    assert np.all(np.cumsum(L)[:-1] % 16 != 0)


def test_distributions_and_determinism():
    s = ki.custom("t", "bf16", [300, 77], 3, 32, s0_std=0.02, pin_frac=0.25)
    a = ki.generate_numpy(s)
    b = ki.generate_numpy(s)
    for x, y in zip((a.q, a.k, a.v, a.beta, a.g, a.S0), (b.q, b.k, b.v, b.beta, b.g, b.S0)):
        assert np.array_equal(x, y)
    assert a.g.max() < 0 and a.g.min() >= -5.0
    assert a.beta.min() > 0 and a.beta.max() < 1
    assert np.allclose(np.linalg.norm(a.q, axis=-1), 1.0, atol=1e-2)
    assert np.allclose(np.linalg.norm(a.k, axis=-1), 1.0, atol=1e-2)
    assert np.array_equal(ki.round_bf16(a.v), a.v)          # bf16-exact values
    assert a.pinned.sum(axis=1).tolist() == [8, 8, 8]
    assert np.all(a.g[:, a.pinned] == -5.0)
    assert a.cu_seqlens.tolist() == [0, 300, 377]


def test_round_bf16():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.0e38, 1e-40], dtype=np.float32)
    r = ki.round_bf16(x)
    assert r[0] == 1.0 and r[1] == 1.0        # tie to even
    assert r[2] == np.float32(1.0078125)
    assert np.array_equal(ki.round_bf16(r), r)
