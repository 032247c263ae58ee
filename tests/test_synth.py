"""The seeded input generator: determinism, rounding and distributions."""
import numpy as np

from hybrid_linear_memory_amd import synth


def test_bf16_round_ties_to_even_and_exactness():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 65504.0], np.float32)
    r = synth.bf16_round(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert r[1] == np.float32(1.0)
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even is 1 + 2^-6
    assert r[2] == np.float32(1.015625)
    assert r[3] == np.float32(-2.5)
    # idempotent, low 16 bits clear
    np.testing.assert_array_equal(synth.bf16_round(r), r)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    g = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    rg = synth.bf16_round(g)
    assert np.max(np.abs(rg - g) / np.abs(g)) <= 2.0 ** -8


def test_determinism_and_independence():
    w = synth.WORKLOADS[0]
    a = synth.qkv(w, 3, 1)
    b = synth.qkv(w, 3, 1)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    c = synth.qkv(w, 3, 0)
    assert not np.array_equal(a[0], c[0])
    k2, v2 = synth.kv(w, 3, 1)
    np.testing.assert_array_equal(k2, a[1])
    np.testing.assert_array_equal(v2, a[2])
    q_rows = synth.qkv(w, 3, 1, rows=slice(5, 9))[0]
    np.testing.assert_array_equal(q_rows, a[0][:, :, 5:9])


def test_shapes_and_distributions():
    w = synth.WORKLOADS[1].replace(T=200, frames=2)
    q, k, v = synth.qkv(w, 0, 0)
    assert q.shape == (1, 12, 200, 128) and q.dtype == np.float32
    np.testing.assert_array_equal(synth.bf16_round(q), q)
    n = np.linalg.norm(k.astype(np.float64), axis=-1)
    np.testing.assert_allclose(n, 1.0, atol=2e-2)
    beta, alpha = synth.gates(w, 0)
    assert beta.shape == (1, 12, 200) and alpha.shape == (1, 12)
    assert np.all(beta > 0) and np.all(beta < 1.0 / 200)
    assert np.all((alpha > 0) & (alpha < 1)) and alpha.mean() > 0.8
    pq, pk, pv = synth.phi_maps(w)
    assert pq.shape == (12, 128, 128)
    assert abs(pq.std() - 1 / np.sqrt(128)) < 0.01
    w0 = synth.WORKLOADS[0]
    p0 = synth.phi_maps(w0)[0]
    assert abs(np.mean(np.diagonal(p0, axis1=1, axis2=2)) - 1.0) < 0.1


def test_stress_logit_spread():
    w = synth.WORKLOADS[1].replace(T=256, H=2)
    q, k, _ = synth.stress_qkv(w, 0, 0, logit_std=3.0)
    logits = (q[0, 0].astype(np.float64) @ k[0, 0].T.astype(np.float64)) / np.sqrt(128)
    assert 2.5 < logits.std() < 3.5
