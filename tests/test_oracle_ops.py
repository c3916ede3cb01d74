"""Pins for oracle.ops -- closed forms, invariants and brute force (CPU only)."""
import math

import numpy as np
import pytest

from oracle import ops

rng = np.random.default_rng(1234)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_hand_value():
    y = ops.rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    r = math.sqrt((9 + 16) / 2)
    assert np.allclose(y, [3 / r, 8 / r], rtol=1e-15)


def test_rmsnorm_unit_rms_before_gain():
    x = rng.standard_normal((5, 300)) * 3.0
    eps = 1e-6
    y = ops.rmsnorm(x, np.ones(300), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-12)


def test_rmsnorm_scale_invariance_and_gain_is_elementwise():
    x = rng.standard_normal(64)
    w = 1 + 0.1 * rng.standard_normal(64)
    a = ops.rmsnorm(x, w, 1e-12)
    b = ops.rmsnorm(7.5 * x, w, 1e-12)
    assert np.allclose(a, b, rtol=1e-10)
    assert np.allclose(ops.rmsnorm(x, w, 1e-12), ops.rmsnorm(x, np.ones(64), 1e-12) * w, rtol=1e-14)


def test_rmsnorm_no_mean_subtraction():
    x = np.full(8, 5.0)
    assert np.allclose(ops.rmsnorm(x, np.ones(8), 0.0), np.ones(8))


# ---------------------------------------------------------------- RoPE
def test_inv_freq_closed_form():
    f = ops.rope_inv_freq(10000.0, 4)
    assert f.dtype == np.float32
    assert f[0] == 1.0 and f[1] == np.float32(0.01)
    f = ops.rope_inv_freq(1e6, 128)
    assert f[0] == 1.0
    assert f[32] == np.float32(1e6 ** -0.5)


def test_rope_zero_position_is_identity():
    x = rng.standard_normal((3, 1, 64))
    ang = ops.rope_angles([0], ops.rope_inv_freq(1e4, 64))
    assert np.array_equal(ops.apply_rope(x, ang), x)


def test_rope_head_dim_two_is_plane_rotation():
    # hd = 2: one pair, inv_freq[0] = 1, so the angle is the position itself
    x = np.array([[[0.3, -1.1]]])
    for p in [1, 5, 100]:
        y = ops.apply_rope(x, ops.rope_angles([p], ops.rope_inv_freq(1e4, 2)))
        c, s = math.cos(p), math.sin(p)
        assert np.allclose(y[0, 0], [0.3 * c + 1.1 * s, 0.3 * s - 1.1 * c], rtol=1e-14)


def test_rope_preserves_pair_norms():
    hd = 128
    x = rng.standard_normal((4, 7, hd))
    pos = np.arange(100, 107)
    y = ops.apply_rope(x, ops.rope_angles(pos, ops.rope_inv_freq(1e6, hd)))
    n_in = x[..., :64] ** 2 + x[..., 64:] ** 2
    n_out = y[..., :64] ** 2 + y[..., 64:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-12)


def test_rope_relative_position():
    hd = 64
    f = ops.rope_inv_freq(1e4, hd)
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))

    def dot(pq, pk):
        a = ops.apply_rope(q, ops.rope_angles([pq], f))
        b = ops.apply_rope(k, ops.rope_angles([pk], f))
        return float(np.sum(a * b))

    for (pq, pk, s) in [(5, 2, 3), (9, 9, 4), (12, 1, 2)]:
        assert math.isclose(dot(pq, pk), dot(pq + s, pk + s), rel_tol=1e-5, abs_tol=1e-6)


def test_rope_pairs_d_with_d_plus_half():
    # only element 0 set: rotation moves it into element half, nothing else
    hd = 8
    x = np.zeros((1, 1, hd))
    x[0, 0, 0] = 1.0
    y = ops.apply_rope(x, ops.rope_angles([1], ops.rope_inv_freq(1e4, hd)))
    assert np.allclose(y[0, 0], [math.cos(1), 0, 0, 0, math.sin(1), 0, 0, 0], atol=1e-15)


# ---------------------------------------------------------------- softmax
def test_softmax_rows_sum_to_one_and_shift_invariant():
    s = rng.standard_normal((6, 40)) * 10
    p = ops.softmax(s)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=1e-14)
    assert np.allclose(ops.softmax(s + 123.0), p, rtol=1e-12)


def test_softmax_masked_entries_get_zero():
    p = ops.softmax(np.array([1.0, -np.inf, 3.0]))
    assert p[1] == 0.0 and math.isclose(p.sum(), 1.0)


# ---------------------------------------------------------------- attention
def brute_attention(q, k, v, q_pos, window):
    """Pure-python triple loop over heads, queries, keys."""
    nh, T, hd = q.shape
    nkv = k.shape[0]
    out = np.zeros_like(q)
    for h in range(nh):
        g = h // (nh // nkv)
        for i in range(T):
            p = q_pos[i]
            keys = [j for j in range(k.shape[1]) if j <= p and (window <= 0 or j > p - window)]
            sc = [sum(q[h, i, d] * k[g, j, d] for d in range(hd)) / math.sqrt(hd) for j in keys]
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            z = sum(e)
            for d in range(hd):
                out[h, i, d] = sum(e[t] * v[g, keys[t], d] for t in range(len(keys))) / z
    return out


@pytest.mark.parametrize("nh,nkv,hd,T,past,window", [
    (2, 2, 2, 4, 0, 0), (4, 2, 4, 5, 3, 0), (4, 1, 2, 6, 2, 0), (4, 2, 4, 6, 4, 3), (2, 1, 4, 8, 0, 2),
])
def test_attention_matches_brute_force(nh, nkv, hd, T, past, window):
    q = rng.standard_normal((nh, T, hd))
    k = rng.standard_normal((nkv, past + T, hd))
    v = rng.standard_normal((nkv, past + T, hd))
    pos = np.arange(past, past + T)
    got = ops.attention(q, k, v, pos, window)
    assert np.allclose(got, brute_attention(q, k, v, pos, window), rtol=1e-12, atol=1e-14)


def test_attention_zero_query_is_running_mean():
    k = rng.standard_normal((1, 6, 4))
    v = rng.standard_normal((1, 6, 4))
    got = ops.attention(np.zeros((2, 6, 4)), k, v, np.arange(6))
    for i in range(6):
        assert np.allclose(got[0, i], v[0, :i + 1].mean(axis=0), rtol=1e-13)
        assert np.allclose(got[1, i], v[0, :i + 1].mean(axis=0), rtol=1e-13)


def test_attention_gqa_is_repeat_not_tile():
    # kv head 0 and kv head 1 hold distinct constant V; with 4 q heads, heads 0,1 -> kv 0
    k = np.zeros((2, 3, 2))
    v = np.stack([np.full((3, 2), 1.0), np.full((3, 2), 2.0)])
    got = ops.attention(rng.standard_normal((4, 3, 2)), k, v, np.arange(3))
    assert np.allclose(got[0], 1.0) and np.allclose(got[1], 1.0)
    assert np.allclose(got[2], 2.0) and np.allclose(got[3], 2.0)


def test_attention_single_key_returns_v():
    v = rng.standard_normal((1, 5, 4))
    got = ops.attention(rng.standard_normal((1, 5, 4)), rng.standard_normal((1, 5, 4)), v, np.arange(5), window=1)
    assert np.allclose(got[0], v[0], rtol=1e-15)


def test_attention_wide_window_equals_causal():
    q = rng.standard_normal((2, 7, 4))
    k = rng.standard_normal((1, 7, 4))
    v = rng.standard_normal((1, 7, 4))
    assert np.array_equal(ops.attention(q, k, v, np.arange(7), 7), ops.attention(q, k, v, np.arange(7), 0))


def test_window_boundary():
    ok = ops.allowed_keys([10], 11, 4)
    assert list(np.nonzero(ok[0])[0]) == [7, 8, 9, 10]


# ---------------------------------------------------------------- activations
def test_silu_closed_form():
    assert ops.silu(0.0) == 0.0
    for x in [-3.0, -0.5, 0.7, 4.0]:
        assert math.isclose(float(ops.silu(x)), x / (1 + math.exp(-x)), rel_tol=1e-15)
    assert math.isclose(float(ops.silu(1.0)), 1 / (1 + math.exp(-1)), rel_tol=1e-15)


def test_gelu_tanh_identities():
    assert ops.gelu_tanh(0.0) == 0.0
    x = np.linspace(-6, 6, 101)
    assert np.allclose(ops.gelu_tanh(x) - ops.gelu_tanh(-x), x, rtol=1e-14, atol=1e-14)
    # far tails: gelu_tanh(x) -> x for large x, -> 0 for very negative x
    assert math.isclose(float(ops.gelu_tanh(10.0)), 10.0, rel_tol=1e-15)
    assert abs(float(ops.gelu_tanh(-10.0))) < 1e-15


def test_gelu_tanh_differs_from_erf_gelu():
    # the two GELUs differ by a few 1e-4 near |x| ~ 2.7: a test there tells them apart
    d = abs(float(ops.gelu_tanh(2.7)) - float(ops.gelu_erf(2.7)))
    assert 1e-4 < d < 1e-3


def test_argmax_first_on_ties_and_nan():
    assert ops.argmax_first([1.0, 3.0, 3.0, 2.0]) == 1
    assert ops.argmax_first([0.0, -0.0]) == 0
    assert ops.argmax_first([1.0, np.nan, 5.0, np.nan]) == 1
