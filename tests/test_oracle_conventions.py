"""Pins of the oracle's convention flags ("Forward Cuda Gemma", decodeBatch:
"per-head V/Q/K norm"; the variants a model may use: interleaved RoPE pairs
and (1 + w) norm weights).

Each variant is tied to the default convention, which the other pin files fix
to closed forms: interleaved RoPE is rotate-half conjugated by the even/odd
permutation, (1 + w) with w = 0 is the unit-weight norm, and V-norm writes the
weightless RMSNorm of the value, which a one-key step returns unchanged.
"""
import math

import numpy as np
import pytest

import oracle
from sequence_slot_kv_amd import workloads as wl


def perm(D):
    """Even/odd permutation: (x0, x1, x2, x3, ...) -> (x0, x2, ..., x1, x3, ...)."""
    return np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])


def layer(rng, H, Hkv, D, flags, sinks=False):
    return wl.LayerParams(
        n_heads=H, n_kv_heads=Hkv, head_dim=D,
        q_norm_w=(1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
        k_norm_w=(1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
        inv_freq=wl.rope_inv_freq(1e4, D),
        sinks=rng.standard_normal(H).astype(np.float32) if sinks else None,
        eps=1e-6, scale=float(np.float32(1 / math.sqrt(D))), flags=flags)


def test_interleaved_rope_is_rotate_half_of_the_even_odd_permutation():
    rng = np.random.default_rng(1)
    D = 16
    P = perm(D)
    inv = wl.rope_inv_freq(1e4, D)
    for pos in (0, 1, 7, 1000):
        x = rng.standard_normal(D)
        y = oracle.rope_interleaved(x, inv, pos)
        z = oracle.rope(x[P], inv, pos)
        assert np.array_equal(y[P], z)


def test_interleaved_rope_rotates_the_first_pair():
    D = 8
    inv = np.array([0.5, 0.25, 0.125, 0.0625], np.float32)
    e0 = np.zeros(D)
    e0[0] = 1.0
    y = oracle.rope_interleaved(e0, inv, 3)
    th = float(np.float32(3.0) * np.float32(0.5))
    np.testing.assert_allclose(y, [math.cos(th), math.sin(th), 0, 0, 0, 0, 0, 0], atol=1e-15)
    assert np.array_equal(oracle.rope_interleaved(e0, inv, 0), e0)


def test_one_plus_w_norm():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(32).astype(np.float32)
    zero, ones = np.zeros(32, np.float32), np.ones(32, np.float32)
    assert np.array_equal(oracle.rms_norm_1pw(x, zero, 1e-6), oracle.rms_norm(x, ones, 1e-6))
    c, eps = 3.0, 1e-3
    w = rng.standard_normal(32).astype(np.float32)
    y = oracle.rms_norm_1pw(np.full(32, c, np.float32), w, eps)
    np.testing.assert_allclose(y, c / math.sqrt(c * c + eps) * (1 + w.astype(np.float64)), rtol=1e-14)


def test_plain_norm():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(64).astype(np.float32)
    y = oracle.rms_norm_plain(x, 0.0)
    np.testing.assert_allclose(np.mean(y * y), 1.0, rtol=1e-13)
    np.testing.assert_allclose(y / np.linalg.norm(y), x / np.linalg.norm(x.astype(np.float64)), rtol=1e-12)


def _row(L, pos, rng, hist=None):
    D, H, kvd = L.head_dim, L.n_heads, L.kv_dim
    q = rng.standard_normal(H * D).astype(np.float32)
    k = rng.standard_normal(kvd).astype(np.float32)
    v = rng.standard_normal(kvd).astype(np.float32)
    hk = rng.standard_normal((pos, kvd)).astype(np.float32) if hist is None else hist[0]
    hv = rng.standard_normal((pos, kvd)).astype(np.float32) if hist is None else hist[1]
    return q, k, v, hk, hv


def test_decode_row_interleaved_equals_default_on_permuted_heads():
    rng = np.random.default_rng(4)
    H, Hkv, D, pos = 4, 2, 8, 5
    Li = layer(rng, H, Hkv, D, oracle.ROPE_INTERLEAVED, sinks=True)
    P = perm(D)
    Ld = wl.LayerParams(**{**Li.__dict__, "flags": 0, "q_norm_w": Li.q_norm_w[P],
                           "k_norm_w": Li.k_norm_w[P]})
    q, k, v, hk, hv = _row(Li, pos, rng)
    heads = lambda a, n: a.reshape(n, D)[:, P].reshape(-1)
    hkp = hk.reshape(pos, Hkv, D)[:, :, P].reshape(pos, -1)
    kw_i, vw_i, out_i = oracle.decode_row(Li, pos, q, k, v, hk, hv)
    kw_d, vw_d, out_d = oracle.decode_row(Ld, pos, heads(q, H), heads(k, Hkv), v, hkp, hv)
    assert np.array_equal(heads(kw_i, Hkv), kw_d)  # the written key, permuted
    assert np.array_equal(vw_i, vw_d)
    np.testing.assert_allclose(out_i, out_d, rtol=1e-6, atol=1e-7)  # V is not permuted


def test_decode_row_one_plus_w_equals_shifted_weights():
    rng = np.random.default_rng(5)
    L1 = layer(rng, 4, 2, 8, oracle.NORM_ONE_PLUS_W)
    L0 = wl.LayerParams(**{**L1.__dict__, "flags": 0,
                           "q_norm_w": (1 + L1.q_norm_w.astype(np.float64)).astype(np.float32),
                           "k_norm_w": (1 + L1.k_norm_w.astype(np.float64)).astype(np.float32)})
    q, k, v, hk, hv = _row(L1, 6, rng)
    a = oracle.decode_row(L1, 6, q, k, v, hk, hv)
    b = oracle.decode_row(L0, 6, q, k, v, hk, hv)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-6, atol=1e-7)
    assert not np.array_equal(a[0], oracle.decode_row(
        wl.LayerParams(**{**L1.__dict__, "flags": 0}), 6, q, k, v, hk, hv)[0])


def test_decode_row_v_norm_writes_normalised_value_and_returns_it_at_pos_zero():
    rng = np.random.default_rng(6)
    H, Hkv, D = 4, 2, 8
    L = layer(rng, H, Hkv, D, oracle.V_NORM)
    q, k, v, hk, hv = _row(L, 0, rng)
    kw, vw, out = oracle.decode_row(L, 0, q, k, v, hk, hv)
    for j in range(Hkv):
        ref = oracle.rms_norm_plain(v[j * D:(j + 1) * D], L.eps).astype(np.float32)
        assert np.array_equal(vw[j * D:(j + 1) * D], ref)
    G = H // Hkv
    for h in range(H):  # one key: the output is the written value of the head's kv head
        assert np.array_equal(out[h * D:(h + 1) * D], vw[(h // G) * D:(h // G + 1) * D])
    # the key is unaffected by V-norm
    L0 = wl.LayerParams(**{**L.__dict__, "flags": 0})
    assert np.array_equal(kw, oracle.decode_row(L0, 0, q, k, v, hk, hv)[0])
