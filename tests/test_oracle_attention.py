"""Pins of the oracle's attention and LSE merge (CPU only).

Closed forms of softmax attention, an independent library attention
(torch scaled_dot_product_attention in float64 on the CPU, with the one
latent KV head broadcast to every query head), scipy's logsumexp, and the
defining invariant of the method: merging the per-shard partials of any
partition of the attended tokens gives full-context attention.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention

SCALE = 1.0 / np.sqrt(192.0)


def _rand(rng, H, T, dk=576, dv=512):
    q = rng.standard_normal((H, dk))
    k = rng.standard_normal((T, dk))
    return q, k, k[:, :dv].copy()


def _sdpa(q, k, v, scale):
    qt = torch.from_numpy(q)[None, :, None, :]             # [1, H, 1, Dk]
    kt = torch.from_numpy(k)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(v)[None, None].expand(1, q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, :, 0].numpy()


@pytest.mark.parametrize("H,T", [(1, 1), (4, 7), (16, 300), (64, 33)])
def test_matches_library_attention(H, T):
    rng = np.random.default_rng(H * 1000 + T)
    q, k, v = _rand(rng, H, T)
    o, lse = attention.attend(q, k, v, SCALE)
    assert np.allclose(o, _sdpa(q, k, v, SCALE), atol=1e-12, rtol=1e-12)
    assert np.allclose(lse, logsumexp(SCALE * (q @ k.T), axis=1), atol=1e-12)


def test_value_is_latent_part_only():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 3, 20)
    o, _ = attention.attend(q, k, v, SCALE)
    assert o.shape == (3, 512)
    k2 = k.copy()
    k2[:, 512:] = 0.0  # rope changes scores only
    o2, _ = attention.attend(q, k2, k2[:, :512], SCALE)
    assert not np.allclose(o, o2)


def test_single_token():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 5, 1)
    o, lse = attention.attend(q, k, v, SCALE)
    assert np.allclose(o, np.broadcast_to(v[0], o.shape), atol=0)
    assert np.allclose(lse, SCALE * (q @ k[0]), atol=1e-13)


def test_identical_keys():
    rng = np.random.default_rng(7)
    q, k, _ = _rand(rng, 4, 1)
    L = 37
    kk = np.repeat(k, L, axis=0)
    o, lse = attention.attend(q, kk, kk[:, :512], SCALE)
    assert np.allclose(o, np.broadcast_to(k[0, :512], o.shape), atol=1e-13)
    assert np.allclose(lse, SCALE * (q @ k[0]) + np.log(L), atol=1e-12)


def test_zero_query_is_mean_and_log_count():
    rng = np.random.default_rng(8)
    _, k, v = _rand(rng, 1, 50)
    q = np.zeros((3, 576))
    o, lse = attention.attend(q, k, v, SCALE)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-13)
    assert np.allclose(lse, np.log(50.0), atol=1e-13)


def test_dominant_key():
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 1, 10)
    k[3] = q[0] * (60.0 / SCALE / (q[0] @ q[0]))  # score 60 vs ~N(0,3)
    o, lse = attention.attend(q, k, k[:, :512], SCALE)
    assert np.allclose(o[0], k[3, :512], atol=1e-12)
    assert abs(lse[0] - 60.0) < 1e-12


def test_empty_set_is_identity_row():
    o, lse = attention.attend(np.ones((4, 576)), np.zeros((0, 576)), np.zeros((0, 512)), SCALE)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_shift_invariance():
    rng = np.random.default_rng(10)
    s = rng.standard_normal((3, 40)) * 3
    v = rng.standard_normal((40, 512))
    o1, l1 = attention.softmax_average(s, v)
    o2, l2 = attention.softmax_average(s + 123.25, v)
    assert np.allclose(o1, o2, atol=1e-12)
    assert np.allclose(l2 - l1, 123.25, atol=1e-12)


def test_permutation_invariance():
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 2, 64)
    perm = rng.permutation(64)
    o1, l1 = attention.attend(q, k, v, SCALE)
    o2, l2 = attention.attend(q, k[perm], v[perm], SCALE)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


@pytest.mark.parametrize("n_parts", [1, 2, 3, 8, 16])
def test_merge_of_any_partition_is_full_attention(n_parts):
    rng = np.random.default_rng(100 + n_parts)
    H, T = 6, 90
    q, k, v = _rand(rng, H, T)
    for trial in range(5):
        label = rng.integers(0, n_parts, size=T)
        if trial == 0 and n_parts > 1:
            label[label == 0] = 1  # force an empty part
        o_p, l_p = [], []
        for s in range(n_parts):
            m = label == s
            o, l = attention.attend(q, k[m], v[m], SCALE)
            o_p.append(o)
            l_p.append(l)
        om, lm = attention.merge(np.stack(o_p), np.stack(l_p))
        assert np.allclose(om, _sdpa(q, k, v, SCALE), atol=1e-12)
        assert np.allclose(lm, logsumexp(SCALE * (q @ k.T), axis=1), atol=1e-12)


def test_merge_single_part_is_identity():
    rng = np.random.default_rng(12)
    o = rng.standard_normal((1, 5, 512))
    l = rng.standard_normal((1, 5))
    om, lm = attention.merge(o, l)
    assert np.allclose(om, o[0], atol=1e-15) and np.allclose(lm, l[0], atol=1e-15)


def test_merge_is_associative():
    rng = np.random.default_rng(13)
    o = rng.standard_normal((6, 4, 512))
    l = rng.standard_normal((6, 4)) * 4
    l[2, 1] = -np.inf
    flat = attention.merge(o, l)
    a = attention.merge(o[:2], l[:2])
    b = attention.merge(o[2:5], l[2:5])
    c = attention.merge(o[5:], l[5:])
    two = attention.merge(np.stack([a[0], b[0], c[0]]), np.stack([a[1], b[1], c[1]]))
    assert np.allclose(flat[0], two[0], atol=1e-13) and np.allclose(flat[1], two[1], atol=1e-13)


def test_merge_all_empty_and_partly_empty():
    o = np.zeros((3, 2, 512))
    l = np.full((3, 2), -np.inf)
    om, lm = attention.merge(o, l)
    assert np.all(om == 0) and np.all(np.isneginf(lm)) and not np.isnan(om).any()
    rng = np.random.default_rng(14)
    o = rng.standard_normal((3, 2, 512))
    l = rng.standard_normal((3, 2))
    l[1] = -np.inf
    o[1] = 0.0
    om, lm = attention.merge(o, l)
    om2, lm2 = attention.merge(o[[0, 2]], l[[0, 2]])
    assert np.allclose(om, om2, atol=1e-15) and np.allclose(lm, lm2, atol=1e-15)


def test_merge_weights_follow_lse():
    # two parts with LSE a and b: weights e^a/(e^a+e^b)
    o = np.stack([np.full((1, 512), 1.0), np.full((1, 512), 3.0)])
    l = np.array([[np.log(1.0)], [np.log(3.0)]])
    om, lm = attention.merge(o, l)
    assert np.allclose(om, 0.25 * 1.0 + 0.75 * 3.0, atol=1e-15)
    assert np.allclose(lm, np.log(4.0), atol=1e-15)
