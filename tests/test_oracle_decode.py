"""Pins of the oracle's batched decode step (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import attention, decode, sharding

SCALE = 1.0 / np.sqrt(192.0)


def _make(rng, B, Tq, H, lens):
    q = rng.standard_normal((B, Tq, H, 576))
    store = [rng.standard_normal((int(L), 576)) for L in lens]

    def rows(b, pos):
        r = store[b][np.asarray(pos, dtype=np.int64)]
        return r[:, :512], r[:, 512:]
    return q, store, rows


def _sdpa(q, k, scale):
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(k)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(np.ascontiguousarray(k[:, :512]))[None, None].expand(1, q.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, :, 0].numpy()


def test_dense_single_token_sees_whole_context():
    rng = np.random.default_rng(1)
    lens = [1, 5, 64, 130]
    q, store, rows = _make(rng, 4, 1, 3, lens)
    r = decode.mla_decode(q, rows, np.array(lens), 1, 3, SCALE)
    for b in range(4):
        assert np.allclose(r["o"][b, 0], _sdpa(q[b, 0], store[b], SCALE), atol=1e-12)


def test_causal_range_of_two_query_tokens():
    # the last cached row is the second query token's own KV: query 0 must
    # not see it, query 1 must.
    rng = np.random.default_rng(2)
    L = 40
    q, store, rows = _make(rng, 1, 2, 2, [L])
    big = q[0, 1, 0] * (80.0 / SCALE / (q[0, 1, 0] @ q[0, 1, 0]))
    store[0][L - 1] = big
    r = decode.mla_decode(q, rows, np.array([L]), 2, 1, SCALE)
    assert np.allclose(r["o"][0, 1, 0], big[:512], atol=1e-9)
    assert np.allclose(r["o"][0, 0], _sdpa(q[0, 0], store[0][:L - 1], SCALE), atol=1e-12)
    assert np.allclose(r["o"][0, 1], _sdpa(q[0, 1], store[0][:L], SCALE), atol=1e-12)


def test_per_shard_partial_is_attention_over_owned_tokens():
    rng = np.random.default_rng(3)
    lens = [70, 9]
    N = 4
    q, store, rows = _make(rng, 2, 1, 2, lens)
    r = decode.mla_decode(q, rows, np.array(lens), 1, N, SCALE)
    for b, L in enumerate(lens):
        for s in range(N):
            owned = [p for p in range(L) if p % N == s]   # dealt one at a time
            o, l = attention.attend(q[b, 0], store[b][owned], store[b][owned][:, :512], SCALE)
            assert np.allclose(r["o_shards"][s, b, 0], o, atol=1e-13)
            assert np.allclose(r["lse_shards"][s, b, 0], l, atol=1e-13)
        om, lm = attention.merge(r["o_shards"][:, b], r["lse_shards"][:, b])
        assert np.allclose(om, r["o"][b], atol=1e-12) and np.allclose(lm, r["lse"][b], atol=1e-12)


def test_more_shards_than_tokens_gives_identity_rows():
    rng = np.random.default_rng(4)
    q, store, rows = _make(rng, 1, 1, 2, [3])
    r = decode.mla_decode(q, rows, np.array([3]), 1, 8, SCALE)
    for s in range(3, 8):
        assert np.all(r["o_shards"][s] == 0) and np.all(np.isneginf(r["lse_shards"][s]))
    assert np.allclose(r["o"][0, 0], _sdpa(q[0, 0], store[0], SCALE), atol=1e-12)


def test_sparse_uses_only_selected_rows():
    rng = np.random.default_rng(5)
    L, K, N = 500, 33, 8
    q, store, rows = _make(rng, 1, 2, 4, [L])
    idx = np.full((1, 2, K + 3), -1, dtype=np.int32)
    for j in range(2):
        idx[0, j, :K] = rng.choice(L - 2 + j + 1, size=K, replace=False)
    r = decode.mla_decode(q, rows, np.array([L]), 2, N, SCALE, topk_idx=idx)
    for j in range(2):
        sel = idx[0, j][idx[0, j] >= 0]
        assert np.allclose(r["o"][0, j], _sdpa(q[0, j], store[0][sel], SCALE), atol=1e-12)
        for s in range(N):
            loc = sharding.localize(idx[0, j], s, N)
            mine = sharding.global_position(loc[loc >= 0], s, N)
            o, l = attention.attend(q[0, j], store[0][mine], store[0][mine][:, :512], SCALE)
            assert np.allclose(r["o_shards"][s, 0, j], o, atol=1e-13)


def test_sparse_rejects_index_beyond_prefix():
    rng = np.random.default_rng(6)
    q, store, rows = _make(rng, 1, 2, 1, [10])
    idx = np.array([[[9, 0], [3, 1]]], dtype=np.int32)  # query 0 may see 0..8
    with pytest.raises(ValueError):
        decode.mla_decode(q, rows, np.array([10]), 2, 2, SCALE, topk_idx=idx)


def test_sparse_row_with_no_valid_index():
    rng = np.random.default_rng(7)
    q, store, rows = _make(rng, 1, 1, 2, [10])
    idx = np.full((1, 1, 4), -1, dtype=np.int32)
    r = decode.mla_decode(q, rows, np.array([10]), 1, 2, SCALE, topk_idx=idx)
    assert np.all(r["o"] == 0) and np.all(np.isneginf(r["lse"]))
    assert np.all(r["o_shards"] == 0) and np.all(np.isneginf(r["lse_shards"]))


def test_brute_force_scalar_loops():
    """Pure-Python scalar loops on tiny inputs: every shard's partial and the
    merged result, written out term by term with math.exp / math.log."""
    import math
    rng = np.random.default_rng(8)
    B, Tq, H, N = 2, 2, 2, 3
    lens = [7, 12]
    q, store, rows = _make(rng, B, Tq, H, lens)
    r = decode.mla_decode(q, rows, np.array(lens), Tq, N, SCALE)
    for b in range(B):
        L = lens[b]
        for t in range(Tq):
            last = L - Tq + t
            for h in range(H):
                qv = [float(v) for v in q[b, t, h]]
                parts = []
                for s in range(N):
                    sc = {}
                    for p in range(last + 1):
                        if p % N != s:
                            continue
                        kv = store[b][p]
                        dot = 0.0
                        for d in range(576):
                            dot += qv[d] * float(kv[d])
                        sc[p] = SCALE * dot
                    if not sc:
                        parts.append((None, -math.inf))
                        o_ref, l_ref = [0.0] * 512, -math.inf
                    else:
                        mx = max(sc.values())
                        den = sum(math.exp(v - mx) for v in sc.values())
                        l_ref = mx + math.log(den)
                        o_ref = [0.0] * 512
                        for p, v in sc.items():
                            w = math.exp(v - l_ref)
                            for d in range(512):
                                o_ref[d] += w * float(store[b][p][d])
                        parts.append((o_ref, l_ref))
                    assert abs(r["lse_shards"][s, b, t, h] - l_ref) < 1e-12 or (
                        l_ref == -math.inf and r["lse_shards"][s, b, t, h] == -np.inf)
                    assert np.allclose(r["o_shards"][s, b, t, h], o_ref, atol=1e-12)
                m = max(l for _, l in parts)
                wsum = sum(math.exp(l - m) for _, l in parts if l > -math.inf)
                o_m = [0.0] * 512
                for o, l in parts:
                    if o is None:
                        continue
                    w = math.exp(l - m) / wsum
                    for d in range(512):
                        o_m[d] += w * o[d]
                assert abs(r["lse"][b, t, h] - (m + math.log(wsum))) < 1e-12
                assert np.allclose(r["o"][b, t, h], o_m, atol=1e-12)


def _masked_softmax_attention(q, keys, visible, scale):
    """Textbook attention of q [H, 576] over all keys with positions >=
    visible masked to -inf (scipy's softmax and logsumexp)."""
    from scipy.special import logsumexp, softmax
    s = (q @ keys.T) * scale
    s[:, visible:] = -np.inf
    if visible <= 0:
        return np.zeros((q.shape[0], 512)), np.full(q.shape[0], -np.inf)
    return softmax(s, axis=1) @ keys[:, :512], logsumexp(s, axis=1)


def test_varlen_matches_masked_softmax_per_token():
    # requests with 2, 0, 3, 1 query tokens; the causal limit moves with the
    # request's own count
    rng = np.random.default_rng(21)
    lens = [9, 4, 30, 2]
    counts = [2, 0, 3, 1]
    qsl = np.concatenate([[0], np.cumsum(counts)])
    H, N = 2, 3
    store = [rng.standard_normal((L, 576)) for L in lens]
    q = rng.standard_normal((int(qsl[-1]), H, 576))

    def rows(b, pos):
        r = store[b][np.asarray(pos, dtype=np.int64)]
        return r[:, :512], r[:, 512:]
    r = decode.mla_decode_varlen(q, rows, np.array(lens), qsl, N, SCALE)
    i = 0
    for b, c in enumerate(counts):
        for t in range(c):
            o, l = _masked_softmax_attention(q[i], store[b], lens[b] - c + t + 1, SCALE)
            assert np.allclose(r["o"][i], o, atol=1e-12) and np.allclose(r["lse"][i], l, atol=1e-12)
            om, lm = attention.merge(r["o_shards"][:, i], r["lse_shards"][:, i])
            assert np.allclose(om, o, atol=1e-12) and np.allclose(lm, l, atol=1e-12)
            i += 1
    # the newest token of each request sees its whole context, itself included
    assert np.allclose(r["o"][1], _sdpa(q[1], store[0], SCALE), atol=1e-12)


def test_varlen_sparse_and_token_subset():
    rng = np.random.default_rng(22)
    lens, counts, N = [50, 80], [3, 1], 4
    qsl = np.array([0, 3, 4])
    store = [rng.standard_normal((L, 576)) for L in lens]
    q = rng.standard_normal((4, 2, 576))
    idx = np.full((4, 6), -1, dtype=np.int32)
    idx[0, :3] = [0, 47, 10]        # token 0 of request 0 sees up to 47
    idx[2, :2] = [49, 3]
    idx[3, :4] = [79, 0, 1, 2]

    def rows(b, pos):
        r = store[b][np.asarray(pos, dtype=np.int64)]
        return r[:, :512], r[:, 512:]
    r = decode.mla_decode_varlen(q, rows, np.array(lens), qsl, N, SCALE, topk_idx=idx, tokens=[3, 0, 1])
    for ti, (i, b) in enumerate([(3, 1), (0, 0), (1, 0)]):
        sel = idx[i][idx[i] >= 0]
        o, l = attention.attend(q[i], store[b][sel], store[b][sel][:, :512], SCALE)
        assert np.allclose(r["o"][ti], o, atol=1e-12) and np.allclose(r["lse"][ti], l, atol=1e-12)
    assert np.all(np.isneginf(r["lse"][2]))          # token 1 has no index
    bad = idx.copy()
    bad[0, 0] = 48                                   # beyond L - 3 + 0
    with pytest.raises(ValueError):
        decode.mla_decode_varlen(q, rows, np.array(lens), qsl, N, SCALE, topk_idx=bad)
    with pytest.raises(ValueError):
        decode.mla_decode_varlen(q, rows, np.array(lens), np.array([0, 3, 2]), N, SCALE)


def test_sparse_repeated_positions_count_with_multiplicity():
    """Reading taken: a top-K list is a multiset, one softmax term per entry.
    Closed form: one position listed m times gives its latent as O and
    s + ln m as LSE.  In general, a position listed m times equals the same
    key listed once with ln m added to its score (scipy's logsumexp over the
    distinct keys with those weights)."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(8)
    L, N, H = 50, 3, 2
    q, store, rows = _make(rng, 1, 2, H, [L])
    idx = np.array([[[7, 7, 7, 7, 7, -1], [4, 9, 9, 20, 4, 4]]], dtype=np.int32)
    r = decode.mla_decode(q, rows, np.array([L]), 2, N, SCALE, topk_idx=idx)
    s7 = SCALE * (q[0, 0] @ store[0][7])
    assert np.allclose(r["o"][0, 0], np.broadcast_to(store[0][7, :512], (H, 512)), atol=1e-13)
    assert np.allclose(r["lse"][0, 0], s7 + np.log(5.0), atol=1e-13)
    keys, mult = np.array([4, 9, 20]), np.array([3.0, 2.0, 1.0])
    s = SCALE * (q[0, 1] @ store[0][keys].T) + np.log(mult)[None, :]
    lse = logsumexp(s, axis=1)
    o = np.exp(s - lse[:, None]) @ store[0][keys][:, :512]
    assert np.allclose(r["lse"][0, 1], lse, atol=1e-12)
    assert np.allclose(r["o"][0, 1], o, atol=1e-12)
    # the shard owning position 4 (4 mod 3 = 1) counts it three times
    k4 = store[0][[4]]
    o1, l1 = attention.attend(q[0, 1], k4, k4[:, :512], SCALE)
    assert np.allclose(r["lse_shards"][1, 0, 1], l1 + np.log(3.0), atol=1e-12)
    assert np.allclose(r["o_shards"][1, 0, 1], o1, atol=1e-13)
