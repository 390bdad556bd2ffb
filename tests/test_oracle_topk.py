"""Pins of the oracle's top-K selection (oracle/topk.py).

The selected set is checked against the definition by brute force
(dominance over every unselected candidate), against torch.topk on distinct
scores, on all-equal and -inf scores, and the per-shard decomposition (merge
of the shards' local lists) against the direct global selection.
"""

import itertools

import numpy as np
import pytest
import torch

from oracle import topk as otk


def dominates(pc, sc, pu, su):
    return sc > su or (sc == su and pc < pu)


def test_select_brute_force_small():
    rng = np.random.default_rng(1)
    for trial in range(300):
        n = int(rng.integers(0, 9))
        k = int(rng.integers(1, 6))
        pos = rng.permutation(40)[:n]
        sc = rng.integers(-2, 3, n).astype(np.float32)        # many ties
        got, got_s = otk.select(pos, sc, k)
        m = min(k, n)
        assert np.all(got[m:] == -1) and np.all(np.isneginf(got_s[m:]))
        chosen = set(int(p) for p in got[:m])
        assert list(got[:m]) == sorted(chosen)
        # the chosen set is the unique m-subset dominating every other candidate
        winners = [c for c in itertools.combinations(range(n), m)
                   if all(dominates(pos[i], sc[i], pos[j], sc[j])
                          for i in c for j in range(n) if j not in c)]
        assert len(winners) == 1
        assert chosen == {int(pos[i]) for i in winners[0]}
        for p, s in zip(got[:m], got_s[:m]):
            assert s == sc[list(pos).index(p)]


def test_select_matches_torch_topk_on_distinct_scores():
    rng = np.random.default_rng(2)
    for n, k in [(5000, 2048), (2048, 2048), (100, 2048), (70000, 3000)]:
        sc = rng.permutation(n).astype(np.float32) - n / 2      # distinct
        got, _ = otk.select(np.arange(n), sc, k)
        ref = torch.topk(torch.from_numpy(sc), min(k, n)).indices.numpy()
        assert set(got[got >= 0].tolist()) == set(ref.tolist())


def test_ties_take_lower_positions_and_signed_zero_is_one_value():
    got, _ = otk.select(np.arange(10), np.zeros(10, np.float32), 4)
    assert list(got) == [0, 1, 2, 3]
    sc = np.array([-0.0, 0.0, -0.0, 0.0, 1.0], np.float32)
    got, _ = otk.select(np.arange(5), sc, 3)
    assert list(got) == [0, 1, 4]
    sc = np.array([-np.inf, 1.0, -np.inf, -5.0], np.float32)
    got, s = otk.select(np.arange(4), sc, 3)
    assert list(got) == [0, 1, 3] and np.isneginf(s[0])


@pytest.mark.parametrize("n_shards", [1, 2, 3, 8, 9])
def test_merge_of_local_lists_is_the_global_selection(n_shards):
    rng = np.random.default_rng(3 + n_shards)
    B, Tq, k = 3, 2, 64
    lens = np.array([1, 700, 5000])
    # bf16-rounded normal scores: plenty of equal values
    raw = rng.standard_normal((B, Tq, 5000)).astype(np.float32)
    sc = (raw.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    ref = otk.global_topk(sc, lens, Tq, k)
    parts = [otk.local_topk(sc, lens, Tq, k, s, n_shards) for s in range(n_shards)]
    cand_pos = np.stack([p for p, _ in parts]).reshape(n_shards, B * Tq, k)
    cand_sc = np.stack([s for _, s in parts]).reshape(n_shards, B * Tq, k)
    for s, (p, _) in enumerate(parts):
        assert np.all((p < 0) | (p % n_shards == s))
    merged = otk.merge_topk(cand_pos, cand_sc, k).reshape(B, Tq, k)
    assert np.array_equal(merged, ref)
    # causal range: query token t of a request of length L sees L - Tq + t + 1
    assert np.all(ref[0, 0] == -1) and ref[0, 1, 0] == 0 and np.all(ref[0, 1, 1:] == -1)
    assert ref[1, 0].max() <= 698 and ref[1, 1].max() <= 699


def test_varlen_local_lists_cover_each_tokens_causal_prefix():
    """Varlen: request b with c tokens; its token t sees positions 0 .. L_b -
    c + t.  With k above every prefix, a shard's list is exactly its owned
    positions of that prefix; a request with no tokens contributes no row."""
    lens = np.array([10, 0, 7, 3])
    qsl = np.array([0, 3, 3, 4, 6])  # counts 3, 0, 1, 2
    N = 3
    sc = np.random.default_rng(5).standard_normal((6, 16)).astype(np.float32)
    limits = [8, 9, 10, 7, 2, 3]  # visible positions per token, by hand
    for s in range(N):
        pos, _ = otk.local_topk_varlen(sc, lens, qsl, 16, s, N)
        for i, v in enumerate(limits):
            want = np.arange(s, v, N)
            assert np.array_equal(pos[i, :want.size], want) and np.all(pos[i, want.size:] == -1)


def test_varlen_merge_is_brute_force_top_k():
    rng = np.random.default_rng(17)
    lens = np.array([300, 50, 1, 220])
    qsl = np.array([0, 2, 5, 5, 9])  # counts 2, 3, 0, 4
    k, N = 20, 4
    raw = rng.standard_normal((9, 300)).astype(np.float32)
    sc = (raw.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    sc[0, :40] = 0.5  # a run of equal scores
    parts = [otk.local_topk_varlen(sc, lens, qsl, k, s, N) for s in range(N)]
    merged = otk.merge_topk(np.stack([p for p, _ in parts]), np.stack([s for _, s in parts]), k)
    tok = [(0, 0, 2), (0, 1, 2), (1, 0, 3), (1, 1, 3), (1, 2, 3), (3, 0, 4), (3, 1, 4), (3, 2, 4), (3, 3, 4)]
    for i, (b, t, c) in enumerate(tok):
        v = max(int(lens[b]) - c + t + 1, 0)
        best = sorted(range(v), key=lambda j: (-float(sc[i, j]), j))[:k]
        want = sorted(best) + [-1] * (k - len(best))
        assert list(merged[i]) == want, i
