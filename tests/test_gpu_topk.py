"""GPU parity of the top-K selection calls against the oracle, bit for bit.

mla_topk_local (every shard's candidates in one launch, or one shard) and
mla_topk_merge run through the C ABI on seeded indexer scores; the oracle
(oracle/topk.py) gives the expected candidate lists, scores and the merged
global selection.  Cases: ragged causal prefixes (shorter than K, shorter
than N, empty), bf16-rounded scores with many equal values, rows of equal
scores, -inf and signed zeros, K above the LDS-resolved group, and the
full-size selection workload on sampled rows.  The varlen call
(mla_topk_local_varlen: a query count per request) is checked the same way,
against the fixed form when every request is full, with more requests than
a workgroup has threads, and with offsets that are not a partition.
"""

import numpy as np
import pytest
import torch

import workload
from oracle import topk as otk
from sequence_sharded_mla_amd import (MLA_DEVERR_QUERY, MLA_DEVERR_SCORES, layout,
                                      mla_clear_device_error, mla_get_device_error, mla_topk_local,
                                      mla_topk_local_varlen, mla_topk_merge)

from gpu_cases import say

pytestmark = pytest.mark.gpu


def run_local(sc_sh, lens, K, shard_begin, n_shards, ws=None):
    d = torch.from_numpy(np.ascontiguousarray(sc_sh)).cuda()
    S, B, Tq, _ = sc_sh.shape
    ci = torch.empty((S, B, Tq, K), dtype=torch.int32, device="cuda")
    cs = torch.empty((S, B, Tq, K), dtype=torch.float32, device="cuda")
    mla_topk_local(d, torch.from_numpy(np.asarray(lens, np.int32)).cuda(), K, shard_begin, n_shards,
                   ci, cs, workspace=ws)
    return ci, cs


def check_selection(scores, lens, Tq, K, N):
    B = scores.shape[0]
    sc_sh = layout.shard_scores(scores, N)
    ci, cs = run_local(sc_sh, lens, K, 0, N)
    merged = torch.empty((B * Tq, K), dtype=torch.int32, device="cuda")
    mla_topk_merge(ci.view(N, B * Tq, K), cs.view(N, B * Tq, K), K, merged)
    torch.cuda.synchronize()
    ci_h, cs_h = ci.cpu().numpy(), cs.cpu().numpy()
    for s in range(N):
        ref_p, ref_s = otk.local_topk(scores, lens, Tq, K, s, N)
        assert np.array_equal(ci_h[s], ref_p), f"shard {s} positions"
        assert np.array_equal(cs_h[s].view(np.uint32), ref_s.view(np.uint32)), f"shard {s} scores"
    ref = otk.global_topk(scores, lens, Tq, K)
    assert np.array_equal(merged.cpu().numpy().reshape(B, Tq, K), ref)
    return ref


@pytest.mark.parametrize("N", [1, 3, 8])
@pytest.mark.parametrize("K", [64, 2048])
def test_local_and_merge_match_oracle(N, K):
    say(f"topk N={N} K={K}")
    rng = np.random.default_rng(100 + N + K)
    B, Tq, L = 5, 2, 20000
    lens = np.array([1, 2, 3 * K // 2, L, 9000])
    scores = workload.indexer_scores(B, Tq, L, seed=N * 31 + K)
    scores[4, 0, :500] = 0.25                       # a run of equal scores
    scores[4, 1, ::7] = -np.inf
    scores[2, 0, :] = np.where(rng.random(L) < 0.5, np.float32(-0.0), np.float32(0.0))
    check_selection(scores, lens, Tq, K, N)


@pytest.mark.parametrize("N", [2, 8])
def test_bf16_scores_with_many_ties(N):
    say(f"topk ties N={N}")
    B, Tq, L, K = 3, 2, 40000, 2048
    lens = np.array([L, 30000, 2500])
    scores = workload.indexer_scores(B, Tq, L, seed=200 + N, ties=True)
    scores[1, 1, :] = 1.0                           # one value everywhere: positions decide
    check_selection(scores, lens, Tq, K, N)


def test_tied_group_larger_than_lds_candidates():
    """5000 equal scores straddle the K-th place: digits of the position
    decide the group before it fits in LDS."""
    say("topk wide tie")
    B, Tq, L, K = 1, 1, 12000, 3000
    scores = workload.indexer_scores(B, Tq, L, seed=300)
    scores[0, 0, 2000:7000] = 0.5
    scores[0, 0, 7000:] = -1.0 + scores[0, 0, 7000:] * 1e-3
    scores[0, 0, :2000] = 2.0 + np.abs(scores[0, 0, :2000])
    check_selection(scores, np.array([L]), Tq, K, 1)


def test_one_shard_call_matches_all_shards_call():
    B, Tq, L, K, N = 4, 2, 50000, 2048, 8
    lens = np.array([L, 100, 33333, 7])
    scores = workload.indexer_scores(B, Tq, L, seed=400)
    sc_sh = layout.shard_scores(scores, N)
    ci_all, cs_all = run_local(sc_sh, lens, K, 0, N)
    for s in (0, 5):
        ci, cs = run_local(sc_sh[s:s + 1], lens, K, s, N)
        torch.cuda.synchronize()
        assert torch.equal(ci[0], ci_all[s]) and torch.equal(cs[0], cs_all[s])


def test_short_score_rows_raise_the_error_word():
    B, Tq, L, K, N = 2, 1, 3000, 64, 4
    lens = np.array([L, L])
    scores = workload.indexer_scores(B, Tq, L, seed=500)
    sc_sh = layout.shard_scores(scores, N)[:, :, :, :600]   # 750 needed
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    mla_clear_device_error(ws)
    ci, _ = run_local(sc_sh, lens, K, 0, N, ws=ws)
    torch.cuda.synchronize()
    assert mla_get_device_error(ws) == MLA_DEVERR_SCORES
    # only the stored prefix of each shard's row counts
    trimmed = layout.shard_scores(scores, N)[:, :, :, :600]
    for s in range(N):
        ref, _ = otk.select(np.arange(600) * N + s, trimmed[s, 0, 0], K)
        assert np.array_equal(ci[s, 0, 0].cpu().numpy(), ref)


def test_full_size_selection_sampled():
    """The selection workload in the launch configuration the benchmark
    times (all shards in one launch, then the merge); 12 sampled rows."""
    w = workload.SELECT_SPECS["topk_select_262k"]
    B, Tq, L, K, N = w["batch"], w["q_len"], w["context"], w["topk"], w["n_shards"]
    say(f"full-size selection B={B} Tq={Tq} L={L} K={K} N={N}")
    scores = workload.indexer_scores(B, Tq, L, seed=w["seed"])
    lens = np.full(B, L)
    sc_sh = layout.shard_scores(scores, N)
    ci, cs = run_local(sc_sh, lens, K, 0, N)
    merged = torch.empty((B * Tq, K), dtype=torch.int32, device="cuda")
    mla_topk_merge(ci.view(N, B * Tq, K), cs.view(N, B * Tq, K), K, merged)
    torch.cuda.synchronize()
    got = merged.cpu().numpy().reshape(B, Tq, K)
    ci_h = ci.cpu().numpy()
    rng = np.random.default_rng(7)
    for b in rng.choice(B, 6, replace=False):
        ref = otk.global_topk(scores[b:b + 1], lens[b:b + 1], Tq, K)
        assert np.array_equal(got[b], ref[0])
        s = int(rng.integers(N))
        ref_p, _ = otk.local_topk(scores[b:b + 1], lens[b:b + 1], Tq, K, s, N)
        assert np.array_equal(ci_h[s, b], ref_p[0])


def test_merge_of_lists_in_any_order():
    """mla_topk_merge takes candidate lists in any order: the shards' lists
    shuffled within each row give the same selection (the ascending lists of
    mla_topk_local take the merge of sorted runs, these the general sort)."""
    B, Tq, L, K, N = 3, 2, 30000, 2048, 8
    lens = np.array([L, 20000, 9000])
    scores = workload.indexer_scores(B, Tq, L, seed=600)
    sc_sh = layout.shard_scores(scores, N)
    ci, cs = run_local(sc_sh, lens, K, 0, N)
    torch.cuda.synchronize()
    rng = np.random.default_rng(601)
    ci_h = ci.cpu().numpy().reshape(N, B * Tq, K)
    cs_h = cs.cpu().numpy().reshape(N, B * Tq, K)
    for s in range(N):
        for r in range(B * Tq):
            perm = rng.permutation(K)
            ci_h[s, r] = ci_h[s, r, perm]
            cs_h[s, r] = cs_h[s, r, perm]
    merged = torch.empty((B * Tq, K), dtype=torch.int32, device="cuda")
    mla_topk_merge(torch.from_numpy(ci_h).cuda(), torch.from_numpy(cs_h).cuda(), K, merged)
    torch.cuda.synchronize()
    ref = otk.global_topk(scores, lens, Tq, K)
    assert np.array_equal(merged.cpu().numpy().reshape(B, Tq, K), ref)


@pytest.mark.parametrize("shuffled", [False, True])
def test_merge_with_positions_beyond_the_bitmap(shuffled):
    """Candidate positions up to 2^30 (past the merge's position bitmap): the
    chosen entries are ordered by merging the lists' ascending runs, or by a
    sort when the lists are shuffled; the selection matches the oracle's."""
    rng = np.random.default_rng(700 + shuffled)
    n_lists, rows, k_in, K = 8, 5, 1500, 2048
    ci = np.full((n_lists, rows, k_in), -1, dtype=np.int32)
    cs = np.full((n_lists, rows, k_in), -np.inf, dtype=np.float32)
    for r in range(rows):
        pos = rng.choice(1 << 30, size=n_lists * k_in, replace=False).astype(np.int64)
        for s in range(n_lists):
            n_s = int(rng.integers(k_in // 2, k_in + 1))
            p_s = np.sort(pos[s * k_in: s * k_in + n_s])
            sc = rng.standard_normal(n_s).astype(np.float32)
            sc[rng.random(n_s) < 0.2] = 0.5                  # ties among lists
            if shuffled:
                perm = rng.permutation(n_s)
                p_s, sc = p_s[perm], sc[perm]
            ci[s, r, :n_s] = p_s
            cs[s, r, :n_s] = sc
    out = torch.empty((rows, K), dtype=torch.int32, device="cuda")
    mla_topk_merge(torch.from_numpy(ci).cuda(), torch.from_numpy(cs).cuda(), K, out)
    torch.cuda.synchronize()
    ref = otk.merge_topk(ci, cs, K)
    assert np.array_equal(out.cpu().numpy(), ref)


def run_local_varlen(scores, lens, qsl, K, N, ws=None):
    """scores [n_q][L] (global positions) -> device candidate lists [N][n_q][K]."""
    n_q, L = scores.shape
    sc_sh = layout.shard_scores(scores.reshape(n_q, 1, L), N).reshape(N, n_q, -1)
    ci = torch.empty((N, n_q, K), dtype=torch.int32, device="cuda")
    cs = torch.empty((N, n_q, K), dtype=torch.float32, device="cuda")
    mla_topk_local_varlen(torch.from_numpy(np.ascontiguousarray(sc_sh)).cuda(),
                          torch.from_numpy(np.asarray(lens, np.int32)).cuda(),
                          torch.from_numpy(np.asarray(qsl, np.int32)).cuda(), K, 0, N, ci, cs, workspace=ws)
    return ci, cs


def check_varlen(scores, lens, qsl, K, N):
    n_q = scores.shape[0]
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    ci, cs = run_local_varlen(scores, lens, qsl, K, N, ws=ws)
    merged = torch.empty((n_q, K), dtype=torch.int32, device="cuda")
    mla_topk_merge(ci, cs, K, merged)
    torch.cuda.synchronize()
    assert mla_get_device_error(ws) == 0
    ci_h, cs_h = ci.cpu().numpy(), cs.cpu().numpy()
    parts = [otk.local_topk_varlen(scores, lens, qsl, K, s, N) for s in range(N)]
    for s, (ref_p, ref_s) in enumerate(parts):
        assert np.array_equal(ci_h[s], ref_p), f"shard {s} positions"
        assert np.array_equal(cs_h[s].view(np.uint32), ref_s.view(np.uint32)), f"shard {s} scores"
    ref = otk.merge_topk(np.stack([p for p, _ in parts]), np.stack([q for _, q in parts]), K)
    assert np.array_equal(merged.cpu().numpy(), ref)


@pytest.mark.parametrize("N", [1, 8])
@pytest.mark.parametrize("K", [64, 2048])
def test_varlen_local_and_merge_match_oracle(N, K):
    say(f"topk varlen N={N} K={K}")
    lens = np.array([20000, 5000, 3 * K // 2, 2, 9000])
    counts = np.array([2, 0, 3, 1, 2])
    qsl = np.concatenate([[0], np.cumsum(counts)])
    n_q = int(qsl[-1])
    scores = workload.indexer_scores(n_q, 1, 20000, seed=600 + N + K, ties=True).reshape(n_q, 20000)
    scores[0, :500] = 0.25
    scores[6, ::5] = -np.inf
    check_varlen(scores, lens, qsl, K, N)


def test_varlen_all_full_matches_fixed_form():
    B, Tq, L, K, N = 4, 2, 30000, 2048, 8
    lens = np.array([L, 100, 23456, 4097])
    scores = workload.indexer_scores(B, Tq, L, seed=610)
    ci_f, cs_f = run_local(layout.shard_scores(scores, N), lens, K, 0, N)
    ci_v, cs_v = run_local_varlen(scores.reshape(B * Tq, L), lens, np.arange(0, B * Tq + 1, Tq), K, N)
    torch.cuda.synchronize()
    assert torch.equal(ci_v, ci_f.view(N, B * Tq, K))
    assert torch.equal(cs_v.view(torch.int32), cs_f.view(N, B * Tq, K).view(torch.int32))


def test_varlen_more_requests_than_threads():
    """700 requests: each workgroup counts the offsets in two passes."""
    say("topk varlen 700 requests")
    rng = np.random.default_rng(620)
    B, K, N = 700, 64, 4
    lens = rng.integers(0, 3000, size=B)
    counts = rng.integers(0, 3, size=B)
    qsl = np.concatenate([[0], np.cumsum(counts)])
    n_q = int(qsl[-1])
    scores = workload.indexer_scores(n_q, 1, 3000, seed=621).reshape(n_q, 3000)
    check_varlen(scores, lens, qsl, K, N)


def test_varlen_offsets_not_a_partition_raise_the_error_word():
    lens = np.array([5000, 4000, 3000])
    scores = workload.indexer_scores(5, 1, 5000, seed=630).reshape(5, 5000)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    for bad in ([0, 3, 2, 5], [1, 2, 3, 5], [0, 2, 3, 4]):
        mla_clear_device_error(ws)
        ci, cs = run_local_varlen(scores, lens, bad, 64, 4, ws=ws)
        torch.cuda.synchronize()
        assert mla_get_device_error(ws) & MLA_DEVERR_QUERY, bad
        assert torch.all(ci == -1) and torch.all(torch.isneginf(cs)), bad


def test_longest_supported_local_row():
    """A shard row at the longest supported stride (393,216 positions, the
    largest whose position bitmap fits in LDS beside the selection state)."""
    say("topk longest row")
    L = 393216
    scores = workload.indexer_scores(1, 1, L, seed=77)
    check_selection(scores, np.array([L]), 1, 2048, 1)
