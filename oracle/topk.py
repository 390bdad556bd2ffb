"""Top-K selection of sparse-attention indices, per shard and merged.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The sparse path attends, for each query token, a fixed number K of earlier
tokens chosen by an indexer that scores the token's causal prefix ("GLM-5.2
vLLM Decode Context Parallelism", section "Understand the cache-copy
opportunity": sparse index top-K of 2,048; "How vLLM Serves GLM-5.3 with
Million-Token Contexts on 16 H200s", section "Why conventional TP and DP fall
short": the indexer scores earlier tokens, then sparse attention selects a
fixed set).  With the cache sharded round-robin, each rank holds the scores
of its own tokens, so selection splits into a local top-K per shard and a
merge of the shards' lists: every token of the global top-K is in its
owner's local top-K, so the top-K of the union of the local lists is the
global top-K.

Readings (the pages give no selection rule beyond "top-K"):
* order: larger score first; equal scores are ordered by position, lower
  position first, so the selected set is unique;
* a list is returned as its positions in ascending order, padded with -1
  when fewer than K positions exist (scores of padded entries are -inf);
* scores are finite float32 or -inf; +0 and -0 are one value, and a
  candidate list returns that value as +0.
"""

import numpy as np


def select(positions, scores, k):
    """The k best (position, score) pairs: ascending positions, -1 padded.

    Plain definition: order all candidates by (score descending, position
    ascending), keep the first k, then list the kept positions in ascending
    order.
    """
    positions = np.asarray(positions, dtype=np.int64)
    scores = np.asarray(scores, dtype=np.float32)
    order = np.lexsort((positions, -scores.astype(np.float64)))
    keep = order[:k]
    kept_pos = positions[keep]
    kept_score = scores[keep]
    asc = np.argsort(kept_pos, kind="stable")
    out_pos = np.full(k, -1, dtype=np.int64)
    out_score = np.full(k, -np.inf, dtype=np.float32)
    out_pos[:keep.size] = kept_pos[asc]
    out_score[:keep.size] = kept_score[asc]
    return out_pos, out_score


def visible(context_len, q_len, t):
    """Positions query token t of a request with context_len tokens sees."""
    return max(int(context_len) - q_len + t + 1, 0)


def global_topk(scores, context_lens, q_len, k):
    """scores [B][Tq][Lmax] float32 (global positions) -> [B][Tq][k] int64."""
    B = scores.shape[0]
    out = np.full((B, q_len, k), -1, dtype=np.int64)
    for b in range(B):
        for t in range(q_len):
            n = visible(context_lens[b], q_len, t)
            out[b, t], _ = select(np.arange(n), scores[b, t, :n], k)
    return out


def local_topk(scores, context_lens, q_len, k, shard, n_shards):
    """The shard's own candidates: top-k over the positions it owns.

    Returns (positions [B][Tq][k] global, -1 padded; scores [B][Tq][k]).
    """
    B = scores.shape[0]
    pos = np.full((B, q_len, k), -1, dtype=np.int64)
    sc = np.full((B, q_len, k), -np.inf, dtype=np.float32)
    for b in range(B):
        for t in range(q_len):
            n = visible(context_lens[b], q_len, t)
            owned = np.arange(shard, n, n_shards)
            pos[b, t], sc[b, t] = select(owned, scores[b, t, owned], k)
    # -0 and +0 are one value; a candidate's score is returned as +0
    sc[sc == 0] = 0.0
    return pos, sc


def merge_topk(cand_pos, cand_score, k):
    """cand_* [n_lists][rows][k'] (padding: position -1) -> [rows][k] positions."""
    cand_pos = np.asarray(cand_pos, dtype=np.int64)
    cand_score = np.asarray(cand_score, dtype=np.float32)
    n_lists, rows, _ = cand_pos.shape
    out = np.full((rows, k), -1, dtype=np.int64)
    for r in range(rows):
        p = cand_pos[:, r].reshape(-1)
        s = cand_score[:, r].reshape(-1)
        valid = p >= 0
        out[r], _ = select(p[valid], s[valid], k)
    return out


def local_topk_varlen(scores, context_lens, query_start_loc, k, shard, n_shards):
    """The shard's own candidates when request b holds query tokens
    query_start_loc[b] .. query_start_loc[b + 1] - 1 (the varlen-decode
    layout; "GLM-5.2 vLLM Decode Context Parallelism", section "See why vLLM
    0.26.0 fails").  Reading taken: a request with c tokens is the fixed form
    with Tq = c, so its token t selects among positions 0 .. L_b - c + t.

    scores [n_q][Lmax] float32 (global positions) -> (positions [n_q][k],
    scores [n_q][k]) as local_topk.
    """
    from .decode import varlen_tokens
    toks = varlen_tokens(query_start_loc)
    pos = np.full((len(toks), k), -1, dtype=np.int64)
    sc = np.full((len(toks), k), -np.inf, dtype=np.float32)
    for i, (b, t, c) in enumerate(toks):
        n = visible(context_lens[b], c, t)
        owned = np.arange(shard, n, n_shards)
        pos[i], sc[i] = select(owned, scores[i, owned], k)
    sc[sc == 0] = 0.0
    return pos, sc
