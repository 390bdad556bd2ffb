"""Softmax attention with log-sum-exp, and the LSE merge of partials.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain float64 numpy.

Definitions followed:

* Each shard attends over only the tokens it owns and hands back its partial
  output together with the softmax log-sum-exp; the partials are then
  combined with the softmax normalisation restored from those LSE values
  ("GLM-5.2 vLLM Decode Context Parallelism", section "See why vLLM 0.26.0
  fails", and "Frequently asked questions": why DCP needs softmax LSE).
* A shard with no token to attend contributes the neutral pair
  (output 0, LSE -inf), which drops out of the merge (same page, section
  "Separate the backend merge from stable").
* MLA with one latent KV head: the key of token t is its 576-d row
  [latent(512) | rope(64)], its value is the 512-d latent part; every query
  head uses the same key/value rows ("GLM-5.2 vLLM Decode Context
  Parallelism", section "Understand the cache-copy opportunity").

Readings taken where the pages are silent:

* the score is s_t = scale * <q, k_t> and the LSE is the natural log of
  sum_t exp(s_t), scale included;
* each partial output is normalised over its own tokens
  (O_s = sum_t exp(s_t - LSE_s) v_t), so merge weights are
  exp(LSE_s - LSE);
* merging parts whose LSEs are all -inf gives (0, -inf), never NaN.
"""

import numpy as np

NEG_INF = -np.inf


def scores(q, k, scale):
    """s[h, t] = scale * sum_d q[h, d] * k[t, d].  q [H, D], k [T, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    return scale * (q @ k.T)


def softmax_average(s, v):
    """Softmax over the token axis of s [H, T] applied to v [T, Dv].

    Returns (o [H, Dv], lse [H]) with lse = log sum_t exp(s[:, t]) and
    o = sum_t exp(s[:, t] - lse) v[t].  With T == 0 returns (0, -inf).
    """
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    H, T = s.shape
    if T == 0:
        return np.zeros((H, v.shape[1])), np.full(H, NEG_INF)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    o = (e @ v) / l[:, None]
    return o, m + np.log(l)


def attend(q, k, v, scale):
    """Attention of query heads q [H, Dk] over keys k [T, Dk], values v [T, Dv]."""
    return softmax_average(scores(q, k, scale), v)


def merge(o_parts, lse_parts):
    """LSE-weighted merge over the leading (part) axis.

    o_parts [n, ..., Dv], lse_parts [n, ...] -> (o [..., Dv], lse [...]).
    M = max_s LSE_s; w_s = exp(LSE_s - M); O = sum_s w_s O_s / sum_s w_s;
    LSE = M + log sum_s w_s.  Where every LSE_s is -inf the result is
    (0, -inf).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    empty = np.isneginf(M)
    M_safe = np.where(empty, 0.0, M)
    w = np.where(np.isneginf(lse_parts), 0.0, np.exp(lse_parts - M_safe))
    W = w.sum(axis=0)
    W_safe = np.where(empty, 1.0, W)
    o = (w[..., None] * o_parts).sum(axis=0) / W_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, NEG_INF, M_safe + np.log(W_safe))
    return o, lse
