"""One decode step of sequence-sharded MLA attention over a batch.

TEST INFRASTRUCTURE ONLY (see the package docstring).

For request b, query token j and head h:

1. the attended global positions P:
   dense  -- every cached position the query may see.  Reading taken: the
             context length L_b counts the query tokens' own KV rows (the
             cache write precedes attention, "GLM-5.2 vLLM Decode Context
             Parallelism", section "Keep the current-main correctness blocker
             visible"), so query j of Tq sits at position L_b - Tq + j and
             sees positions 0 .. L_b - Tq + j inclusive;
   sparse -- the valid (non-negative) entries of that query token's global
             top-K index list ("GLM-5.2 vLLM Decode Context Parallelism",
             section "Understand the cache-copy opportunity": sparse MLA
             with index top-K).
2. the partial of shard s is attention over P_s = {p in P : p mod N = s}
   (round-robin ownership, oracle.sharding), returning (O_s, LSE_s), with
   (0, -inf) when P_s is empty;
3. the exact full-context result is attention over all of P; the LSE merge
   of the N partials must reproduce it.

Rows are fetched through a caller-supplied function so that very long
contexts can be evaluated a slice at a time; only the order in which the
plain sums are added changes.
"""

import numpy as np

from . import attention, sharding

DK = 576
DV = 512
CHUNK = 65536


def _attend_positions(q, rows, b, positions, scale):
    """Attention of q [H, 576] over the given global positions of request b.

    Scores for all positions are formed first (slice by slice), then the
    softmax statistics, then the weighted sum of values (slice by slice).
    """
    H = q.shape[0]
    n = positions.shape[0]
    if n == 0:
        return np.zeros((H, DV)), np.full(H, attention.NEG_INF)
    s = np.empty((H, n))
    for c0 in range(0, n, CHUNK):
        lat, rope = rows(b, positions[c0:c0 + CHUNK])
        k = np.concatenate([lat, rope], axis=1)
        s[:, c0:c0 + CHUNK] = attention.scores(q, k, scale)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    acc = np.zeros((H, DV))
    for c0 in range(0, n, CHUNK):
        lat, _ = rows(b, positions[c0:c0 + CHUNK])
        acc += e[:, c0:c0 + CHUNK] @ lat
    return acc / l[:, None], m + np.log(l)


def attended_positions(b, j, context_lens, q_len, topk_idx=None):
    """Global positions query token j of request b attends (step 1)."""
    if topk_idx is None:
        last = int(context_lens[b]) - q_len + j
        return np.arange(max(last + 1, 0), dtype=np.int64)
    idx = np.asarray(topk_idx[b, j], dtype=np.int64)
    idx = idx[idx >= 0]
    limit = int(context_lens[b]) - q_len + j
    if idx.size and idx.max() > limit:
        raise ValueError("top-K index outside the causal prefix")
    return idx


def mla_decode(q, rows, context_lens, q_len, n_shards, scale,
               topk_idx=None, requests=None, shards=None, full=True):
    """Per-shard partials and the exact result for a batch.

    q            float64 [B, Tq, H, 576]
    rows(b, pos) -> (latent float64 [n, 512], rope float64 [n, 64])
    context_lens int [B]
    topk_idx     int [B, Tq, K] global indices (-1 = none) or None (dense)
    requests     subset of request ids to evaluate (default: all)
    shards       subset of shard ids to evaluate (default: all)
    full         also compute the unsharded result

    Returns a dict with, over the evaluated requests in the given order:
      o_shards [S, R, Tq, H, 512], lse_shards [S, R, Tq, H],
      o, lse   (unsharded, when full) [R, Tq, H, 512], [R, Tq, H].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Tq, H, D = q.shape
    assert D == DK and Tq == q_len
    requests = list(range(B)) if requests is None else list(requests)
    shards = list(range(n_shards)) if shards is None else list(shards)
    R, S = len(requests), len(shards)
    o_sh = np.zeros((S, R, Tq, H, DV))
    lse_sh = np.zeros((S, R, Tq, H))
    o = np.zeros((R, Tq, H, DV)) if full else None
    lse = np.zeros((R, Tq, H)) if full else None
    for ri, b in enumerate(requests):
        for j in range(Tq):
            P = attended_positions(b, j, context_lens, q_len, topk_idx)
            for si, s in enumerate(shards):
                Ps = sharding.shard_positions(P, s, n_shards)
                o_sh[si, ri, j], lse_sh[si, ri, j] = _attend_positions(
                    q[b, j], rows, b, Ps, scale)
            if full:
                o[ri, j], lse[ri, j] = _attend_positions(q[b, j], rows, b, P, scale)
    out = {"o_shards": o_sh, "lse_shards": lse_sh}
    if full:
        out["o"], out["lse"] = o, lse
    return out


def varlen_tokens(query_start_loc):
    """(request, index in it, the request's count) for every query token of
    a call whose request b holds tokens query_start_loc[b] .. [b + 1] - 1."""
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    if qsl.ndim != 1 or qsl.size < 1 or qsl[0] != 0 or np.any(np.diff(qsl) < 0):
        raise ValueError("query_start_loc must start at 0 and not decrease")
    out = []
    for b in range(qsl.size - 1):
        c = int(qsl[b + 1] - qsl[b])
        out.extend((b, t, c) for t in range(c))
    return out


def mla_decode_varlen(q, rows, context_lens, query_start_loc, n_shards, scale,
                      topk_idx=None, tokens=None):
    """The decode step when requests carry different numbers of query tokens
    (multi-token prediction drafts; "GLM-5.2 vLLM Decode Context
    Parallelism", section "See why vLLM 0.26.0 fails": the DCP backend must
    accept the varlen-decode layout).

    Reading taken: a request with c query tokens is the fixed form with
    Tq = c, so its token t sits at position L_b - c + t and sees positions
    0 .. L_b - c + t; only the count varies from request to request.

    q            float64 [n_q, H, 576], tokens of request b at rows
                 query_start_loc[b] .. query_start_loc[b + 1] - 1
    topk_idx     int [n_q, K] global indices (-1 = none) or None (dense)
    tokens       subset of query-token rows to evaluate (default: all)

    Returns o_shards [N, T, H, 512], lse_shards [N, T, H], o [T, H, 512],
    lse [T, H] over the evaluated tokens T in the given order.
    """
    q = np.asarray(q, dtype=np.float64)
    n_q, H, D = q.shape
    assert D == DK
    where = varlen_tokens(query_start_loc)
    if len(where) != n_q:
        raise ValueError("query_start_loc does not cover the query rows")
    tokens = list(range(n_q)) if tokens is None else list(tokens)
    T = len(tokens)
    o_sh = np.zeros((n_shards, T, H, DV))
    lse_sh = np.zeros((n_shards, T, H))
    o = np.zeros((T, H, DV))
    lse = np.zeros((T, H))
    for ti, i in enumerate(tokens):
        b, t, c = where[i]
        last = int(context_lens[b]) - c + t
        if topk_idx is None:
            P = np.arange(max(last + 1, 0), dtype=np.int64)
        else:
            P = np.asarray(topk_idx[i], dtype=np.int64)
            P = P[P >= 0]
            if P.size and P.max() > last:
                raise ValueError("top-K index outside the causal prefix")
        for s in range(n_shards):
            Ps = sharding.shard_positions(P, s, n_shards)
            o_sh[s, ti], lse_sh[s, ti] = _attend_positions(q[i], rows, b, Ps, scale)
        o[ti], lse[ti] = _attend_positions(q[i], rows, b, P, scale)
    return {"o_shards": o_sh, "lse_shards": lse_sh, "o": o, "lse": lse}


def query_to_f64(q, q_dtype):
    """Stored query (float32, or bf16 bits as uint16) -> float64."""
    from . import codecs
    if q_dtype == "f32":
        return codecs.f32_to_f64(q)
    if q_dtype == "bf16":
        return codecs.bf16_bits_to_f64(q)
    raise ValueError(q_dtype)


def storage_rows(kv_dtype, latent, scales, rope, row_offsets, row_pos):
    """Row accessor over logical cache arrays in their stored formats.

    Rows of request b are row_offsets[b]:row_offsets[b+1], holding the
    global positions row_pos[...] in increasing order.  The accessor returns
    float64 (latent, rope) for a list of global positions of one request,
    decoding f32 / bf16 bits / fp8 codes with per-group scales.
    """
    from . import codecs

    def decode(r):
        if kv_dtype == "f32":
            return codecs.f32_to_f64(latent[r]), codecs.f32_to_f64(rope[r])
        if kv_dtype == "bf16":
            return codecs.bf16_bits_to_f64(latent[r]), codecs.bf16_bits_to_f64(rope[r])
        if kv_dtype == "fp8_ds":
            return (codecs.fp8_ds_latent_to_f64(latent[r], scales[r]),
                    codecs.bf16_bits_to_f64(rope[r]))
        raise ValueError(kv_dtype)

    def rows(b, positions):
        lo, hi = int(row_offsets[b]), int(row_offsets[b + 1])
        pos_b = row_pos[lo:hi]
        positions = np.asarray(positions, dtype=np.int64)
        k = np.searchsorted(pos_b, positions)
        if positions.size and (k.max() >= pos_b.size or np.any(pos_b[k] != positions)):
            raise KeyError("position not stored for this request")
        return decode(lo + k)

    return rows
