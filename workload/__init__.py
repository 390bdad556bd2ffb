"""Seeded synthetic inputs for one MLA decode step.

This module only draws random numbers and stores them in the number formats
the cache uses; it holds none of the attention arithmetic, the sharding or
the paged layout.  Its outputs are the *logical* arrays (one row per cached
token, in global token order), which feed both the float64 oracle and the
layout packer of the GPU library.

Workloads (the shapes of the pages' long-context MLA decode settings; the
trace and tasks the pages measure on are not available, and these synthetic
draws stand in for them):

  tiny_f32             1 request, 1 query token, 16 heads, context 1024,
                       4 shards, float32 query and cache
  dense_bf16_32k       32 requests, 128 heads, context 32768, 8 shards,
                       bf16 query and cache
  dense_bf16_h64_32k   the same with 64 heads (the gathered-head pad)
  dense_fp8_mixed      64 requests, 64 heads, context uniform on
                       [4096, 131072], 8 shards, fp8 cache
  long_fp8_1m          4 requests, 64 heads, context 1048576, 8 shards,
                       fp8 cache
  sparse_fp8_topk2048  128 requests, 2 query tokens each, 64 heads,
                       context 262144, 2048 top-K indices per query token
                       drawn uniformly without replacement from its causal
                       prefix, 8 shards, fp8 cache

Values: query, latent and rope entries are independent N(0, 1).  The fp8
cache stores the latent part per 128-dimension group as E4M3FN codes with
one float32 scale (scale = group max |x| / 448, 1 for an all-zero group;
codes are x / scale rounded to nearest-even after clamping to +-448) and
the rope part as bf16.  bf16 values are float32 draws rounded to
nearest-even.  Draws are made per (request, 65536-token slice) from seeds
derived from the workload seed, so the result does not depend on how many
threads generate it.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
import math
import os

import numpy as np
import torch

LATENT = 512
ROPE = 64
DK = LATENT + ROPE
FP8_GROUP = 128
FP8_MAX = 448.0
SLICE = 65536


@dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    q_len: int
    heads: int
    n_shards: int
    q_dtype: str            # 'f32' | 'bf16'
    kv_dtype: str           # 'f32' | 'bf16' | 'fp8_ds'
    out_dtype: str          # 'f32' | 'bf16'
    context: int = 0        # fixed context length, or 0 with ctx_range
    ctx_range: tuple = ()   # (lo, hi) inclusive, uniform integers
    topk: int = 0           # 0 = dense
    scale: float = 1.0 / math.sqrt(192.0)
    block_size: int = 64
    seed: int = 0

    def with_(self, **kw):
        return replace(self, **kw)


SPECS = {
    "tiny_f32": Spec("tiny_f32", batch=1, q_len=1, heads=16, n_shards=4,
                     q_dtype="f32", kv_dtype="f32", out_dtype="f32",
                     context=1024, seed=101),
    "dense_bf16_32k": Spec("dense_bf16_32k", batch=32, q_len=1, heads=128,
                           n_shards=8, q_dtype="bf16", kv_dtype="bf16",
                           out_dtype="bf16", context=32768, seed=202),
    "dense_bf16_h64_32k": Spec("dense_bf16_h64_32k", batch=32, q_len=1, heads=64,
                               n_shards=8, q_dtype="bf16", kv_dtype="bf16",
                               out_dtype="bf16", context=32768, seed=212),
    "dense_fp8_mixed": Spec("dense_fp8_mixed", batch=64, q_len=1, heads=64,
                            n_shards=8, q_dtype="bf16", kv_dtype="fp8_ds",
                            out_dtype="bf16", ctx_range=(4096, 131072),
                            seed=303),
    "long_fp8_1m": Spec("long_fp8_1m", batch=4, q_len=1, heads=64, n_shards=8,
                        q_dtype="bf16", kv_dtype="fp8_ds", out_dtype="bf16",
                        context=1048576, seed=404),
    "sparse_fp8_topk2048": Spec("sparse_fp8_topk2048", batch=128, q_len=2,
                                heads=64, n_shards=8, q_dtype="bf16",
                                kv_dtype="fp8_ds", out_dtype="bf16",
                                context=262144, topk=2048, seed=505),
    # the same top-K step over a bf16 cache (a supported shape that runs on
    # the VALU kernel; measured, not one of the headline workloads)
    "sparse_bf16_topk2048": Spec("sparse_bf16_topk2048", batch=128, q_len=2,
                                 heads=64, n_shards=8, q_dtype="bf16",
                                 kv_dtype="bf16", out_dtype="bf16",
                                 context=262144, topk=2048, seed=515),
}


@dataclass
class Inputs:
    """Logical arrays of one decode step (host numpy).

    q            [B, Tq, H, 576]  float32, or uint16 bf16 bits
    context_lens [B] int64        tokens in each request's cache, including
                                  the query tokens' own rows
    row_offsets  [B + 1] int64    rows of request b are row_offsets[b]:row_offsets[b+1]
    row_pos      [T] int64        global position of each stored row
                                  (dense: 0..L_b-1; sparse: the sorted union
                                  of the request's selected positions)
    latent       [T, 512]  float32 | uint16 bf16 bits | uint8 E4M3FN codes
    scales       [T, 4]    float32 (fp8 only, else None)
    rope         [T, 64]   float32 | uint16 bf16 bits
    topk_idx     [B, Tq, K] int32 global indices, or None (dense)
    layout_seed  seed for the physical block order of the paged cache
    """
    spec: Spec
    q: np.ndarray
    context_lens: np.ndarray
    row_offsets: np.ndarray
    row_pos: np.ndarray
    latent: np.ndarray
    scales: object
    rope: np.ndarray
    topk_idx: object
    layout_seed: int = 0
    dense: bool = field(default=True)

    @property
    def total_rows(self):
        return int(self.row_offsets[-1])


def _bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_fp8_groups(x):
    """float32 [n, 512] -> (codes uint8 [n, 512], scales float32 [n, 4])."""
    n = x.shape[0]
    g = x.reshape(n, LATENT // FP8_GROUP, FP8_GROUP)
    amax = np.abs(g).max(axis=2)
    scales = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(g / scales[:, :, None], -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(y.reshape(n, LATENT)).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).numpy(), scales


def _context_lens(spec, rng):
    if spec.context:
        return np.full(spec.batch, spec.context, dtype=np.int64)
    lo, hi = spec.ctx_range
    return rng.integers(lo, hi + 1, size=spec.batch, dtype=np.int64)


def _draw_rows(spec, seed_words, n):
    """Draw n cache rows in the spec's storage format."""
    rng = np.random.default_rng(seed_words)
    lat = rng.standard_normal((n, LATENT), dtype=np.float32)
    rope = rng.standard_normal((n, ROPE), dtype=np.float32)
    if spec.kv_dtype == "f32":
        return lat, None, rope
    if spec.kv_dtype == "bf16":
        return _bf16_bits(lat), None, _bf16_bits(rope)
    codes, scales = quantize_fp8_groups(lat)
    return codes, scales, _bf16_bits(rope)


def generate(spec, threads=None):
    """Draw the logical inputs of `spec` (deterministic in spec.seed)."""
    root = np.random.default_rng([spec.seed, 0])
    lens = _context_lens(spec, root)
    B, Tq, H = spec.batch, spec.q_len, spec.heads
    if np.any(lens < Tq):
        raise ValueError("context shorter than the query tokens")

    qrng = np.random.default_rng([spec.seed, 1])
    q = qrng.standard_normal((B, Tq, H, DK), dtype=np.float32)
    if spec.q_dtype == "bf16":
        q = _bf16_bits(q)

    topk_idx = None
    if spec.topk:
        irng = np.random.default_rng([spec.seed, 2])
        topk_idx = np.full((B, Tq, spec.topk), -1, dtype=np.int32)
        pos_lists = []
        for b in range(B):
            for j in range(Tq):
                prefix = int(lens[b]) - Tq + j + 1
                k = min(spec.topk, prefix)
                topk_idx[b, j, :k] = irng.choice(prefix, size=k, replace=False)
            sel = topk_idx[b].reshape(-1)
            pos_lists.append(np.unique(sel[sel >= 0]).astype(np.int64))
    else:
        pos_lists = [np.arange(int(L), dtype=np.int64) for L in lens]

    counts = np.array([p.size for p in pos_lists], dtype=np.int64)
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    T = int(offsets[-1])
    row_pos = np.concatenate(pos_lists) if B else np.zeros(0, np.int64)

    if spec.kv_dtype == "f32":
        latent = np.empty((T, LATENT), np.float32)
        rope = np.empty((T, ROPE), np.float32)
        scales = None
    elif spec.kv_dtype == "bf16":
        latent = np.empty((T, LATENT), np.uint16)
        rope = np.empty((T, ROPE), np.uint16)
        scales = None
    elif spec.kv_dtype == "fp8_ds":
        latent = np.empty((T, LATENT), np.uint8)
        rope = np.empty((T, ROPE), np.uint16)
        scales = np.empty((T, LATENT // FP8_GROUP), np.float32)
    else:
        raise ValueError(spec.kv_dtype)

    tasks = []
    for b in range(B):
        for s0 in range(0, int(counts[b]), SLICE):
            tasks.append((b, s0, min(SLICE, int(counts[b]) - s0)))

    def run(task):
        b, s0, n = task
        lat, sc, rp = _draw_rows(spec, [spec.seed, 3, b, s0 // SLICE], n)
        r0 = int(offsets[b]) + s0
        latent[r0:r0 + n] = lat
        rope[r0:r0 + n] = rp
        if scales is not None:
            scales[r0:r0 + n] = sc

    nthreads = threads or min(16, os.cpu_count() or 1)
    if len(tasks) > 1 and nthreads > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(run, tasks))
    else:
        for t in tasks:
            run(t)

    return Inputs(spec=spec, q=q, context_lens=lens, row_offsets=offsets,
                  row_pos=row_pos, latent=latent, scales=scales, rope=rope,
                  topk_idx=topk_idx, layout_seed=spec.seed * 7919 + 17,
                  dense=not spec.topk)


# Cache writes: new tokens' rows (latent + rope) as a model layer hands them
# to the cache.  The long-context write stands in for filling one request's
# 1M-token cache (the shape of long_fp8_1m) from bf16 activations, with the
# tokens dealt round-robin over 8 shards.
WRITE_SPECS = {
    "kv_write_fp8_1m": dict(tokens=1048576, n_shards=8, src_dtype="bf16", kv_dtype="fp8_ds",
                            seed=606),
}


def new_token_rows(n, seed, dtype="bf16", spread=0):
    """Seeded [n, 576] rows of new cache tokens: float32, or uint16 bf16 bits.

    Entries are N(0, 1); with spread > 0 each row is multiplied by 2^k, k a
    uniform integer in [-spread, spread], so group maxima span many binades.
    """
    out = np.empty((n, DK), np.float32 if dtype == "f32" else np.uint16)
    for r0 in range(0, n, SLICE):
        m = min(SLICE, n - r0)
        rng = np.random.default_rng([seed, 7, r0 // SLICE])
        x = rng.standard_normal((m, DK), dtype=np.float32)
        if spread:
            x *= np.exp2(rng.integers(-spread, spread + 1, (m, 1))).astype(np.float32)
        out[r0:r0 + m] = x if dtype == "f32" else _bf16_bits(x)
    return out


# Indexer scores for top-K selection: the scoring model needs trained
# weights, so scores are seeded N(0, 1) draws over each request's whole
# context (global positions), optionally rounded to bf16 so that equal
# scores are common.  The selection workload has the shape of
# sparse_fp8_topk2048: 128 requests x 2 query tokens, context 262144,
# top-2048, 8 shards.
SELECT_SPECS = {
    "topk_select_262k": dict(batch=128, q_len=2, context=262144, topk=2048, n_shards=8, seed=707),
}


def indexer_scores(batch, q_len, context, seed, ties=False):
    """Seeded scores [batch][q_len][context] float32."""
    out = np.empty((batch, q_len, context), np.float32)
    for b in range(batch):
        rng = np.random.default_rng([seed, 9, b])
        x = rng.standard_normal((q_len, context), dtype=np.float32)
        if ties:
            x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
        out[b] = x
    return out


# Varlen decode: multi-token-prediction drafts give requests different query
# counts in one call.  The spec is the fp8 mixed-length cache generated with
# two query tokens per request; request b keeps its last counts[b] tokens,
# counts drawn uniformly from 1 .. q_len.
VARLEN_SPECS = {
    "varlen_fp8_mtp2": dict(base="dense_fp8_mixed", q_len=2, seed=808),
}


def varlen_counts(batch, q_len, seed):
    """Seeded query counts per request, each uniform on 1 .. q_len."""
    rng = np.random.default_rng([seed, 11])
    return rng.integers(1, q_len + 1, size=batch).astype(np.int64)
