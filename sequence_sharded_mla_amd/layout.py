"""Round-robin paged layout of the latent cache on the device.

One pool of 64-token blocks holds the cache rows of every shard.  Global
token p of request b belongs to shard p mod N, where it is local token
j = p div N ("How vLLM Serves GLM-5.3 with Million-Token Contexts on 16 H200s",
section "The core design": tokens are dealt round-robin, each rank keeping
1/N).  Each shard keeps its local tokens densely, in local order, in its own
blocks, and has its own block table [B][max_blocks]; the tables of the N
shards are stacked as [N][B][max_blocks].  Physical block ids come from one
seeded permutation of the pool, so consecutive local blocks are scattered.

Row formats (see include/mla_dcp.h): f32 576 x 4 B; bf16 576 x 2 B; fp8_ds
512 E4M3FN codes, 4 float32 group scales, 64 bf16 rope values (656 B).

Every byte of the pool that holds no cache row (the tail of each shard's
last block, blocks of positions a sparse workload never selects) is filled
with NaN patterns, so any read of an unowned or unused row shows up as NaN
in the output.

This module runs on the host and uses torch only to move bytes; it is the
cache writer of the test and benchmark harness, not part of the decode step.
"""

from dataclasses import dataclass

import numpy as np
import torch

from . import make_desc

ROW_BYTES = {"f32": 2304, "bf16": 1152, "fp8_ds": 656}
BLOCK = 64
UPLOAD_ROWS = 1 << 18


def poison_row(kv_dtype):
    """One row of NaN patterns in the given format (uint8)."""
    if kv_dtype == "f32":
        return np.tile(np.array([0x00, 0x00, 0xC0, 0x7F], np.uint8), 576)
    if kv_dtype == "bf16":
        return np.tile(np.array([0xC0, 0x7F], np.uint8), 576)
    codes = np.full(512, 0x7F, np.uint8)
    scales = np.tile(np.array([0x00, 0x00, 0xC0, 0x7F], np.uint8), 4)
    rope = np.tile(np.array([0xC0, 0x7F], np.uint8), 64)
    return np.concatenate([codes, scales, rope])


def pack_rows(kv_dtype, latent, scales, rope):
    """Logical row arrays -> packed row bytes [T, row_bytes] (uint8)."""
    T = latent.shape[0]
    parts = [np.ascontiguousarray(latent).view(np.uint8).reshape(T, -1)]
    if kv_dtype == "fp8_ds":
        parts.append(np.ascontiguousarray(scales).view(np.uint8).reshape(T, -1))
    parts.append(np.ascontiguousarray(rope).view(np.uint8).reshape(T, -1))
    out = np.concatenate(parts, axis=1)
    assert out.shape[1] == ROW_BYTES[kv_dtype]
    return out


def shard_local_lens(context_lens, n_shards):
    """[N, B] tokens each shard stores of each request (round-robin deal)."""
    L = np.asarray(context_lens, dtype=np.int64)
    s = np.arange(n_shards, dtype=np.int64)[:, None]
    return np.where(L[None, :] > s, (L[None, :] - s + n_shards - 1) // n_shards, 0)


@dataclass
class PagedCache:
    pool: torch.Tensor          # uint8 [pool_blocks, 64, row_bytes]
    block_tables: torch.Tensor  # int32 [N, B, max_blocks]
    context_lens: torch.Tensor  # int32 [B]
    q: torch.Tensor             # [B, Tq, H, 576] float32 or bfloat16
    topk_idx: object            # int32 [B, Tq, K] or None
    n_shards: int
    max_blocks: int
    tables_host: np.ndarray
    desc: object

    @property
    def pool_blocks(self):
        return self.pool.shape[0]


def build_block_tables(context_lens, n_shards, seed, extra_width=0):
    """Per-shard block tables over one shuffled pool.

    Returns (tables int32 [N, B, max_blocks] with -1 in unused entries,
    total blocks).  extra_width widens every row (unused entries stay -1).
    """
    loc = shard_local_lens(context_lens, n_shards)
    nblk = (loc + BLOCK - 1) // BLOCK
    B = loc.shape[1]
    max_blocks = max(1, int(nblk.max()) if nblk.size else 1) + extra_width
    total = int(nblk.sum())
    perm = np.random.default_rng(seed).permutation(max(total, 1)).astype(np.int32)
    tables = np.full((n_shards, B, max_blocks), -1, dtype=np.int32)
    flat = nblk.reshape(-1)
    starts = np.concatenate([[0], np.cumsum(flat)[:-1]]) if flat.size else flat
    for i, (n, st) in enumerate(zip(flat, starts)):
        s, b = divmod(i, B)
        tables[s, b, :n] = perm[st:st + n]
    return tables, max(total, 1)


def pack(x, device="cuda", extra_width=0):
    """Place the logical inputs `x` (workload.Inputs) in a paged device cache."""
    spec = x.spec
    N, B = spec.n_shards, spec.batch
    kv = spec.kv_dtype
    rb = ROW_BYTES[kv]
    tables, total = build_block_tables(x.context_lens, N, x.layout_seed, extra_width)
    max_blocks = tables.shape[2]

    pool = torch.empty((total, BLOCK, rb), dtype=torch.uint8, device=device)
    pool.view(-1, rb)[:] = torch.from_numpy(poison_row(kv)).to(device)

    counts = np.diff(x.row_offsets)
    req = np.repeat(np.arange(B, dtype=np.int64), counts)
    p = x.row_pos
    s = p % N
    j = p // N
    blk = tables[s, req, j // BLOCK].astype(np.int64)
    assert np.all(blk >= 0)
    dest = blk * BLOCK + j % BLOCK
    flat_pool = pool.view(-1, rb)
    for r0 in range(0, x.total_rows, UPLOAD_ROWS):
        r1 = min(r0 + UPLOAD_ROWS, x.total_rows)
        rows = pack_rows(kv, x.latent[r0:r1], None if x.scales is None else x.scales[r0:r1],
                         x.rope[r0:r1])
        flat_pool[torch.from_numpy(dest[r0:r1]).to(device)] = torch.from_numpy(rows).to(device)

    if spec.q_dtype == "f32":
        q = torch.from_numpy(np.ascontiguousarray(x.q)).to(device)
    else:
        q = torch.from_numpy(np.ascontiguousarray(x.q).view(np.int16)).to(device).view(torch.bfloat16)
    topk = None
    if x.topk_idx is not None:
        topk = torch.from_numpy(np.ascontiguousarray(x.topk_idx)).to(device)
    desc = make_desc(B, spec.q_len, spec.heads, max_blocks, total, spec.q_dtype, kv,
                     spec.out_dtype, spec.scale, topk=spec.topk)
    return PagedCache(pool=pool, block_tables=torch.from_numpy(tables).to(device),
                      context_lens=torch.from_numpy(x.context_lens.astype(np.int32)).to(device),
                      q=q, topk_idx=topk, n_shards=N, max_blocks=max_blocks,
                      tables_host=tables, desc=desc)


def shard_scores(scores, n_shards):
    """Global indexer scores [B][Tq][L] -> per-shard rows [N][B][Tq][ceil(L / N)].

    Entry j of shard s is the score of global position j * N + s (the scores
    a DCP rank computes for its own tokens); entries past the context are
    -inf.
    """
    B, Tq, L = scores.shape
    width = -(-L // n_shards)
    out = np.full((n_shards, B, Tq, width), -np.inf, dtype=np.float32)
    for s in range(n_shards):
        part = scores[:, :, s::n_shards]
        out[s, :, :, :part.shape[2]] = part
    return out
