"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Small workloads are compared element by element on every output (per-shard
partials and merged results); they span several 64-token tiles, ragged
tails, more shards than tokens, multi-chunk splitting and the sparse path
with its empty-shard rows.
"""
import numpy as np
import pytest
import torch

import workload
from oracle import attention, sharding
from sequence_sharded_mla_amd import (layout, mla_clear_device_error, mla_decode_partial,
                                      mla_get_device_error, mla_localize_indices, mla_lse_merge,
                                      MLA_DEVERR_BLOCK_TABLE, MLA_DEVERR_INDEX)
from sequence_sharded_mla_amd.step import ShardedDecodeStep

from gpu_cases import compare, run_gpu, say, to_np, TOL_LSE, TOL_O

pytestmark = pytest.mark.gpu

S = workload.SPECS


def test_tiny_f32_full():
    x = workload.generate(S["tiny_f32"])
    _, step = run_gpu(x)
    errs = compare(x, step)
    # float32 path: well inside the bar.  O within 1e-5; LSE within 2e-6:
    # a shard's LSE here is about 6.5, where one float32 ulp is 4.8e-7, and
    # the float32 sum of its 256 exponentials carries a relative rounding
    # of about sqrt(256) * 2^-24 -- a few ulps of LSE (1e-6 is not reachable
    # in float32 for every row).
    assert errs["o"] < 1e-5 and errs["o_shards"] < 1e-5
    assert errs["lse"] < 2e-6 and errs["lse_shards"] < 2e-6


@pytest.mark.parametrize("kv,heads", [("bf16", 128), ("bf16", 64), ("bf16", 16), ("fp8_ds", 64), ("fp8_ds", 128),
                                      ("f32", 16)])
def test_tile_boundary_lengths(kv, heads):
    """Local lengths at and around the 32-token sub-tile and the 64-token
    block: requests whose context puts 31, 32, 33, 63, 64, 65, 127, 128 and
    129 tokens on shard 0 (context = N * local - k), and contexts N does not
    divide, so the shards' lengths differ by one."""
    N = 8
    lens = [N * n - k for n in (31, 32, 33, 63, 64, 65, 127, 128, 129) for k in (0, 3)]
    lens += [63, 64, 65, 511, 513]
    qd = "f32" if kv == "f32" else "bf16"
    sp = S["dense_bf16_32k"].with_(batch=len(lens), heads=heads, kv_dtype=kv, q_dtype=qd, out_dtype=qd,
                                   context=0, ctx_range=(1, 2), seed=31 + heads)
    x = workload.generate(sp)
    x = _with_lengths(x, lens)
    say(f"tile boundaries {kv} H={heads}: lens {lens}")
    _, step = run_gpu(x)
    compare(x, step)


def _with_lengths(x, lens):
    """The same spec redrawn with the given context lengths."""
    sp = x.spec
    g = workload.generate(sp.with_(batch=len(lens), context=0, ctx_range=(max(lens), max(lens))))
    keep = []
    for b, L in enumerate(lens):
        r0 = int(g.row_offsets[b])
        keep.append(np.arange(r0, r0 + L))
    keep = np.concatenate(keep)
    g.latent, g.rope = g.latent[keep], g.rope[keep]
    if g.scales is not None:
        g.scales = g.scales[keep]
    g.row_pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int64)
    g.row_offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    g.context_lens = np.asarray(lens, dtype=np.int64)
    return g


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
def test_dense_bf16_heads(heads):
    sp = S["dense_bf16_32k"].with_(batch=3, heads=heads, context=0, ctx_range=(1, 5000), seed=11 + heads)
    x = workload.generate(sp)
    _, step = run_gpu(x)
    compare(x, step)


def test_dense_bf16_ragged_lengths():
    sp = S["dense_bf16_32k"].with_(batch=6, context=0, ctx_range=(1, 9), seed=3)
    x = workload.generate(sp)   # fewer tokens than shards
    _, step = run_gpu(x)
    compare(x, step)
    sp = S["dense_bf16_32k"].with_(batch=4, context=0, ctx_range=(4095, 4097 + 64 * 8), seed=4)
    x = workload.generate(sp)
    _, step = run_gpu(x)
    compare(x, step)


def test_dense_fp8_mixed_small():
    sp = S["dense_fp8_mixed"].with_(batch=5, ctx_range=(1, 6000), seed=5)
    x = workload.generate(sp)
    _, step = run_gpu(x)
    compare(x, step)


def test_dense_fp8_multi_chunk():
    # one long request: the shard rows are split into chunks and recombined
    sp = S["long_fp8_1m"].with_(batch=1, context=300_001, seed=6)
    x = workload.generate(sp)
    _, step = run_gpu(x)
    compare(x, step)


def test_dense_multi_query_tokens():
    sp = S["dense_fp8_mixed"].with_(batch=3, q_len=3, ctx_range=(3, 700), seed=7)
    x = workload.generate(sp)
    _, step = run_gpu(x)
    compare(x, step)


@pytest.mark.parametrize("n_shards", [1, 2, 3, 8, 16])
def test_shard_counts(n_shards):
    sp = S["dense_bf16_32k"].with_(batch=2, heads=64, n_shards=n_shards, context=0,
                                   ctx_range=(900, 1300), seed=8 + n_shards)
    x = workload.generate(sp)
    _, step = run_gpu(x)
    compare(x, step)
    if n_shards == 1:
        assert torch.equal(step.o_partials[0], step.o)


def test_sparse_small():
    sp = S["sparse_fp8_topk2048"].with_(batch=3, context=5000, topk=256, seed=9)
    x = workload.generate(sp)
    _, step = run_gpu(x)
    compare(x, step)


def test_sparse_empty_shards_and_padding():
    sp = S["sparse_fp8_topk2048"].with_(batch=2, context=3000, topk=64, seed=10)
    x = workload.generate(sp)
    N = sp.n_shards
    # request 0, token 0: every selection on shard 3; token 1: no valid entry
    own = np.arange(3, 2998, N)[:64]
    x.topk_idx[0, 0] = own
    x.topk_idx[0, 1] = -1
    x.topk_idx[1, 0, 10:] = -1
    # rows for the newly selected positions: re-draw every stored row
    x = _reselect(x)
    _, step = run_gpu(x)
    compare(x, step)
    lse = to_np(step.lses).reshape(N, 2, 2, sp.heads)
    for s in range(N):
        if s != 3:
            assert np.all(np.isneginf(lse[s, 0, 0]))
            assert torch.count_nonzero(step.o_partials.view(N, 2, 2, sp.heads, 512)[s, 0, 0]) == 0
    assert np.all(np.isneginf(to_np(step.lse).reshape(2, 2, sp.heads)[0, 1]))


@pytest.mark.parametrize("kv,heads", [("fp8_ds", 64), ("fp8_ds", 128), ("fp8_ds", 16), ("bf16", 64)])
def test_sparse_repeated_positions(kv, heads):
    """A position listed more than once is attended once per entry (the
    list is a multiset), on the matrix-core sparse kernel (fp8, 64 and 128
    heads) and the VALU one (fp8 with 16 heads, bf16)."""
    sp = S["sparse_fp8_topk2048"].with_(batch=2, context=3000, topk=256, heads=heads, kv_dtype=kv,
                                        seed=21 + heads)
    x = workload.generate(sp)
    idx = x.topk_idx
    idx[0, 0, 10:40] = idx[0, 0, 40:70]     # 30 positions listed twice
    idx[0, 1, 0:3] = idx[0, 1, 5]           # one position four times
    idx[1, 0, :] = idx[1, 0, 7]             # one position, every entry
    idx[1, 1, 100:] = -1
    idx[1, 1, 50:100] = idx[1, 1, 0:50]     # duplicates next to padding
    say(f"sparse repeated positions {kv} H={heads}")
    _, step = run_gpu(x)
    compare(x, step)


@pytest.mark.parametrize("heads,n_shards", [(64, 1), (128, 1), (64, 2), (128, 2)])
def test_sparse_full_list_one_owner(heads, n_shards):
    """The longest top-K list the matrix-core sparse kernel keeps in LDS
    (2048 entries), every entry owned by the last shard: each wave keeps its
    whole slice, and with two shards the first shard's workgroup drops every
    entry (an empty row, (0, -inf))."""
    N = n_shards
    ctx = 2048 * N + 300
    sp = S["sparse_fp8_topk2048"].with_(batch=1, context=ctx, topk=2048, heads=heads, n_shards=N,
                                        seed=31 + heads + N)
    x = workload.generate(sp)
    rng = np.random.default_rng(77)
    for t in range(sp.q_len):
        vis = ctx - sp.q_len + t + 1
        x.topk_idx[0, t] = rng.permutation(np.arange(N - 1, vis, N))[:2048]
    x = _reselect(x)
    say(f"sparse full list, one owner: H={heads} N={N}")
    _, step = run_gpu(x)
    compare(x, step)
    if N == 2:
        assert np.all(np.isneginf(to_np(step.lses).reshape(N, 1, sp.q_len, heads)[0]))


def _reselect(x):
    """Regenerate stored rows after editing topk_idx (materialise the union)."""
    sp = x.spec
    rng = np.random.default_rng(1234)
    pos_lists = []
    for b in range(sp.batch):
        sel = x.topk_idx[b].reshape(-1)
        pos_lists.append(np.unique(sel[sel >= 0]).astype(np.int64))
    counts = np.array([p.size for p in pos_lists])
    offs = np.concatenate([[0], np.cumsum(counts)])
    T = int(offs[-1])
    lat = rng.standard_normal((T, 512), dtype=np.float32)
    if sp.kv_dtype == "bf16":
        codes, scales = workload._bf16_bits(lat), None
    else:
        codes, scales = workload.quantize_fp8_groups(lat)
    rope = workload._bf16_bits(rng.standard_normal((T, 64), dtype=np.float32))
    x.row_offsets, x.row_pos = offs, np.concatenate(pos_lists)
    x.latent, x.scales, x.rope = codes, scales, rope
    return x


def test_single_shard_entry_matches_shards_call():
    sp = S["dense_fp8_mixed"].with_(batch=3, ctx_range=(100, 3000), seed=12)
    x = workload.generate(sp)
    cache, step = run_gpu(x)
    d = cache.desc
    from sequence_sharded_mla_amd import alloc_workspace
    ws = alloc_workspace(d, 1)
    for s in (0, 5):
        o = torch.empty_like(step.o_partials[s])
        l = torch.empty_like(step.lses[s])
        mla_decode_partial(d, cache.q, cache.pool, cache.block_tables[s].contiguous(),
                           cache.context_lens, None, s, sp.n_shards, o, l, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, step.o_partials[s]) and torch.equal(l, step.lses[s])


@pytest.mark.parametrize("name,kw", [
    ("dense_bf16_32k", dict(batch=4, seed=14)),                       # 4 rows x 4096 tokens
    ("long_fp8_1m", dict(batch=1, context=300_000, seed=15)),         # 1 row x 37500 tokens
])
def test_single_shard_call_splits_rows_to_fill_the_chip(name, kw):
    """One rank's call with fewer rows than the chip holds workgroups: the
    plan splits rows down to 512-token chunks, and the shard's partials still
    match the oracle's."""
    from oracle import decode as odecode
    from sequence_sharded_mla_amd import alloc_workspace
    from gpu_cases import max_err, oracle_for
    sp = S[name].with_(**kw)
    say(f"single-shard {sp.name} {kw}")
    x = workload.generate(sp)
    cache = layout.pack(x, device="cuda")
    d = cache.desc
    ws = alloc_workspace(d, 1)
    s = 3
    rows = sp.batch * sp.q_len
    dt = torch.bfloat16 if sp.out_dtype == "bf16" else torch.float32
    o = torch.empty((rows, sp.heads, 512), dtype=dt, device="cuda")
    l = torch.empty((rows, sp.heads), dtype=torch.float32, device="cuda")
    mla_decode_partial(d, cache.q, cache.pool, cache.block_tables[s].contiguous(), cache.context_lens,
                       None, s, sp.n_shards, o, l, ws)
    torch.cuda.synchronize()
    hdr = ws[:256].cpu().numpy().view(np.int32)
    say(f"  items {hdr[1]} chunk {hdr[2]}")
    assert hdr[2] < 4096 and hdr[1] > rows       # split below the large-call floor
    assert mla_get_device_error(ws) == 0
    ref = odecode.mla_decode(odecode.query_to_f64(x.q, sp.q_dtype),
                             odecode.storage_rows(sp.kv_dtype, x.latent, x.scales, x.rope,
                                                  x.row_offsets, x.row_pos),
                             x.context_lens, sp.q_len, sp.n_shards, sp.scale, shards=[s], full=False)
    eo = max_err(to_np(o).reshape(sp.batch, sp.q_len, sp.heads, 512), ref["o_shards"][0])
    el = max_err(to_np(l).reshape(sp.batch, sp.q_len, sp.heads), ref["lse_shards"][0])
    say(f"  o={eo:.3e} lse={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


def test_bitwise_reproducible():
    sp = S["dense_fp8_mixed"].with_(batch=4, ctx_range=(1000, 9000), seed=13)
    x = workload.generate(sp)
    cache, step = run_gpu(x)
    o1, l1 = step.o.clone(), step.lse.clone()
    p1 = step.o_partials.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(o1, step.o) and torch.equal(l1, step.lse) and torch.equal(p1, step.o_partials)


def test_lse_merge_entry():
    rng = np.random.default_rng(14)
    n, rows = 8, 300
    o = rng.standard_normal((n, rows, 512)).astype(np.float32)
    l = (rng.standard_normal((n, rows)) * 5).astype(np.float32)
    l[:, :7] = -np.inf            # all parts empty
    l[2:, 7:20] = -np.inf         # some parts empty
    o[2:, 7:20] = np.nan          # empty parts' outputs are never read
    for pd in (torch.float32, torch.bfloat16):
        ot = torch.from_numpy(o).cuda().to(pd)
        src = ot.float().cpu().numpy().astype(np.float64)
        ref_o, ref_l = attention.merge(np.nan_to_num(src), l.astype(np.float64))
        out = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
        lo = torch.empty(rows, dtype=torch.float32, device="cuda")
        mla_lse_merge(ot, torch.from_numpy(l).cuda(), out, lo)
        torch.cuda.synchronize()
        got = to_np(out)
        assert not np.isnan(got).any()
        assert np.abs(got - ref_o).max() <= 2 ** -8 * max(1.0, np.abs(ref_o).max())
        gl = lo.cpu().numpy()
        assert np.array_equal(np.isneginf(gl), np.isneginf(ref_l))
        fin = np.isfinite(ref_l)
        assert np.abs(gl[fin] - ref_l[fin]).max() < 1e-5


def test_localize_bit_exact():
    rng = np.random.default_rng(15)
    g = rng.integers(-5, 1 << 20, size=300_001).astype(np.int32)
    gt = torch.from_numpy(g).cuda()
    out = torch.empty_like(gt)
    for N in (1, 3, 8):
        for s in range(N):
            mla_localize_indices(gt, s, N, out)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), sharding.localize(g, s, N))


def test_device_error_narrow_block_table():
    sp = S["dense_bf16_32k"].with_(batch=2, heads=64, context=0, ctx_range=(3000, 3000), seed=16)
    x = workload.generate(sp)
    cache = layout.pack(x, device="cuda")
    # a table one block too narrow for the longest shard
    narrow = cache.block_tables[:, :, :-1].contiguous()
    cache.block_tables = narrow
    cache.desc.max_blocks = narrow.shape[2]
    step = ShardedDecodeStep(cache, sp.out_dtype)
    step()
    torch.cuda.synchronize()
    assert mla_get_device_error(step.workspace) & MLA_DEVERR_BLOCK_TABLE
    mla_clear_device_error(step.workspace)
    assert mla_get_device_error(step.workspace) == 0


def test_device_error_index_beyond_prefix():
    sp = S["sparse_fp8_topk2048"].with_(batch=1, context=1000, topk=16, seed=17)
    x = workload.generate(sp)
    cache = layout.pack(x, device="cuda")
    bad = cache.topk_idx.clone()
    bad[0, 0, 0] = 999  # query 0 sees positions 0..998
    cache.topk_idx = bad
    step = ShardedDecodeStep(cache, sp.out_dtype)
    step()
    torch.cuda.synchronize()
    assert mla_get_device_error(step.workspace) & MLA_DEVERR_INDEX
    # the offending entry is skipped: result equals the oracle without it
    x.topk_idx = bad.cpu().numpy()
    x.topk_idx[0, 0, 0] = -1
    mla_clear_device_error(step.workspace)
    compare(x, step)


def test_bf16_h128_bitwise_reproducible_and_chunked():
    # one long request forces several chunks per shard row (chunk combine)
    sp = S["dense_bf16_32k"].with_(batch=1, context=600_000, seed=18)
    x = workload.generate(sp)
    cache, step = run_gpu(x)
    compare(x, step)
    o1, p1 = step.o.clone(), step.o_partials.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(o1, step.o) and torch.equal(p1, step.o_partials)


@pytest.mark.parametrize("heads", [64, 128])
def test_bad_block_id_is_skipped(heads):
    sp = S["dense_bf16_32k"].with_(batch=2, heads=heads, context=0, ctx_range=(5000, 5000), seed=19)
    x = workload.generate(sp)
    cache = layout.pack(x, device="cuda")
    N = sp.n_shards
    bt = cache.block_tables.clone()
    bt[2, 0, 3] = -7                     # shard 2, request 0, local block 3
    bt[5, 1, 0] = cache.pool_blocks      # shard 5, request 1, local block 0
    cache.block_tables = bt
    step = ShardedDecodeStep(cache, sp.out_dtype)
    step()
    torch.cuda.synchronize()
    assert mla_get_device_error(step.workspace) & MLA_DEVERR_BLOCK_TABLE
    from oracle import decode as odecode
    q = odecode.query_to_f64(x.q, sp.q_dtype)
    rows = odecode.storage_rows(sp.kv_dtype, x.latent, x.scales, x.rope, x.row_offsets, x.row_pos)
    H = sp.heads
    o_sh = to_np(step.o_partials).reshape(N, 2, H, 512)
    l_sh = to_np(step.lses).reshape(N, 2, H)
    for s, b, blk in ((2, 0, 3), (5, 1, 0)):
        L = int(x.context_lens[b])
        owned = [p for p in range(L) if p % N == s and not (blk * 64 <= p // N < blk * 64 + 64)]
        lat, rope = rows(b, np.array(owned))
        k = np.concatenate([lat, rope], axis=1)
        o_ref, l_ref = attention.attend(q[b, 0], k, lat, sp.scale)
        assert np.abs(o_sh[s, b] - o_ref).max() <= TOL_O
        assert np.abs(l_sh[s, b] - l_ref).max() <= TOL_LSE


@pytest.mark.parametrize("topk", [0, 300])
def test_fp8_128_heads(topk):
    if topk:
        sp = S["sparse_fp8_topk2048"].with_(batch=2, heads=128, context=4000, topk=topk, seed=20)
    else:
        sp = S["dense_fp8_mixed"].with_(batch=3, heads=128, ctx_range=(50, 5000), seed=21)
    x = workload.generate(sp)
    _, step = run_gpu(x)
    compare(x, step)


def test_sparse_topk_beyond_lds_list():
    # more top-K entries than the matrix-core path keeps in LDS
    sp = S["sparse_fp8_topk2048"].with_(batch=1, context=40000, topk=2500, seed=22)
    x = workload.generate(sp)
    _, step = run_gpu(x)
    compare(x, step)


def test_fp8_zero_scale_groups_and_bad_block():
    sp = S["dense_fp8_mixed"].with_(batch=2, ctx_range=(3000, 3000), seed=23)
    x = workload.generate(sp)
    x.scales[:50, 1] = 0.0          # a whole group of some rows scaled to zero
    cache = layout.pack(x, device="cuda")
    bt = cache.block_tables.clone()
    bt[1, 1, 2] = -1                 # shard 1, request 1, local block 2
    cache.block_tables = bt
    step = ShardedDecodeStep(cache, sp.out_dtype)
    step()
    torch.cuda.synchronize()
    assert mla_get_device_error(step.workspace) & MLA_DEVERR_BLOCK_TABLE
    o_sh = to_np(step.o_partials).reshape(sp.n_shards, 2, sp.heads, 512)
    assert np.isfinite(o_sh).all()
    # shard 0 is untouched by the bad block: compare it with the oracle
    from gpu_cases import oracle_for, max_err
    ref = oracle_for(x, full=False)
    assert max_err(o_sh[0], ref["o_shards"][0][:, 0]) <= TOL_O


def test_chunk_combine_more_than_64_chunks():
    # one shard holding 266K tokens: the row splits into more than 64 chunks,
    # so the combine runs its weights in two groups of parts
    sp = S["long_fp8_1m"].with_(batch=1, n_shards=1, context=65 * 4096 + 100, seed=12)
    x = workload.generate(sp)
    cache, step = run_gpu(x)
    rows = sp.batch * sp.q_len
    assert step.workspace.numel() > 64 * rows * sp.heads * 512 * 4, "expected > 64 chunks"
    compare(x, step)


# ---- top-K steps over a bf16 cache: list pass + matrix-core kernel ---------


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
def test_bf16_sparse(heads):
    sp = S["sparse_bf16_topk2048"].with_(batch=3, context=5000, topk=256, heads=heads, seed=40 + heads)
    say(f"bf16 sparse H={heads}")
    x = workload.generate(sp)
    _, step = run_gpu(x)
    compare(x, step)


def test_bf16_sparse_empty_shards_padding_and_long_list():
    """Every entry of one token on one shard, a token with no entry, padding
    mid-list, and a list longer than the fp8 kernel keeps in LDS."""
    sp = S["sparse_bf16_topk2048"].with_(batch=2, context=40000, topk=2500, heads=64, seed=50)
    x = workload.generate(sp)
    N = sp.n_shards
    x.topk_idx[0, 0] = np.random.default_rng(5).permutation(np.arange(3, 39990, N))[:2500]
    x.topk_idx[0, 1] = -1
    x.topk_idx[1, 0, 100:] = -1
    x = _reselect(x)
    _, step = run_gpu(x)
    compare(x, step)
    lse = to_np(step.lses).reshape(N, 2, 2, sp.heads)
    for s in range(N):
        if s != 3:
            assert np.all(np.isneginf(lse[s, 0, 0]))
    assert np.all(np.isneginf(to_np(step.lse).reshape(2, 2, sp.heads)[0, 1]))


@pytest.mark.parametrize("heads,n_shards", [(64, 1), (128, 2)])
def test_bf16_sparse_full_list_one_owner(heads, n_shards):
    N = n_shards
    ctx = 2048 * N + 300
    sp = S["sparse_bf16_topk2048"].with_(batch=1, context=ctx, topk=2048, heads=heads, n_shards=N,
                                         seed=60 + heads + N)
    x = workload.generate(sp)
    rng = np.random.default_rng(78)
    for t in range(sp.q_len):
        vis = ctx - sp.q_len + t + 1
        x.topk_idx[0, t] = rng.permutation(np.arange(N - 1, vis, N))[:2048]
    x = _reselect(x)
    _, step = run_gpu(x)
    compare(x, step)


def test_bf16_sparse_errors_and_single_shard_call():
    """An entry past its token's prefix (MLA_DEVERR_INDEX) and a block id
    outside the pool (MLA_DEVERR_BLOCK_TABLE): the offending entries are
    dropped and every other result matches the oracle without them; one
    shard's own call gives that shard's partials bit for bit."""
    from sequence_sharded_mla_amd import MLA_DEVERR_BLOCK_TABLE, MLA_DEVERR_INDEX, alloc_workspace
    sp = S["sparse_bf16_topk2048"].with_(batch=2, context=3000, topk=300, heads=64, seed=70)
    x = workload.generate(sp)
    N = sp.n_shards
    cache = layout.pack(x, device="cuda")
    idx = cache.topk_idx.clone()
    idx[0, 0, 5] = 3000                # past the prefix of request 0's last token (2999 positions)
    cache.topk_idx = idx
    bt = cache.block_tables.clone()
    bt[5, 1, 0] = cache.pool_blocks    # shard 5, request 1, local block 0
    cache.block_tables = bt
    step = ShardedDecodeStep(cache, sp.out_dtype)
    step()
    torch.cuda.synchronize()
    err = mla_get_device_error(step.workspace)
    assert err & MLA_DEVERR_INDEX and err & MLA_DEVERR_BLOCK_TABLE
    mla_clear_device_error(step.workspace)
    g = idx.cpu().numpy()
    g[0, 0, 5] = -1
    drop = (g[1] >= 0) & (g[1] % N == 5) & ((g[1] // N) // 64 == 0)
    g[1][drop] = -1
    assert drop.any()
    x.topk_idx = g
    compare(x, step)
    d = cache.desc
    ws = alloc_workspace(d, 1)
    for s in (0, 5):
        o = torch.empty_like(step.o_partials[s])
        l = torch.empty_like(step.lses[s])
        mla_decode_partial(d, cache.q, cache.pool, cache.block_tables[s].contiguous(), cache.context_lens,
                           cache.topk_idx, s, N, o, l, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, step.o_partials[s]) and torch.equal(l, step.lses[s])
