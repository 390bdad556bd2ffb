"""GPU parity of the cache-write calls against the oracle, bit for bit.

mla_dcp_slot_mapping and mla_kv_write run through the C ABI on seeded
inputs; the oracle (oracle/kv_write.py) computes the expected slots and the
expected bytes of the whole pool.  Codes, scales, bf16 values and slots are
integers or bit patterns, so the bar is equality.  The sweep cases drive the
E4M3FN rounding over every bfloat16 value up to 448 and the float32
divisions through exact E4M3 midpoints; the end-to-end cases write a
request's newest token through the per-shard calls and decode over it.
"""

import numpy as np
import pytest
import torch

import workload
from oracle import codecs, kv_write as okw
from sequence_sharded_mla_amd import (MLA_DEVERR_BLOCK_TABLE, MLA_DEVERR_SLOT, layout,
                                      mla_clear_device_error, mla_dcp_kv_write, mla_dcp_slot_mapping,
                                      mla_get_device_error, mla_kv_write)
from sequence_sharded_mla_amd.step import ShardedDecodeStep

from gpu_cases import compare, say

pytestmark = pytest.mark.gpu

ROWB = okw.ROW_BYTES


def dev_src(rows, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(rows, np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(rows, np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def host_f32(rows, dtype):
    if dtype == "f32":
        return np.asarray(rows, np.float32)
    return (np.asarray(rows, np.uint16).astype(np.uint32) << 16).view(np.float32)


def new_ws():
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    mla_clear_device_error(ws)
    return ws


def gpu_write(src_rows, src_dtype, slots, pool_np, kv_dtype):
    pool = torch.from_numpy(pool_np.copy()).cuda()
    ws = new_ws()
    sl = torch.from_numpy(np.asarray(slots, np.int64)).cuda()
    mla_kv_write(dev_src(src_rows, src_dtype), sl, pool, kv_dtype,
                 pool_np.size // (64 * ROWB[kv_dtype]), workspace=ws)
    torch.cuda.synchronize()
    return pool.cpu().numpy(), mla_get_device_error(ws)


def check_write(src_rows, src_dtype, slots, kv_dtype, pool_blocks, seed, expect_err=0):
    rb = ROWB[kv_dtype]
    pool_np = np.random.default_rng(seed).integers(0, 256, pool_blocks * 64 * rb, dtype=np.uint8)
    got, err = gpu_write(src_rows, src_dtype, slots, pool_np, kv_dtype)
    ref, bad = okw.kv_write(pool_np, kv_dtype, host_f32(src_rows, src_dtype), slots)
    diff = np.nonzero(got != ref)[0]
    if diff.size:
        r = int(diff[0]) // rb
        say(f"first differing byte {diff[0]} (row {r}, byte {int(diff[0]) % rb}); "
            f"{diff.size} bytes differ")
    assert diff.size == 0
    assert err == (MLA_DEVERR_SLOT if bad.any() else 0) | expect_err
    return got


@pytest.mark.parametrize("src_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kv_dtype", ["fp8_ds", "bf16", "f32"])
def test_write_matches_oracle_bit_exact(src_dtype, kv_dtype):
    say(f"kv_write parity src={src_dtype} kv={kv_dtype}")
    T, blocks = 301, 16
    rows = workload.new_token_rows(T, seed=11, dtype=src_dtype, spread=20)
    if src_dtype == "f32":
        rows[3, :128] = 0.0
        rows[3, 7] = -0.0
        rows[4, 128:256] = -0.0
        rows[5] *= np.float32(2.0 ** 110)           # group scales above 2^100
        rows[6] *= np.float32(2.0 ** -90)           # group scales below 2^-80
    else:
        rows[3, :128] = 0
        rows[3, 7] = 0x8000
        rows[4, 128:256] = 0x8000
        for r, k in ((5, 110), (6, -90)):           # exact power-of-two rescaling
            rows[r] = ((host_f32(rows[r], "bf16") * np.float32(2.0 ** k)).view(np.uint32) >> 16).astype(np.uint16)
    rng = np.random.default_rng(12)
    slots = rng.permutation(blocks * 64)[:T].astype(np.int64)
    slots[::5] = -1
    slots[9] = blocks * 64 + 3                     # past the pool: flagged, not written
    check_write(rows, src_dtype, slots, kv_dtype, blocks, seed=13)


def sweep_rows(values, lead):
    """Groups of 127 sweep values, each led by `lead` (the group maximum)."""
    per = 127
    n_groups = -(-values.size // per)
    n_groups += (-n_groups) % 4                     # whole tokens of 4 groups
    g = np.zeros((n_groups, 128), values.dtype)
    g[:, 0] = lead
    flat = g[:, 1:].reshape(-1)
    flat[:values.size] = values
    g[:, 1:] = flat.reshape(n_groups, per)
    lat = g.reshape(-1, 512)
    rope = np.zeros((lat.shape[0], 64), values.dtype)
    return np.concatenate([lat, rope], axis=1)


def test_fp8_codes_for_every_bf16_value_up_to_448():
    say("kv_write fp8 sweep over bf16 values")
    pos = np.arange(0, 0x43E1, dtype=np.uint16)          # +0 .. 448 as bf16 patterns
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    rows = sweep_rows(vals, np.uint16(0x43E0))           # lead 448: scale 1, quotient exact
    slots = np.arange(rows.shape[0], dtype=np.int64)
    blocks = -(-rows.shape[0] // 64)
    check_write(rows, "bf16", slots, "fp8_ds", blocks, seed=14)
    # lead 448 * 2^9: scale 2^9, quotients still exact powers-of-two shifts
    shifted = (vals.astype(np.uint32) + (9 << 7)).astype(np.uint16)
    keep = (vals & 0x7F80) != 0                          # normals only (exact shift)
    rows = sweep_rows(shifted[keep], np.uint16(0x43E0 + (9 << 7)))
    check_write(rows, "bf16", np.arange(rows.shape[0], dtype=np.int64), "fp8_ds",
                -(-rows.shape[0] // 64), seed=15)


def test_fp8_quotients_at_and_around_every_midpoint():
    say("kv_write fp8 midpoints")
    pos = codecs.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(16)
    rows = []
    for amax in rng.uniform(0.01, 1000.0, 24).astype(np.float32):
        s = np.float32(amax / np.float32(448.0))
        x = (mids * np.float64(s)).astype(np.float32)
        up1 = np.nextafter(x, np.float32(np.inf))
        up2 = np.nextafter(up1, np.float32(np.inf))
        dn1 = np.nextafter(x, np.float32(0))
        dn2 = np.nextafter(dn1, np.float32(0))
        vals = np.concatenate([x, up1, up2, dn1, dn2])
        vals = np.concatenate([vals, -vals]).astype(np.float32)
        vals = vals[np.abs(vals) <= amax]
        rows.append(sweep_rows(vals, amax))
    rows = np.concatenate(rows).astype(np.float32)
    slots = np.arange(rows.shape[0], dtype=np.int64)
    check_write(rows, "f32", slots, "fp8_ds", -(-rows.shape[0] // 64), seed=17)


@pytest.mark.parametrize("src_dtype", ["bf16", "f32"])
def test_fp8_tiny_groups(src_dtype):
    """Group maxima in the subnormal range: float32 subnormal scales and
    quotients that saturate at 448."""
    say(f"kv_write fp8 tiny groups src={src_dtype}")
    rng = np.random.default_rng(18)
    T = 64
    if src_dtype == "bf16":
        # bf16 subnormals and the least normals; per-token limits put some
        # group maxima as low as 2^-133 (the least bf16 subnormal)
        limit = np.exp2(np.linspace(0, 8, T)).astype(np.int64)[:, None]
        rows = (rng.random((T, 576)) * (limit + 1)).astype(np.uint16)
        rows[rng.random((T, 576)) < 0.5] |= np.uint16(0x8000)
    else:
        mag = np.exp2(rng.uniform(-149, -110, (T, 576))).astype(np.float32)
        rows = np.where(rng.random((T, 576)) < 0.5, -mag, mag).astype(np.float32)
    check_write(rows, src_dtype, np.arange(T, dtype=np.int64), "fp8_ds", 1, seed=19)


def test_slot_mapping_matches_oracle():
    N, B, mb, pool = 8, 5, 7, 400
    ids = np.random.default_rng(20).permutation(pool)[: N * B * mb].astype(np.int32)
    bt = ids.reshape(N, B, mb)
    bt[2, 1, 3] = pool                              # outside the pool
    bt[5, 4, 0] = -1
    rng = np.random.default_rng(21)
    T = 5000
    req = rng.integers(-1, B + 1, T).astype(np.int32)
    pos = rng.integers(-5, N * mb * 64 + 300, T).astype(np.int32)
    for begin, count in [(0, 8), (3, 1), (2, 4), (7, 1)]:
        say(f"slot mapping shards {begin}..{begin + count - 1}")
        ws = new_ws()
        out = torch.full((T,), 99, dtype=torch.int64, device="cuda")
        mla_dcp_slot_mapping(torch.from_numpy(req).cuda(), torch.from_numpy(pos).cuda(),
                             torch.from_numpy(np.ascontiguousarray(bt[begin:begin + count])).cuda(),
                             begin, N, pool, out, workspace=ws)
        torch.cuda.synchronize()
        ref, bad = okw.dcp_slot_mapping(req, pos, bt[begin:begin + count], begin, count, N, pool)
        assert np.array_equal(out.cpu().numpy(), ref)
        assert mla_get_device_error(ws) == (MLA_DEVERR_BLOCK_TABLE if bad.any() else 0)


@pytest.mark.parametrize("src_dtype,kv_dtype", [("bf16", "fp8_ds"), ("f32", "bf16"), ("bf16", "f32")])
def test_fused_write_matches_oracle(src_dtype, kv_dtype):
    """mla_dcp_kv_write: the oracle's slot mapping followed by its write, for
    every shard range a rank or the emulation uses, with padding, tokens past
    the table and a block id outside the pool."""
    N, B, mb, pool = 8, 3, 5, 150
    ids = np.random.default_rng(25).permutation(pool)[: N * B * mb].astype(np.int32)
    bt = ids.reshape(N, B, mb)
    bt[4, 2, 1] = pool + 7                          # outside the pool
    rng = np.random.default_rng(26)
    T = 1003                                        # not a multiple of 8 or 64
    # distinct (request, position) pairs, so no two tokens share a slot;
    # then padding: negative positions and request ids outside the batch
    span = N * mb * 64 + 200
    pick = rng.choice(B * span, T, replace=False)
    req = (pick // span).astype(np.int32)
    pos = (pick % span).astype(np.int32)
    pos[rng.random(T) < 0.05] = -1
    req[rng.random(T) < 0.03] = B
    rows = workload.new_token_rows(T, seed=27, dtype=src_dtype, spread=6)
    rb = ROWB[kv_dtype]
    pool_np = np.random.default_rng(28).integers(0, 256, pool * 64 * rb, dtype=np.uint8)
    for begin, count in [(0, 8), (0, 1), (5, 1), (2, 3)]:
        say(f"fused write src={src_dtype} kv={kv_dtype} shards {begin}..{begin + count - 1}")
        tab = bt[begin:begin + count]
        ws = new_ws()
        d_pool = torch.from_numpy(pool_np.copy()).cuda()
        mla_dcp_kv_write(dev_src(rows, src_dtype), torch.from_numpy(req).cuda(),
                         torch.from_numpy(pos).cuda(), torch.from_numpy(np.ascontiguousarray(tab)).cuda(),
                         begin, N, d_pool, kv_dtype, pool, workspace=ws)
        torch.cuda.synchronize()
        slots, bad = okw.dcp_slot_mapping(req, pos, tab, begin, count, N, pool)
        ref, _ = okw.kv_write(pool_np, kv_dtype, host_f32(rows, src_dtype), slots)
        assert np.array_equal(d_pool.cpu().numpy(), ref)
        assert mla_get_device_error(ws) == (MLA_DEVERR_BLOCK_TABLE if bad.any() else 0)


def test_write_with_no_owned_tokens_leaves_the_pool_alone():
    T, blocks = 50, 2
    rows = workload.new_token_rows(T, seed=22, dtype="bf16")
    slots = np.full(T, -1, np.int64)
    got = check_write(rows, "bf16", slots, "fp8_ds", blocks, seed=23)
    assert got.size == blocks * 64 * 656


@pytest.mark.parametrize("name,kw", [
    ("dense_fp8_mixed", dict(batch=3, ctx_range=(1000, 6000), seed=31)),
    ("dense_bf16_32k", dict(batch=2, context=3001, seed=32)),
])
def test_each_rank_writes_its_tokens_then_decodes(name, kw):
    """Every shard writes only the new tokens it owns (the per-rank call);
    the decode over the written cache matches the oracle's decode over the
    oracle's rows."""
    sp = workload.SPECS[name].with_(**kw)
    say(f"write-then-decode {sp.name} {kw}")
    x = workload.generate(sp)
    cache = layout.pack(x, device="cuda")
    B, Tq, N = sp.batch, sp.q_len, sp.n_shards
    req = np.repeat(np.arange(B, dtype=np.int32), Tq)
    posn = np.array([int(x.context_lens[b]) - Tq + t for b in range(B) for t in range(Tq)], np.int32)
    src = workload.new_token_rows(B * Tq, seed=sp.seed + 1, dtype="bf16")
    d_src = dev_src(src, "bf16")
    ws = new_ws()
    owned_total = 0
    for s in range(N):
        slots = torch.empty(B * Tq, dtype=torch.int64, device="cuda")
        mla_dcp_slot_mapping(torch.from_numpy(req).cuda(), torch.from_numpy(posn).cuda(),
                             cache.block_tables[s:s + 1].contiguous(), s, N, cache.pool_blocks,
                             slots, workspace=ws)
        mla_kv_write(d_src, slots, cache.pool, sp.kv_dtype, cache.pool_blocks, workspace=ws)
        torch.cuda.synchronize()
        sl = slots.cpu().numpy()
        owned = posn % N == s
        assert np.all(sl[~owned] == -1) and np.all(sl[owned] >= 0)
        owned_total += int(owned.sum())
    assert owned_total == B * Tq
    assert mla_get_device_error(ws) == 0
    # the oracle's rows for the new tokens
    f = host_f32(src, "bf16")
    rows_at = np.array([int(x.row_offsets[b]) + int(posn[i]) for i, b in enumerate(req)])
    if sp.kv_dtype == "fp8_ds":
        codes, scales = okw.quantize_groups(f[:, :512])
        x.latent[rows_at] = codes
        x.scales[rows_at] = scales
    else:
        x.latent[rows_at] = okw.bf16_round(f[:, :512])
    x.rope[rows_at] = okw.bf16_round(f[:, 512:])
    step = ShardedDecodeStep(cache, sp.out_dtype)
    step()
    torch.cuda.synchronize()
    compare(x, step)


def test_full_size_write_sampled():
    """The 1M-token write (one request's whole cache, 8 shards in one pool,
    bf16 source, fp8 rows) in the launch configuration the benchmark times;
    every slot checked, 4096 sampled rows checked byte for byte."""
    w = workload.WRITE_SPECS["kv_write_fp8_1m"]
    T, N = w["tokens"], w["n_shards"]
    say(f"full-size write {T} tokens over {N} shards")
    tables, blocks = layout.build_block_tables(np.array([T]), N, seed=w["seed"])
    src = workload.new_token_rows(T, seed=w["seed"], dtype=w["src_dtype"], spread=8)
    req = np.zeros(T, np.int32)
    posn = np.arange(T, dtype=np.int32)
    d_slots = torch.empty(T, dtype=torch.int64, device="cuda")
    ws = new_ws()
    mla_dcp_slot_mapping(torch.from_numpy(req).cuda(), torch.from_numpy(posn).cuda(),
                         torch.from_numpy(tables).cuda(), 0, N, blocks, d_slots, workspace=ws)
    rb = ROWB[w["kv_dtype"]]
    pool = torch.zeros(blocks * 64 * rb, dtype=torch.uint8, device="cuda")
    mla_kv_write(dev_src(src, w["src_dtype"]), d_slots, pool, w["kv_dtype"], blocks, workspace=ws)
    torch.cuda.synchronize()
    assert mla_get_device_error(ws) == 0
    slots = d_slots.cpu().numpy()
    # every slot: owner shard's table, local row (closed form of the oracle's rule)
    s, j = posn % N, posn // N
    assert np.array_equal(slots, tables[s, 0, j // 64].astype(np.int64) * 64 + j % 64)
    assert np.unique(slots).size == T
    sample = np.random.default_rng(24).choice(T, 4096, replace=False)
    ref_slots, _ = okw.dcp_slot_mapping(req[sample], posn[sample], tables, 0, N, N, blocks)
    assert np.array_equal(slots[sample], ref_slots)
    f = host_f32(src[sample], w["src_dtype"])
    got = pool.view(-1, rb)[torch.from_numpy(slots[sample]).cuda()].cpu().numpy()
    for i in range(sample.size):
        assert np.array_equal(got[i], okw.row_bytes_for(f[i], w["kv_dtype"])), int(sample[i])
    # the fused call gives the same pool, for all shards at once and shard by shard
    d_src, d_req, d_pos = dev_src(src, w["src_dtype"]), torch.from_numpy(req).cuda(), torch.from_numpy(posn).cuda()
    fused = torch.zeros_like(pool)
    mla_dcp_kv_write(d_src, d_req, d_pos, torch.from_numpy(tables).cuda(), 0, N, fused, w["kv_dtype"],
                     blocks, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(fused, pool)
    fused.zero_()
    for s_ in range(N):
        mla_dcp_kv_write(d_src, d_req, d_pos, torch.from_numpy(np.ascontiguousarray(tables[s_:s_ + 1])).cuda(),
                         s_, N, fused, w["kv_dtype"], blocks, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(fused, pool)
    assert mla_get_device_error(ws) == 0
