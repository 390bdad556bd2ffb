"""Pins of the oracle's cache-write step (encoders, quantiser, slot mapping).

The encoders are checked against the OCP E4M3FN value table, exact midpoints
and torch's own float8 / bfloat16 casts (independent implementations of the
same rounding); the slot mapping against a brute-force inverse built from the
block tables; the write against the row format and the untouched rest of the
pool.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import codecs, kv_write as kw

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_bf16(v):
    t = torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- E4M3FN encode

def test_encode_inverts_decode_for_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = codecs.e4m3fn_to_f64(codes).astype(np.float32)
    assert np.array_equal(kw.e4m3fn_encode(vals), codes)


def test_encode_golden_table(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ocp_e4m3fn.json")))
    for code, val in g["values"].items():
        assert kw.e4m3fn_encode(np.float32(val)) == int(code, 16), code
    assert kw.e4m3fn_encode(np.float32("nan")) == 0x7F


def test_encode_midpoints_tie_to_even_and_neighbours_round_to_nearest():
    pos = codecs.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    for k in range(0x7E):
        mid = np.float32((pos[k] + pos[k + 1]) / 2)
        assert float(mid) == (pos[k] + pos[k + 1]) / 2          # exact in float32
        even = k if k % 2 == 0 else k + 1
        above = np.nextafter(mid, np.float32(np.inf))
        below = np.nextafter(mid, np.float32(0))
        got = kw.e4m3fn_encode(np.array([mid, above, below, -mid, -above, -below], np.float32))
        assert list(got) == [even, k + 1, k, even | 0x80, (k + 1) | 0x80, k | 0x80], k


def test_encode_subnormal_edges():
    t = np.float32(2.0 ** -10)          # halfway between 0 and the least subnormal
    vals = np.array([t, np.nextafter(t, np.float32(1)), 3 * t, 2.0 ** -149, -2.0 ** -149, -0.0, 0.0],
                    np.float32)
    assert list(kw.e4m3fn_encode(vals)) == [0x00, 0x01, 0x02, 0x00, 0x80, 0x80, 0x00]


def test_encode_saturates():
    vals = np.array([448.0, 455.0, 463.99, 464.0, 480.0, 1e6, 3e38, -464.0, -1e30], np.float32)
    assert list(kw.e4m3fn_encode(vals)) == [0x7E] * 7 + [0xFE] * 2


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(3)
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), 400_000)).astype(np.float32)
    v = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    assert np.array_equal(kw.e4m3fn_encode(v), torch_e4m3(v))


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 2 ** 32, 400_000, dtype=np.uint64).astype(np.uint32)
    ties = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    specials = np.array([0x00000000, 0x80000000, 0x7F7F8000, 0x7F7F7FFF, 0x7F7FFFFF, 0xFF7F8000,
                         0x7F800000, 0xFF800000, 0x00008000, 0x00018000, 0x00000001], np.uint32)
    x = np.concatenate([bits, ties, specials]).view(np.float32)
    finite = ~np.isnan(x)
    assert np.array_equal(kw.bf16_round(x)[finite], torch_bf16(x)[finite])
    nan_out = kw.bf16_round(x[~finite])
    assert np.all((nan_out & 0x7F80) == 0x7F80) and np.all((nan_out & 0x7F) != 0)


def test_bf16_round_is_identity_on_bf16_values():
    b = np.arange(0, 2 ** 16, dtype=np.uint32)
    b = b[(b & 0x7F80) != 0x7F80].astype(np.uint16)            # finite patterns only
    x = (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(kw.bf16_round(x), b)


# ---------------------------------------------------------------- quantiser

def test_quantize_matches_independent_cast_pipeline():
    """Same rule built from numpy division and torch's float8 cast."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((300, 512)) * np.exp2(rng.integers(-20, 20, (300, 1)))).astype(np.float32)
    x[7, 128:256] = 0.0
    codes, scales = kw.quantize_groups(x)
    g = x.reshape(300, 4, 128)
    amax = np.abs(g).max(axis=2)
    s_ref = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    c_ref = torch_e4m3(np.clip(g / s_ref[:, :, None], -448, 448).astype(np.float32)).reshape(300, 512)
    assert np.array_equal(scales, s_ref)
    assert np.array_equal(codes, c_ref)


def test_quantize_group_properties():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[3, :128] = 0.0
    x[3, 5] = -0.0
    codes, scales = kw.quantize_groups(x)
    # all-zero group: scale 1, codes keep the sign of zero
    assert scales[3, 0] == 1.0 and codes[3, 5] == 0x80 and codes[3, 4] == 0x00
    # the largest magnitude of every non-zero group encodes to +-448
    g = x.reshape(64, 4, 128)
    arg = np.abs(g).argmax(axis=2)
    top = np.take_along_axis(codes.reshape(64, 4, 128), arg[:, :, None], axis=2)[:, :, 0]
    nz = np.abs(g).max(axis=2) > 0
    assert np.all((top[nz] & 0x7F) == 0x7E)
    # dequantised error: half an E4M3 step (2^-4 relative for normals,
    # 2^-10 of the scale in the subnormal range), plus the float32 quotient's
    # own rounding
    deq = codecs.fp8_ds_latent_to_f64(codes, scales)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - x) <= bound)


def test_quantize_tiny_groups_saturate_instead_of_overflowing():
    # a group whose scale is a float32 subnormal: x / scale can exceed 448
    x = np.zeros((1, 512), np.float32)
    x[0, :128] = np.float32(2.0 ** -133)           # least bf16 subnormal
    x[0, 1] = np.float32(0.0)
    codes, scales = kw.quantize_groups(x)
    assert scales[0, 0] > 0 and scales[0, 0] < np.finfo(np.float32).tiny
    q = (x[0, :128] / scales[0, 0]).astype(np.float32)
    assert np.all(codes[0, :128] == kw.e4m3fn_encode(q))
    assert q.max() > 448 and np.all((codes[0, :128] & 0x7F) <= 0x7E)


# ---------------------------------------------------------------- slot mapping

def tables(n_shards, B, max_blocks, pool_blocks, seed):
    ids = np.random.default_rng(seed).permutation(pool_blocks)[: n_shards * B * max_blocks]
    return ids.reshape(n_shards, B, max_blocks).astype(np.int32)


def test_slot_mapping_inverse_by_brute_force():
    N, B, mb, pool = 4, 3, 5, 80
    bt = tables(N, B, mb, pool, 1)
    where = {}                                   # pool block -> (shard, request, column)
    for s in range(N):
        for b in range(B):
            for c in range(mb):
                where[int(bt[s, b, c])] = (s, b, c)
    rng = np.random.default_rng(2)
    T = 600
    req = rng.integers(0, B, T)
    pos = rng.integers(0, N * mb * 64, T)
    slots, bad = kw.dcp_slot_mapping(req, pos, bt, 0, N, N, pool)
    assert not bad.any() and np.all(slots >= 0)
    for i in range(T):
        s, b, c = where[int(slots[i]) // 64]
        j = c * 64 + int(slots[i]) % 64
        assert (b, j * N + s) == (req[i], pos[i])


def test_slot_mapping_one_shard_keeps_only_owned_tokens():
    N, B, mb, pool = 8, 2, 3, 64
    bt = tables(N, B, mb, pool, 3)
    req = np.repeat(np.arange(B), 1500)
    pos = np.tile(np.arange(1500), B)
    all_slots, _ = kw.dcp_slot_mapping(req, pos, bt, 0, N, N, pool)
    union = np.full_like(all_slots, -1)
    for s in range(N):
        one, bad = kw.dcp_slot_mapping(req, pos, bt[s:s + 1], s, 1, N, pool)
        owned = pos % N == s
        assert not bad.any()
        assert np.all(one[~owned] == -1) and np.array_equal(one[owned], all_slots[owned])
        union[owned] = one[owned]
    assert np.array_equal(union, all_slots)
    # distinct tokens land in distinct rows
    assert np.unique(all_slots).size == all_slots.size


def test_slot_mapping_padding_and_bad_entries():
    N, B, mb, pool = 2, 2, 2, 16
    bt = tables(N, B, mb, pool, 4)
    bt[1, 0, 1] = pool                           # out of the pool
    bt[0, 1, 0] = -3
    req = np.array([0, 0, 5, -1, 0, 1, 1, 0])
    pos = np.array([-1, 2 * 64 * 2, 0, 0, 2 * 64 + 1, 0, 3, 1])
    slots, bad = kw.dcp_slot_mapping(req, pos, bt, 0, N, N, pool)
    # -1 position and bad request ids are padding; column 2 is beyond the
    # table; block ids outside the pool are bad
    assert list(bad) == [False, True, False, False, True, True, False, False]
    assert np.all(slots[[0, 1, 2, 3, 4, 5]] == -1)
    assert slots[6] == bt[1, 1, 0] * 64 + 1 and slots[7] == bt[1, 0, 0] * 64 + 0


# ---------------------------------------------------------------- write

@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "fp8_ds"])
def test_write_touches_only_the_slotted_rows(kv_dtype):
    rb = kw.ROW_BYTES[kv_dtype]
    rows = 200
    rng = np.random.default_rng(7)
    pool = rng.integers(0, 256, rows * rb, dtype=np.uint8)
    src = rng.standard_normal((40, 576)).astype(np.float32)
    slots = rng.permutation(rows)[:40].astype(np.int64)
    slots[::3] = -1
    slots[5] = rows                               # past the end: flagged, not written
    out, bad = kw.kv_write(pool, kv_dtype, src, slots)
    assert list(np.nonzero(bad)[0]) == [5]
    written = set(int(s) for s in slots if 0 <= s < rows)
    view_in, view_out = pool.reshape(rows, rb), out.reshape(rows, rb)
    for r in range(rows):
        if r not in written:
            assert np.array_equal(view_in[r], view_out[r])
    for i, s in enumerate(slots):
        if not 0 <= s < rows:
            continue
        row = view_out[s]
        if kv_dtype == "f32":
            assert np.array_equal(row.view("<f4"), src[i])
        elif kv_dtype == "bf16":
            got = codecs.bf16_bits_to_f64(row.view("<u2"))
            assert np.all(np.abs(got - src[i]) <= np.abs(src[i]) * 2.0 ** -8)
        else:
            lat = codecs.fp8_ds_latent_to_f64(row[:512], row[512:528].view("<f4"))
            assert np.all(np.abs(lat - src[i, :512]) <= np.abs(src[i, :512]).max() / 448 * 32)
            rope = codecs.bf16_bits_to_f64(row[528:656].view("<u2"))
            assert np.all(np.abs(rope - src[i, 512:]) <= np.abs(src[i, 512:]) * 2.0 ** -8)
