"""Properties of the seeded input generator (CPU only)."""
import numpy as np
import pytest

import workload
from oracle import codecs


def _small(name, **kw):
    return workload.SPECS[name].with_(**kw)


def test_deterministic_and_thread_independent():
    sp = _small("dense_fp8_mixed", batch=3, ctx_range=(70000, 140000))
    a = workload.generate(sp, threads=1)
    b = workload.generate(sp, threads=4)
    for f in ("q", "context_lens", "row_offsets", "row_pos", "latent", "scales", "rope"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = workload.generate(sp.with_(seed=sp.seed + 1), threads=2)
    assert not np.array_equal(a.latent[:100], c.latent[:100])


def test_context_ranges_and_rows():
    sp = _small("dense_fp8_mixed", batch=50)
    x = workload.generate(sp.with_(ctx_range=(10, 20)))
    assert x.context_lens.min() >= 10 and x.context_lens.max() <= 20
    assert np.array_equal(np.diff(x.row_offsets), x.context_lens)
    for b in range(3):
        lo, hi = x.row_offsets[b], x.row_offsets[b + 1]
        assert np.array_equal(x.row_pos[lo:hi], np.arange(hi - lo))


def test_fp8_quantiser():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[3] = 0.0
    codes, scales = workload.quantize_fp8_groups(x)
    v = codecs.fp8_ds_latent_to_f64(codes, scales)
    g = x.reshape(64, 4, 128)
    # each group's largest magnitude lands exactly on +-448 * scale
    amax_code = np.abs(codecs.e4m3fn_to_f64(codes).reshape(64, 4, 128)).max(axis=2)
    assert np.all(amax_code[np.abs(g).max(axis=2) > 0] == 448.0)
    assert np.all(scales[3] == 1.0) and np.all(v[3] == 0.0)
    # round to nearest: error at most half a step (relative 2^-4 for normals)
    err = np.abs(v - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, np.repeat(scales, 128, axis=1) * 2.0 ** -10))
    assert not np.isnan(v).any()


def test_bf16_storage_is_rounded_float32():
    sp = _small("dense_bf16_32k", batch=1, context=10)
    x = workload.generate(sp)
    q = codecs.bf16_bits_to_f64(x.q)
    assert np.all(np.isfinite(q)) and abs(q.std() - 1) < 0.1


def test_sparse_indices():
    sp = _small("sparse_fp8_topk2048", batch=3, context=3000, topk=500)
    x = workload.generate(sp)
    assert x.topk_idx.shape == (3, 2, 500) and x.topk_idx.dtype == np.int32
    for b in range(3):
        for j in range(2):
            row = x.topk_idx[b, j]
            assert len(np.unique(row)) == 500
            assert row.min() >= 0 and row.max() <= 3000 - 2 + j
        lo, hi = x.row_offsets[b], x.row_offsets[b + 1]
        assert np.array_equal(x.row_pos[lo:hi], np.unique(x.topk_idx[b]))


def test_sparse_short_prefix_pads_with_minus_one():
    sp = _small("sparse_fp8_topk2048", batch=1, context=5, topk=8)
    x = workload.generate(sp)
    assert np.array_equal(np.sort(x.topk_idx[0, 0][x.topk_idx[0, 0] >= 0]), np.arange(4))
    assert np.sum(x.topk_idx[0, 0] < 0) == 4
    assert np.sum(x.topk_idx[0, 1] < 0) == 3


def test_varlen_counts():
    w = workload.VARLEN_SPECS["varlen_fp8_mtp2"]
    c = workload.varlen_counts(64, w["q_len"], w["seed"])
    assert c.shape == (64,) and c.min() >= 1 and c.max() <= w["q_len"]
    assert set(c.tolist()) == {1, 2}
    assert np.array_equal(c, workload.varlen_counts(64, w["q_len"], w["seed"]))
