"""Pins of the integer sharding steps (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import sharding


def test_round_robin_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "page_tables.json")) as f:
        ex = json.load(f)["round_robin_example"]
    P = np.arange(ex["context"])
    for s, want in enumerate(ex["shards"]):
        got = sharding.shard_positions(P, s, ex["n_shards"])
        assert got.tolist() == want
        assert sharding.local_len(ex["context"], s, ex["n_shards"]) == len(want)
        # local numbering follows global order
        assert sharding.local_index(np.array(want), ex["n_shards"]).tolist() == list(range(len(want)))


def test_local_len_by_enumeration():
    for N in range(1, 10):
        for L in range(0, 60):
            total = 0
            for s in range(N):
                count = sum(1 for p in range(L) if p % N == s)
                assert sharding.local_len(L, s, N) == count
                total += count
            assert total == L


def test_local_len_balanced_and_vectorised():
    L = np.array([0, 1, 7, 8, 9, 32768, 1048576, 131071])
    for N in (1, 2, 3, 8, 16):
        lens = np.stack([sharding.local_len(L, s, N) for s in range(N)])
        assert np.array_equal(lens.sum(0), L)
        assert np.all(np.abs(lens - L / N) < 1)
        assert np.all(np.diff(lens, axis=0) <= 0)  # lower shards own no fewer


def test_positions_partition_and_invert():
    rng = np.random.default_rng(1)
    P = np.sort(rng.choice(10000, size=500, replace=False))
    for N in (1, 3, 8):
        parts = [sharding.shard_positions(P, s, N) for s in range(N)]
        allp = np.sort(np.concatenate(parts))
        assert np.array_equal(allp, P)
        for s, part in enumerate(parts):
            j = sharding.local_index(part, N)
            assert np.array_equal(sharding.global_position(j, s, N), part)
            assert np.all(sharding.owner(part, N) == s)


def test_localize_by_enumeration():
    rng = np.random.default_rng(2)
    idx = rng.integers(-3, 200, size=(3, 2, 37)).astype(np.int32)
    for N in (1, 2, 5, 8):
        for s in range(N):
            got = sharding.localize(idx, s, N)
            assert got.dtype == np.int32 and got.shape == idx.shape
            for pos in np.ndindex(idx.shape):
                g = int(idx[pos])
                want = g // N if (g >= 0 and g % N == s) else -1
                assert got[pos] == want


def test_localize_partitions_valid_entries():
    rng = np.random.default_rng(3)
    idx = rng.integers(-1, 5000, size=4096).astype(np.int32)
    N = 8
    owned = np.zeros(idx.shape, dtype=np.int64)
    for s in range(N):
        loc = sharding.localize(idx, s, N)
        m = loc >= 0
        owned += m
        assert np.array_equal(loc[m].astype(np.int64) * N + s, idx[m])
    assert np.array_equal(owned, (idx >= 0).astype(np.int64))
