"""Integer steps of the sequence sharding, written from the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Round-robin ownership ("How vLLM Serves GLM-5.3 with Million-Token Contexts
on 16 H200s", section "The core design": cache tokens are dealt out
round-robin, so each of N ranks keeps 1/N of the cache).  Reading taken: the
deal is one token at a time, so global position p belongs to shard p mod N
and is that shard's local token number p div N (local order follows global
order).

Localisation ("GLM-5.2 vLLM Decode Context Parallelism", section "Separate
the backend merge from stable": global sparse top-K indices are rewritten
for the rank that owns each position).  Reading taken: the localised index
tensor keeps the global shape; an entry owned by shard s becomes its local
number, every other entry (and every invalid entry, marked by a negative
value) becomes -1.
"""

import numpy as np


def owner(p, n_shards):
    """Shard that stores global token position p."""
    return np.asarray(p) % n_shards


def local_index(p, n_shards):
    """Position of global token p inside its owner's local cache."""
    return np.asarray(p) // n_shards


def global_position(j, shard, n_shards):
    """Inverse of (owner, local_index): local token j of `shard`."""
    return np.asarray(j) * n_shards + shard


def local_len(context_len, shard, n_shards):
    """Number of the first `context_len` tokens that `shard` stores.

    Counting the positions p < L with p mod N == s gives ceil((L - s) / N)
    for s < L and 0 otherwise.
    """
    L = np.asarray(context_len, dtype=np.int64)
    return np.where(L > shard, (L - shard + n_shards - 1) // n_shards, 0)


def shard_positions(positions, shard, n_shards):
    """The subset of `positions` (global, int) owned by `shard`, order kept."""
    positions = np.asarray(positions, dtype=np.int64)
    return positions[positions % n_shards == shard]


def localize(global_idx, shard, n_shards):
    """Global top-K indices -> shard-local indices (int32, same shape).

    Entries g >= 0 with g mod N == shard become g div N; all others -1.
    """
    g = np.asarray(global_idx, dtype=np.int64)
    out = np.where((g >= 0) & (g % n_shards == shard), g // n_shards, -1)
    return out.astype(np.int32)
