"""The paged round-robin layout on the host (CPU tensors).

An independent reader walks each shard's block table the way the decode
kernel addresses the pool (local token j -> block table[j // 64], slot
j % 64) and must recover every logical row at global position j * N + s.
Unused slots must hold the NaN patterns.
"""
import numpy as np
import pytest

import workload
from sequence_sharded_mla_amd import layout


@pytest.mark.parametrize("name,kw", [
    ("tiny_f32", {}),
    ("dense_bf16_32k", dict(batch=3, context=0, ctx_range=(1, 1000))),
    ("dense_fp8_mixed", dict(batch=4, ctx_range=(60, 700))),
    ("sparse_fp8_topk2048", dict(batch=2, context=4000, topk=100)),
])
def test_pack_round_trip(name, kw):
    sp = workload.SPECS[name].with_(**kw)
    x = workload.generate(sp)
    c = layout.pack(x, device="cpu")
    N, B = sp.n_shards, sp.batch
    rb = layout.ROW_BYTES[sp.kv_dtype]
    pool = c.pool.numpy().reshape(-1, 64, rb)
    tables = c.block_tables.numpy()
    want = layout.pack_rows(sp.kv_dtype, x.latent, x.scales, x.rope)
    used = np.zeros(pool.shape[:2], dtype=bool)
    for b in range(B):
        lo, hi = x.row_offsets[b], x.row_offsets[b + 1]
        stored = dict(zip(x.row_pos[lo:hi].tolist(), range(lo, hi)))
        L = int(x.context_lens[b])
        for s in range(N):
            n_local = len(range(s, L, N))
            for j in range(n_local):
                blk = tables[s, b, j // 64]
                assert 0 <= blk < pool.shape[0]
                used[blk, j % 64] = True
                p = j * N + s
                if p in stored:
                    assert np.array_equal(pool[blk, j % 64], want[stored[p]])
                else:
                    assert np.array_equal(pool[blk, j % 64], layout.poison_row(sp.kv_dtype))
            # entries past the shard's blocks are -1
            assert np.all(tables[s, b, (n_local + 63) // 64:] == -1)
    # every pool block is owned by exactly one table entry
    ids = tables[tables >= 0]
    assert len(np.unique(ids)) == len(ids) == pool.shape[0]
    assert np.all(pool[~used] == np.broadcast_to(layout.poison_row(sp.kv_dtype), pool[~used].shape))


def test_tables_shuffled():
    t, total = layout.build_block_tables(np.array([64 * 8 * 10] * 4), 8, seed=1)
    assert total == 320
    flat = t.reshape(-1)
    assert not np.array_equal(flat, np.arange(320))
