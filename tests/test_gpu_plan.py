"""The device plan of a dense step, read back from the workspace.

White-box: the workspace layout (256-B header, query map, items, row_info) is the
library's own.  For each row (shard, request, query token) the plan must
list its chunks exactly once, with the chunk size the total work gives (about
two items per resident workgroup, never below 4096 tokens; one item per
resident workgroup and never below 512 for a call with fewer rows than the
chip holds workgroups), a consecutive block of partial slots for each split
row, and the items
ordered longest first (all full chunks, then the remainders by size class).
The outputs of the same steps are checked against the oracle by the parity
tests; this checks the work split itself.
"""

import numpy as np
import pytest
import torch

import workload
from oracle import sharding
from sequence_sharded_mla_amd import layout
from sequence_sharded_mla_amd.step import ShardedDecodeStep

from gpu_cases import say

pytestmark = pytest.mark.gpu

CHUNK_MIN = 4096      # chunk floor of a call that fills the chip with rows
CHUNK_SMALL = 512     # floor of a call with fewer rows than resident workgroups
BUCKETS = 8


def align(x, a=256):
    return (x + a - 1) // a * a


def target_for(sp):
    if sp.kv_dtype == "fp8_ds" and sp.heads == 64:
        return 1024
    if sp.kv_dtype == "f32" or (sp.kv_dtype == "bf16" and sp.heads != 128):
        return 1024
    return 512


@pytest.mark.parametrize("name,kw", [
    ("dense_fp8_mixed", dict(batch=6, ctx_range=(1000, 70000), seed=41)),
    ("dense_fp8_mixed", dict(seed=42)),                       # full size: chunk above the minimum
    ("dense_bf16_32k", dict(batch=3, context=100_000, seed=43)),
    ("long_fp8_1m", dict(batch=1, seed=44)),
])
def test_plan_lists_every_chunk_once_longest_first(name, kw):
    sp = workload.SPECS[name].with_(**kw)
    say(f"plan {sp.name} {kw}")
    x = workload.generate(sp)
    cache = layout.pack(x, device="cuda")
    step = ShardedDecodeStep(cache, sp.out_dtype)
    step.partials()
    torch.cuda.synchronize()
    ws = step.workspace.cpu().numpy()
    N, B, Tq = sp.n_shards, sp.batch, sp.q_len
    rows = N * B * Tq
    cap = cache.max_blocks * 64
    target = target_for(sp)
    few_rows = rows < target // 2
    floor = CHUNK_SMALL if few_rows else CHUNK_MIN
    if few_rows:
        target //= 2          # one item per resident workgroup
    assert cap > floor, "this case must be planned"
    local = np.zeros(rows, np.int64)
    for r in range(rows):
        t, bt = r % Tq, r // Tq
        b, s = bt % B, bt // B
        visible = max(int(x.context_lens[b]) - Tq + t + 1, 0)
        local[r] = min(int(sharding.local_len(visible, s, N)), cap)
    T = max(floor, -(-(-(-int(local.sum()) // target)) // 64) * 64)
    hdr = ws[:256].view(np.int32)
    assert hdr[2] == T
    full = local // T
    rem = ((local % T) > 0) | (local == 0)
    k = full + rem
    n_items = int(k.sum())
    assert hdr[1] == n_items
    items_max = rows + target
    items_off = align(256 + B * Tq * 16)          # after the per-token query map
    items = ws[items_off:items_off + items_max * 16].view(np.int32).reshape(items_max, 4)[:n_items]
    ri_off = align(items_off + items_max * 16)
    row_info = ws[ri_off:ri_off + rows * 8].view(np.int32).reshape(rows, 2)
    assert np.array_equal(row_info[:, 1], k)
    # every (row, chunk) once
    seen = {(int(a), int(c)) for a, c, _, _ in items}
    assert len(seen) == n_items
    assert seen == {(r, c) for r in range(rows) for c in range(int(k[r]))}
    # slots: -1 for whole rows; consecutive per split row, disjoint overall
    split = k > 1
    assert np.all(row_info[~split, 0] == -1)
    used = []
    for r in np.nonzero(split)[0]:
        used.extend(range(int(row_info[r, 0]), int(row_info[r, 0] + k[r])))
    assert len(set(used)) == len(used) and (not used or min(used) >= 0)
    for a, c, slot, zero in items:
        assert zero == 0
        assert slot == (row_info[a, 0] + c if k[a] > 1 else -1)
    # longest first: full chunks, then remainders by size class, largest first
    size = np.where(items[:, 1] < full[items[:, 0]], T, local[items[:, 0]] % T)
    cls = np.where(size == T, BUCKETS, size * BUCKETS // T)
    assert np.all(np.diff(cls) <= 0)
    say(f"  rows {rows} chunk {T} items {n_items} split rows {int(split.sum())}")
