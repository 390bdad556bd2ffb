"""Parity at the full workload sizes, in the launch configuration the
benchmark times (all shards in one launch, then the merge), checked on
sampled requests that the float64 oracle evaluates one by one."""
import numpy as np
import pytest

import workload
from gpu_cases import compare, run_gpu, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("name,requests", [
    ("dense_bf16_32k", [0, 17, 31]),
    ("dense_fp8_mixed", None),        # shortest, longest and one more request
    ("long_fp8_1m", [2]),
    ("sparse_fp8_topk2048", [0, 77, 127]),
])
def test_full_size_sampled(name, requests):
    sp = workload.SPECS[name]
    say(f"full-size {name}: generating")
    x = workload.generate(sp)
    if requests is None:
        L = x.context_lens
        requests = sorted({int(np.argmin(L)), int(np.argmax(L)), 5})
    say(f"full-size {name}: running the GPU step")
    _, step = run_gpu(x)
    say(f"full-size {name}: oracle on requests {requests}")
    compare(x, step, requests=requests)


@pytest.mark.parametrize("name,requests,shard", [
    ("dense_bf16_32k", [3, 30], 0),
    ("long_fp8_1m", [1], 5),
    ("sparse_fp8_topk2048", [9, 100], 2),
])
def test_full_size_single_shard_sampled(name, requests, shard):
    """One rank's call (mla_decode_partial for one shard of the full cache),
    as the benchmark's single-shard line times it: a dense call with fewer
    rows than resident workgroups splits its rows into small chunks."""
    import torch
    from oracle import decode as odecode
    from sequence_sharded_mla_amd import (alloc_workspace, layout, mla_decode_partial,
                                          mla_get_device_error)
    from gpu_cases import max_err, to_np, TOL_LSE, TOL_O
    sp = workload.SPECS[name]
    say(f"full-size single shard {name}: generating")
    x = workload.generate(sp)
    cache = layout.pack(x, device="cuda")
    d = cache.desc
    rows = sp.batch * sp.q_len
    dt = torch.bfloat16 if sp.out_dtype == "bf16" else torch.float32
    o = torch.empty((rows, sp.heads, 512), dtype=dt, device="cuda")
    l = torch.empty((rows, sp.heads), dtype=torch.float32, device="cuda")
    ws = alloc_workspace(d, 1)
    say(f"full-size single shard {name}: shard {shard}")
    mla_decode_partial(d, cache.q, cache.pool, cache.block_tables[shard].contiguous(),
                       cache.context_lens, cache.topk_idx, shard, sp.n_shards, o, l, ws)
    torch.cuda.synchronize()
    assert mla_get_device_error(ws) == 0
    say(f"full-size single shard {name}: oracle on requests {requests}")
    ref = odecode.mla_decode(odecode.query_to_f64(x.q, sp.q_dtype),
                             odecode.storage_rows(sp.kv_dtype, x.latent, x.scales, x.rope,
                                                  x.row_offsets, x.row_pos),
                             x.context_lens, sp.q_len, sp.n_shards, sp.scale,
                             topk_idx=x.topk_idx, requests=requests, shards=[shard], full=False)
    go = to_np(o).reshape(sp.batch, sp.q_len, sp.heads, 512)[requests]
    gl = to_np(l).reshape(sp.batch, sp.q_len, sp.heads)[requests]
    eo, el = max_err(go, ref["o_shards"][0]), max_err(gl, ref["lse_shards"][0])
    say(f"  o={eo:.3e} lse={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE
