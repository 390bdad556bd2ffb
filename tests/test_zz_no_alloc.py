"""The allocation-free decode call (mla_decode_partial_noalloc) against the
workspace call (mla_decode_partial) through the C ABI: two calls in a row on
one GPU, the second with a smaller input, each compared with the workspace
call's result on the same inputs (bit for bit when both plan the same
chunks, else within the parity bar), plus the scratch-limit error."""
import ctypes

import numpy as np
import pytest
import torch

import workload
from sequence_sharded_mla_amd import (_lib, alloc_workspace, layout, mla_decode_partial,
                                      mla_decode_partial_noalloc, mla_get_device_error, MLAError)

from gpu_cases import TOL_LSE, TOL_O, max_err, say, to_np

pytestmark = pytest.mark.gpu

S = workload.SPECS


def _both(sp, shard):
    x = workload.generate(sp)
    cache = layout.pack(x, device="cuda")
    d = cache.desc
    rows = sp.batch * sp.q_len
    dt = torch.bfloat16 if sp.out_dtype == "bf16" else torch.float32
    bt = cache.block_tables[shard].contiguous()
    o_ref = torch.empty((rows, sp.heads, 512), dtype=dt, device="cuda")
    l_ref = torch.empty((rows, sp.heads), dtype=torch.float32, device="cuda")
    ws = alloc_workspace(d, 1)
    mla_decode_partial(d, cache.q, cache.pool, bt, cache.context_lens, cache.topk_idx, shard,
                       sp.n_shards, o_ref, l_ref, ws)
    o = torch.full_like(o_ref, float("nan"))
    l = torch.full_like(l_ref, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    mla_decode_partial_noalloc(d, cache.q, cache.pool, bt, cache.context_lens, cache.topk_idx, shard,
                               sp.n_shards, o, l, err_word=err)
    torch.cuda.synchronize()
    assert mla_get_device_error(ws) == 0 and int(err.item()) == 0
    return o_ref, l_ref, o, l


@pytest.mark.parametrize("first,second", [
    (("dense_fp8_mixed", dict(batch=6, ctx_range=(3000, 40000), seed=41)),
     ("dense_fp8_mixed", dict(batch=2, ctx_range=(100, 900), seed=42))),
    (("dense_bf16_32k", dict(batch=4, context=20000, seed=43)),
     ("dense_bf16_32k", dict(batch=1, context=700, heads=64, seed=44))),
    (("sparse_fp8_topk2048", dict(batch=3, context=6000, topk=512, seed=45)),
     ("sparse_fp8_topk2048", dict(batch=1, context=900, topk=128, seed=46))),
    (("sparse_bf16_topk2048", dict(batch=3, context=6000, topk=512, seed=47)),
     ("sparse_bf16_topk2048", dict(batch=1, context=900, topk=128, seed=48))),
])
def test_noalloc_matches_workspace_call_twice(first, second):
    for name, kw in (first, second):
        sp = S[name].with_(**kw)
        say(f"noalloc {name} {kw}")
        o_ref, l_ref, o, l = _both(sp, shard=3)
        if torch.equal(o, o_ref) and torch.equal(l, l_ref):
            continue  # same plan, same bits
        eo = max_err(to_np(o), to_np(o_ref))
        el = max_err(to_np(l), to_np(l_ref))
        say(f"  differs from the workspace call by o={eo:.3e} lse={el:.3e}")
        assert eo <= TOL_O and el <= TOL_LSE


def test_noalloc_long_rows_plan_within_the_scratch():
    """A one-rank call whose workspace plan would exceed the 64 MiB scratch
    (128 heads, fp32 partials of many chunks) plans longer chunks instead."""
    sp = S["dense_bf16_32k"].with_(batch=32, context=32768, seed=47)
    say("noalloc C2 shard")
    o_ref, l_ref, o, l = _both(sp, shard=0)
    eo = max_err(to_np(o), to_np(o_ref))
    el = max_err(to_np(l), to_np(l_ref))
    say(f"  o={eo:.3e} lse={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


def test_noalloc_rejects_calls_beyond_the_scratch():
    lib = _lib.load()
    # 2^24 query tokens of 128 heads: the plan's row table alone exceeds the scratch
    d = _lib.MLADecodeDesc(batch=1 << 22, q_len=4, num_heads=128, kv_lora_rank=512, rope_dim=64,
                           block_size=64, max_blocks=4096, topk=0, q_dtype=_lib.MLA_BF16,
                           kv_dtype=_lib.MLA_BF16, out_dtype=_lib.MLA_BF16, softmax_scale=0.07,
                           pool_blocks=100)
    fake = ctypes.c_void_p(1 << 20)
    st = lib.mla_decode_partial_noalloc(ctypes.byref(d), fake, fake, fake, fake, None, 0, 8, fake, fake,
                                        None, None)
    assert st == _lib.MLA_ERR_WORKSPACE
