"""GPU parity of varlen decode (a query count per request) against the oracle.

mla_decode_partial_shards_varlen runs through the C ABI on seeded
workloads whose requests hold different numbers of query tokens (none, one,
up to the descriptor's q_len); the float64 oracle's varlen step gives the
expected per-shard partials and the merged result.  Covered: the bf16
128-head and fp8 64/128-head matrix-core kernels, dense planned (split rows)
and unplanned, sparse top-K, the f32 vector path, the fixed form reproduced
bit for bit when every request holds q_len tokens, and offsets that are not
a partition raising the device error word.
"""

import numpy as np
import pytest
import torch

import workload
from oracle import decode as odecode
from sequence_sharded_mla_amd import (MLA_DEVERR_QUERY, layout, mla_clear_device_error,
                                      mla_get_device_error)
from sequence_sharded_mla_amd.step import ShardedDecodeStep, VarlenDecodeStep

from gpu_cases import TOL_LSE, TOL_O, max_err, say, to_np

pytestmark = pytest.mark.gpu

S = workload.SPECS


def varlen_inputs(x, counts):
    """Request b keeps its last counts[b] query tokens of the fixed form
    (those at positions L_b - counts[b] .. L_b - 1)."""
    Tq = x.spec.q_len
    sel = [(b, j) for b, c in enumerate(counts) for j in range(Tq - c, Tq)]
    q = np.stack([x.q[b, j] for b, j in sel]) if sel else x.q.reshape(-1, *x.q.shape[2:])[:0]
    topk = None
    if x.topk_idx is not None:
        topk = np.stack([x.topk_idx[b, j] for b, j in sel])
    qsl = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return q, topk, qsl


def to_device_q(q, q_dtype):
    if q_dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(q)).cuda()
    return torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).cuda().view(torch.bfloat16)


def run_varlen(x, counts):
    sp = x.spec
    q, topk, qsl = varlen_inputs(x, counts)
    cache = layout.pack(x, device="cuda")
    step = VarlenDecodeStep(cache, sp.out_dtype, to_device_q(q, sp.q_dtype),
                            torch.from_numpy(qsl).cuda(),
                            None if topk is None else torch.from_numpy(topk).cuda())
    step()
    torch.cuda.synchronize()
    return step, q, topk, qsl


def check(x, counts, tokens=None):
    sp = x.spec
    step, q, topk, qsl = run_varlen(x, counts)
    n_q = int(qsl[-1])
    tokens = list(range(n_q)) if tokens is None else list(tokens)
    rows = odecode.storage_rows(sp.kv_dtype, x.latent, x.scales, x.rope, x.row_offsets, x.row_pos)
    ref = odecode.mla_decode_varlen(odecode.query_to_f64(q, sp.q_dtype), rows, x.context_lens,
                                    qsl, sp.n_shards, sp.scale, topk_idx=topk, tokens=tokens)
    errs = dict(o_shards=max_err(to_np(step.o_partials)[:, tokens], ref["o_shards"]),
                lse_shards=max_err(to_np(step.lses)[:, tokens], ref["lse_shards"]),
                o=max_err(to_np(step.o)[tokens], ref["o"]),
                lse=max_err(to_np(step.lse)[tokens], ref["lse"]))
    say(f"varlen {sp.name} counts={list(counts)}: " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    assert errs["o_shards"] <= TOL_O and errs["o"] <= TOL_O, errs
    assert errs["lse_shards"] <= TOL_LSE and errs["lse"] <= TOL_LSE, errs
    assert mla_get_device_error(step.workspace) == 0
    return step


def test_bf16_128_heads_unplanned():
    sp = S["dense_bf16_32k"].with_(batch=5, q_len=4, context=0, ctx_range=(5, 20000), seed=61)
    check(workload.generate(sp), [4, 0, 1, 3, 2])


def test_bf16_128_heads_planned_split_rows():
    sp = S["dense_bf16_32k"].with_(batch=3, q_len=3, context=90000, seed=62)
    x = workload.generate(sp)
    check(x, [1, 3, 2], tokens=[0, 3, 5])


@pytest.mark.parametrize("heads", [64, 128])
def test_fp8_dense_planned(heads):
    sp = S["dense_fp8_mixed"].with_(batch=6, q_len=3, heads=heads, ctx_range=(1000, 70000),
                                    seed=63 + heads)
    check(workload.generate(sp), [3, 1, 0, 2, 3, 1], tokens=[0, 2, 3, 4, 6, 9])


@pytest.mark.parametrize("heads", [64, 128])
def test_fp8_sparse(heads):
    sp = S["sparse_fp8_topk2048"].with_(batch=4, q_len=2, heads=heads, context=0,
                                        ctx_range=(1500, 12000), seed=65 + heads)
    check(workload.generate(sp), [2, 1, 0, 2])


@pytest.mark.parametrize("heads", [32, 128])
def test_bf16_sparse(heads):
    """Top-K over a bf16 cache with a query count per request: the list pass
    resolves each row's request and position through the query map."""
    sp = S["sparse_bf16_topk2048"].with_(batch=4, q_len=2, heads=heads, context=0,
                                         ctx_range=(1500, 12000), topk=300, seed=75 + heads)
    check(workload.generate(sp), [2, 1, 0, 2])


def test_f32_vector_path():
    sp = S["tiny_f32"].with_(batch=4, q_len=3, context=0, ctx_range=(3, 300), seed=67)
    check(workload.generate(sp), [0, 3, 1, 2])


def test_all_requests_full_matches_fixed_form_bitwise():
    sp = S["dense_fp8_mixed"].with_(batch=4, q_len=2, ctx_range=(3000, 60000), seed=68)
    x = workload.generate(sp)
    step, _, _, _ = run_varlen(x, [2, 2, 2, 2])
    cache = layout.pack(x, device="cuda")
    fixed = ShardedDecodeStep(cache, sp.out_dtype)
    fixed()
    torch.cuda.synchronize()
    N = sp.n_shards
    assert torch.equal(step.o_partials, fixed.o_partials.view(N, -1, sp.heads, 512))
    assert torch.equal(step.lses, fixed.lses.view(N, -1, sp.heads))
    assert torch.equal(step.o, fixed.o.view(-1, sp.heads, 512))


def test_offsets_not_a_partition_raise_the_error_word():
    sp = S["dense_fp8_mixed"].with_(batch=3, q_len=2, ctx_range=(500, 3000), seed=69)
    x = workload.generate(sp)
    step, _, _, _ = run_varlen(x, [2, 1, 2])
    assert mla_get_device_error(step.workspace) == 0
    for bad in ([0, 3, 2, 5], [1, 2, 3, 5], [0, 2, 3, 4]):
        step.query_start_loc.copy_(torch.tensor(bad, dtype=torch.int32))
        mla_clear_device_error(step.workspace)
        step()
        torch.cuda.synchronize()
        assert mla_get_device_error(step.workspace) & MLA_DEVERR_QUERY, bad
        assert torch.all(torch.isfinite(step.o.float()))


def test_full_size_varlen_sampled():
    """The varlen workload bench.py times (the fp8 mixed-length cache, 64
    requests holding 1 or 2 query tokens), checked on sampled tokens: both
    tokens of the two shortest two-token requests, the token of the shortest
    one-token request, and the call's last token."""
    w = workload.VARLEN_SPECS["varlen_fp8_mtp2"]
    sp = S[w["base"]].with_(q_len=w["q_len"])
    x = workload.generate(sp)
    counts = workload.varlen_counts(sp.batch, sp.q_len, w["seed"])
    qsl = np.concatenate([[0], np.cumsum(counts)])
    by_len = np.argsort(x.context_lens, kind="stable")
    two = [int(b) for b in by_len if counts[b] == 2][:2]
    one = [int(b) for b in by_len if counts[b] == 1][:1]
    tokens = sorted({int(qsl[b]) + t for b in two for t in range(2)} | {int(qsl[b]) for b in one}
                    | {int(qsl[-1]) - 1})
    check(x, counts, tokens=tokens)
