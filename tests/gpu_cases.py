"""Shared helpers of the GPU parity tests: run a workload through the C ABI
and compare with the float64 oracle on the same seeded inputs."""
import numpy as np
import torch

import workload
from oracle import attention, decode as odecode
from sequence_sharded_mla_amd import layout, mla_get_device_error
from sequence_sharded_mla_amd.step import ShardedDecodeStep

# Tolerances: max abs error on outputs (bf16 / fp8 caches) and on LSE.
TOL_O = 2e-2
TOL_LSE = 1e-3


def say(*a):
    print(*a, flush=True)


def run_gpu(x, extra_width=0):
    cache = layout.pack(x, device="cuda", extra_width=extra_width)
    step = ShardedDecodeStep(cache, x.spec.out_dtype)
    step()
    torch.cuda.synchronize()
    return cache, step


def to_np(t):
    return t.float().cpu().numpy()


def oracle_for(x, requests=None, full=True):
    sp = x.spec
    q = odecode.query_to_f64(x.q, sp.q_dtype)
    rows = odecode.storage_rows(sp.kv_dtype, x.latent, x.scales, x.rope, x.row_offsets, x.row_pos)
    return odecode.mla_decode(q, rows, x.context_lens, sp.q_len, sp.n_shards, sp.scale,
                              topk_idx=x.topk_idx, requests=requests, full=full)


def max_err(a, b):
    """Max abs error over entries finite in the reference; -inf must match."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    ninf_b = np.isneginf(b)
    assert np.array_equal(np.isneginf(a), ninf_b), "-inf pattern differs"
    fin = ~ninf_b
    if not fin.any():
        return 0.0
    assert np.all(np.isfinite(a[fin])), "non-finite where the oracle is finite"
    return float(np.abs(a[fin] - b[fin]).max())


def compare(x, step, requests=None, tol_o=TOL_O, tol_lse=TOL_LSE):
    """Per-shard partials and merged outputs against the oracle."""
    sp = x.spec
    B, Tq, H, N = sp.batch, sp.q_len, sp.heads, sp.n_shards
    ref = oracle_for(x, requests=requests)
    req = list(range(B)) if requests is None else list(requests)
    o_sh = to_np(step.o_partials).reshape(N, B, Tq, H, 512)[:, req]
    l_sh = to_np(step.lses).reshape(N, B, Tq, H)[:, req]
    o = to_np(step.o).reshape(B, Tq, H, 512)[req]
    l = to_np(step.lse).reshape(B, Tq, H)[req]
    errs = dict(o_shards=max_err(o_sh, ref["o_shards"]), lse_shards=max_err(l_sh, ref["lse_shards"]),
                o=max_err(o, ref["o"]), lse=max_err(l, ref["lse"]))
    say(f"{sp.name}: " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    assert errs["o_shards"] <= tol_o and errs["o"] <= tol_o, errs
    assert errs["lse_shards"] <= tol_lse and errs["lse"] <= tol_lse, errs
    assert mla_get_device_error(step.workspace) == 0
    return errs
