"""One decode step over every emulated shard: partials, then the LSE merge.

Holds the output and workspace buffers so repeated steps allocate nothing.
"""

import torch

from . import (alloc_workspace, mla_decode_partial_shards, mla_decode_partial_shards_varlen,
               mla_lse_merge)

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


class ShardedDecodeStep:
    def __init__(self, cache, out_dtype):
        d = cache.desc
        self.cache = cache
        rows = d.batch * d.q_len
        N = cache.n_shards
        dev = cache.pool.device
        dt = _TORCH_DTYPE[out_dtype]
        self.o_partials = torch.empty((N, rows, d.num_heads, 512), dtype=dt, device=dev)
        self.lses = torch.empty((N, rows, d.num_heads), dtype=torch.float32, device=dev)
        self.o = torch.empty((rows, d.num_heads, 512), dtype=dt, device=dev)
        self.lse = torch.empty((rows, d.num_heads), dtype=torch.float32, device=dev)
        self.workspace = alloc_workspace(d, N, device=dev)

    def partials(self, stream=None):
        c = self.cache
        mla_decode_partial_shards(c.desc, c.q, c.pool, c.block_tables, c.context_lens,
                                  c.topk_idx, 0, c.n_shards, c.n_shards, self.o_partials,
                                  self.lses, self.workspace, stream=stream)

    def merge(self, stream=None):
        N, rows, H, dv = self.o_partials.shape
        mla_lse_merge(self.o_partials.view(N, rows * H, dv), self.lses.view(N, rows * H),
                      self.o.view(rows * H, dv), self.lse.view(rows * H), stream=stream)

    def __call__(self, stream=None):
        self.partials(stream)
        self.merge(stream)
        return self.o, self.lse


class VarlenDecodeStep(ShardedDecodeStep):
    """The step for requests with different numbers of query tokens.

    q [n_q][H][576] holds request b's tokens at rows query_start_loc[b] ..
    query_start_loc[b + 1] - 1 (device int32 [B + 1]); topk_idx is
    [n_q][K] or None.  The cache's descriptor q_len bounds n_q / B.
    """

    def __init__(self, cache, out_dtype, q, query_start_loc, topk_idx=None):
        d = cache.desc
        n_q = q.shape[0]
        N = cache.n_shards
        dev = cache.pool.device
        dt = _TORCH_DTYPE[out_dtype]
        self.cache = cache
        self.q, self.query_start_loc, self.topk_idx = q, query_start_loc, topk_idx
        self.o_partials = torch.empty((N, n_q, d.num_heads, 512), dtype=dt, device=dev)
        self.lses = torch.empty((N, n_q, d.num_heads), dtype=torch.float32, device=dev)
        self.o = torch.empty((n_q, d.num_heads, 512), dtype=dt, device=dev)
        self.lse = torch.empty((n_q, d.num_heads), dtype=torch.float32, device=dev)
        self.workspace = alloc_workspace(d, N, device=dev)

    def partials(self, stream=None):
        c = self.cache
        mla_decode_partial_shards_varlen(c.desc, self.q, c.pool, c.block_tables, c.context_lens,
                                         self.query_start_loc, self.topk_idx, 0, c.n_shards,
                                         c.n_shards, self.o_partials, self.lses, self.workspace,
                                         stream=stream)
