"""Sequence-sharded MLA decode attention on MI355X (gfx950).

Thin Python binding of libmla_dcp.so.  Every function has the name of the C
entry point it calls and only marshals arguments: tensors become device
pointers, the current torch stream becomes the HIP stream, and a non-zero
status raises MLAError.  All computation happens in the library's HIP
kernels; there is no Python or CPU fallback.
"""

import ctypes

import torch

from . import _lib
from ._lib import (MLA_BF16, MLA_F32, MLA_FP8_DS, MLA_DEVERR_BLOCK_TABLE,  # noqa: F401
                   MLA_DEVERR_INDEX, MLA_DEVERR_SLOT, MLA_DEVERR_SCORES, MLA_DEVERR_QUERY,
                   MLADecodeDesc)

DTYPE_CODES = {"f32": MLA_F32, "bf16": MLA_BF16, "fp8_ds": MLA_FP8_DS}
LATENT = 512
ROPE = 64
BLOCK = 64


class MLAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({mla_status_string(status)})")


def _check(status, where):
    if status != 0:
        raise MLAError(status, where)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_desc(batch, q_len, num_heads, max_blocks, pool_blocks, q_dtype, kv_dtype, out_dtype,
              softmax_scale, topk=0):
    """Build an mla_decode_desc (dtype arguments are 'f32', 'bf16', 'fp8_ds')."""
    return MLADecodeDesc(batch=batch, q_len=q_len, num_heads=num_heads, kv_lora_rank=LATENT,
                         rope_dim=ROPE, block_size=BLOCK, max_blocks=max_blocks, topk=topk,
                         q_dtype=DTYPE_CODES[q_dtype], kv_dtype=DTYPE_CODES[kv_dtype],
                         out_dtype=DTYPE_CODES[out_dtype], softmax_scale=softmax_scale,
                         pool_blocks=pool_blocks)


def mla_status_string(status):
    return _lib.load().mla_status_string(status).decode()


def mla_shard_local_len(context_len, shard_id, n_shards):
    return _lib.load().mla_shard_local_len(context_len, shard_id, n_shards)


def mla_kv_row_bytes(kv_dtype):
    return _lib.load().mla_kv_row_bytes(DTYPE_CODES.get(kv_dtype, kv_dtype))


def mla_decode_workspace_size(desc, shard_count=1):
    out = ctypes.c_int64(0)
    _check(_lib.load().mla_decode_workspace_size(ctypes.byref(desc), shard_count,
                                                 ctypes.byref(out)),
           "mla_decode_workspace_size")
    return out.value


def alloc_workspace(desc, shard_count=1, device="cuda"):
    """Device workspace for `desc` with its error word cleared."""
    ws = torch.empty(mla_decode_workspace_size(desc, shard_count), dtype=torch.uint8,
                     device=device)
    mla_clear_device_error(ws)
    return ws


def mla_decode_partial(desc, q, kv_pool, block_table, context_lens, topk_idx, shard_id,
                       n_shards, o_partial, lse, workspace, stream=None):
    _check(_lib.load().mla_decode_partial(
        ctypes.byref(desc), _ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(context_lens),
        _ptr(topk_idx), shard_id, n_shards, _ptr(o_partial), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)), "mla_decode_partial")


def mla_decode_partial_noalloc(desc, q, kv_pool, block_table, context_lens, topk_idx, shard_id,
                               n_shards, o_partial, lse, err_word=None, stream=None):
    """mla_decode_partial with the library's own per-device scratch instead of
    a workspace (no allocation inside the call); err_word: a device int32 /
    uint32 tensor receiving the device error bits, or None."""
    _check(_lib.load().mla_decode_partial_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(context_lens),
        _ptr(topk_idx), shard_id, n_shards, _ptr(o_partial), _ptr(lse), _ptr(err_word),
        _stream(stream)), "mla_decode_partial_noalloc")


def mla_decode_partial_shards(desc, q, kv_pool, block_tables, context_lens, topk_idx,
                              shard_begin, shard_count, n_shards, o_partials, lses, workspace,
                              stream=None):
    _check(_lib.load().mla_decode_partial_shards(
        ctypes.byref(desc), _ptr(q), _ptr(kv_pool), _ptr(block_tables), _ptr(context_lens),
        _ptr(topk_idx), shard_begin, shard_count, n_shards, _ptr(o_partials), _ptr(lses),
        _ptr(workspace), workspace.numel(), _stream(stream)), "mla_decode_partial_shards")


def mla_decode_partial_shards_varlen(desc, q, kv_pool, block_tables, context_lens,
                                     query_start_loc, topk_idx, shard_begin, shard_count, n_shards,
                                     o_partials, lses, workspace, stream=None):
    """q [n_q][H][576]; query_start_loc [B + 1] int32 -> o_partials / lses per shard."""
    _check(_lib.load().mla_decode_partial_shards_varlen(
        ctypes.byref(desc), _ptr(q), _ptr(kv_pool), _ptr(block_tables), _ptr(context_lens),
        _ptr(query_start_loc), q.shape[0], _ptr(topk_idx), shard_begin, shard_count, n_shards,
        _ptr(o_partials), _ptr(lses), _ptr(workspace), workspace.numel(), _stream(stream)),
        "mla_decode_partial_shards_varlen")


def mla_lse_merge(o_parts, lse_parts, o_out, lse_out=None, stream=None):
    """o_parts [n][rows][512] (f32/bf16), lse_parts [n][rows] f32 -> o_out, lse_out."""
    n, rows, dv = o_parts.shape
    code = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16}
    _check(_lib.load().mla_lse_merge(
        n, rows, dv, code[o_parts.dtype], _ptr(o_parts), _ptr(lse_parts), code[o_out.dtype],
        _ptr(o_out), _ptr(lse_out), _stream(stream)), "mla_lse_merge")


def mla_localize_indices(global_idx, shard_id, n_shards, local_idx, stream=None):
    _check(_lib.load().mla_localize_indices(
        _ptr(global_idx), global_idx.numel(), shard_id, n_shards, _ptr(local_idx),
        _stream(stream)), "mla_localize_indices")


def mla_dcp_slot_mapping(req_idx, positions, block_tables, shard_begin, n_shards, pool_blocks,
                         slot_mapping, workspace=None, stream=None):
    """req_idx, positions [T] int32; block_tables [shard_count][B][max_blocks] int32
    -> slot_mapping [T] int64 (-1 where no shard in the range writes the token)."""
    shard_count, batch, max_blocks = block_tables.shape
    _check(_lib.load().mla_dcp_slot_mapping(
        _ptr(req_idx), _ptr(positions), positions.numel(), _ptr(block_tables), batch, max_blocks,
        pool_blocks, shard_begin, shard_count, n_shards, _ptr(slot_mapping), _ptr(workspace),
        _stream(stream)), "mla_dcp_slot_mapping")


def mla_kv_write(kv_new, slot_mapping, kv_pool, kv_dtype, pool_blocks, workspace=None,
                 stream=None):
    """kv_new [T][576] f32/bf16, slot_mapping [T] int64 -> rows of kv_pool (in place)."""
    code = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16}
    _check(_lib.load().mla_kv_write(
        _ptr(kv_new), code[kv_new.dtype], slot_mapping.numel(), _ptr(slot_mapping),
        DTYPE_CODES.get(kv_dtype, kv_dtype), _ptr(kv_pool), pool_blocks, _ptr(workspace),
        _stream(stream)), "mla_kv_write")


def mla_dcp_kv_write(kv_new, req_idx, positions, block_tables, shard_begin, n_shards, kv_pool,
                     kv_dtype, pool_blocks, workspace=None, stream=None):
    """Owner slot mapping and row write in one launch (see mla_dcp_slot_mapping, mla_kv_write)."""
    code = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16}
    shard_count, batch, max_blocks = block_tables.shape
    _check(_lib.load().mla_dcp_kv_write(
        _ptr(kv_new), code[kv_new.dtype], _ptr(req_idx), _ptr(positions), positions.numel(),
        _ptr(block_tables), batch, max_blocks, shard_begin, shard_count, n_shards,
        DTYPE_CODES.get(kv_dtype, kv_dtype), _ptr(kv_pool), pool_blocks, _ptr(workspace),
        _stream(stream)), "mla_dcp_kv_write")


def mla_topk_local(scores, context_lens, topk, shard_begin, n_shards, cand_idx, cand_score,
                   workspace=None, stream=None):
    """scores [shard_count][B][Tq][stride] f32 -> cand_idx / cand_score [shard_count][B][Tq][topk]."""
    shard_count, batch, q_len, stride = scores.shape
    _check(_lib.load().mla_topk_local(
        _ptr(scores), stride, _ptr(context_lens), batch, q_len, topk, shard_begin, shard_count,
        n_shards, _ptr(cand_idx), _ptr(cand_score), _ptr(workspace), _stream(stream)),
        "mla_topk_local")



def mla_topk_local_varlen(scores, context_lens, query_start_loc, topk, shard_begin, n_shards, cand_idx,
                          cand_score, workspace=None, stream=None):
    """scores [shard_count][n_q][stride] f32, request b holding query tokens
    query_start_loc[b] .. query_start_loc[b + 1] - 1 -> cand_idx / cand_score
    [shard_count][n_q][topk]."""
    shard_count, n_q, stride = scores.shape
    batch = query_start_loc.numel() - 1
    _check(_lib.load().mla_topk_local_varlen(
        _ptr(scores), stride, _ptr(context_lens), _ptr(query_start_loc), batch, n_q, topk, shard_begin,
        shard_count, n_shards, _ptr(cand_idx), _ptr(cand_score), _ptr(workspace), _stream(stream)),
        "mla_topk_local_varlen")

def mla_topk_merge(cand_idx, cand_score, topk, topk_idx, stream=None):
    """cand_* [n_lists][rows][cand_k] -> topk_idx [rows][topk]."""
    n_lists = cand_idx.shape[0]
    cand_k = cand_idx.shape[-1]
    rows = cand_idx.numel() // (n_lists * cand_k)
    _check(_lib.load().mla_topk_merge(
        _ptr(cand_idx), _ptr(cand_score), n_lists, rows, cand_k, topk, _ptr(topk_idx),
        _stream(stream)), "mla_topk_merge")


def mla_get_device_error(workspace, stream=None):
    code = ctypes.c_int32(0)
    _check(_lib.load().mla_get_device_error(_ptr(workspace), ctypes.byref(code), _stream(stream)),
           "mla_get_device_error")
    return code.value


def mla_clear_device_error(workspace, stream=None):
    _check(_lib.load().mla_clear_device_error(_ptr(workspace), _stream(stream)),
           "mla_clear_device_error")
