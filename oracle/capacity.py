"""Capacity arithmetic that the pages print, used to pin sizes and shares.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* Bytes of one MLA cache row per token and layer: (512 latent + 64 rope)
  values; at 2 bytes each that is 1152 B ("The Final Verification:
  Confirming a 200k Context Deployment on GLM-5", section "The
  Decision-Making Process Visible in the Reasoning").  The packed fp8 row
  holds 512 one-byte codes, one float32 scale per 128-dimension group and 64
  bf16 rope values.
* Cache copies across a TP group and the sequence share per rank under DCP
  ("GLM-5.2 vLLM Decode Context Parallelism", section "Understand the
  cache-copy opportunity", the relative-geometry table and formula).
* Query-head envelope: local heads = global heads / TP, gathered heads =
  local heads * DCP, and the FP8 sparse kernel pads a head count up to 64 or
  128 (same page, section "Calculate the GLM-5.2 head envelope").
"""

from . import sharding

LATENT = 512
ROPE = 64
FP8_GROUP = 128


def kv_row_bytes(kv_dtype):
    """Bytes of one token's cache row for 'f32', 'bf16' or 'fp8_ds'."""
    if kv_dtype == "f32":
        return (LATENT + ROPE) * 4
    if kv_dtype == "bf16":
        return (LATENT + ROPE) * 2
    if kv_dtype == "fp8_ds":
        return LATENT * 1 + (LATENT // FP8_GROUP) * 4 + ROPE * 2
    raise ValueError(kv_dtype)


def bytes_per_token_per_gpu(row_bytes, layers, ranks):
    """Cache bytes one GPU holds per sequence token when `ranks` split it."""
    return row_bytes * layers / ranks


def cache_copies(tp_size, dcp_size):
    """Relative copies of the one-latent-head cache across a TP group."""
    return tp_size / dcp_size


def sequence_share(dcp_size, context_len=None):
    """Fraction of a sequence one rank stores.

    With a context length given, this is the largest shard's measured share
    under round-robin ownership; without, the limit 1 / dcp_size.
    """
    if context_len is None:
        return 1.0 / dcp_size
    lens = [int(sharding.local_len(context_len, s, dcp_size)) for s in range(dcp_size)]
    return max(lens) / context_len


def duplication_reduction(dcp_size):
    """Fractional cut in duplicated cache copies relative to DCP1."""
    return 1.0 - 1.0 / dcp_size


def head_pad(heads):
    """FP8 sparse-kernel head envelope: pad a head count to 64 or 128."""
    if heads <= 64:
        return 64
    if heads <= 128:
        return 128
    raise ValueError("head count above 128")


def head_envelope(global_heads, tp_size, dcp_size):
    """(local heads, gathered heads, local pad, gathered pad)."""
    local = global_heads // tp_size
    gathered = local * dcp_size
    return local, gathered, head_pad(local), head_pad(gathered)
