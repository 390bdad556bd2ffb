"""Writing new tokens into the sharded paged cache, written from the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it comes from:

* Cache slots of new tokens under round-robin ownership.  A token at global
  position p of request b is stored by shard p mod N as that shard's local
  token p div N ("How vLLM Serves GLM-5.3 with Million-Token Contexts on
  16 H200s", section "The core design").  A slot is a row of the shard's
  paged pool: local token j of request b lives in row j mod 64 of pool block
  block_table[b][j div 64].  A shard that does not own the token gets slot -1,
  and a negative slot means "do not write": with DCP it marks a token whose KV
  another rank owns, and it suppresses only the cache write, never the
  token's query work ("GLM-5.2 vLLM Decode Context Parallelism", section
  "Keep the current-main correctness blocker visible").
* The row each written slot receives, in the cache's storage format.  The
  packed fp8 row (512 E4M3FN codes, 4 float32 scales, 64 bf16 rope values)
  is the pages' fp8_ds_mla cache layout ("GLM-5.2 vLLM Decode Context
  Parallelism", section "Understand the cache-copy opportunity").  The pages
  do not say how the codes are chosen; the reading taken here is one float32
  scale per 128-dimension group, scale = max |x| / 448 (1 for an all-zero
  group), code = x / scale rounded to the nearest E4M3FN value, ties to the
  even code, saturating at +-448.  The scale and the quotient are float32
  divisions (IEEE, round to nearest even): they decide an integer code, so
  the oracle takes them in the same precision the GPU does.  Inputs must be
  finite.

Every encoder below is written from the format's definition (the value
table and round-to-nearest-even); none calls a library cast.
"""

import numpy as np

from .codecs import e4m3fn_to_f64

LATENT = 512
ROPE = 64
DK = LATENT + ROPE
BLOCK = 64
GROUP = 128
FP8_MAX = 448.0
ROW_BYTES = {"f32": DK * 4, "bf16": DK * 2, "fp8_ds": LATENT + 4 * 4 + ROPE * 2}

# The 127 non-negative finite E4M3FN values, indexed by code 0x00 .. 0x7E.
_E4M3_POS = e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))


def e4m3fn_encode(v):
    """float32 values -> E4M3FN codes (uint8), round to nearest, ties to even.

    The nearest of the 127 non-negative finite values is found by comparing
    |v| with the midpoints of neighbouring values (all exact in float64); a
    value exactly on a midpoint takes the even code (the code whose last
    mantissa bit is 0).  |v| beyond 448 saturates to 448.  The sign bit is
    copied, so -0.0 gives 0x80.  NaN gives 0x7F.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    # index of the largest table value <= |v| (saturated)
    lo = np.searchsorted(_E4M3_POS, np.minimum(a, FP8_MAX), side="right") - 1
    hi = np.minimum(lo + 1, 0x7E)
    mid = (_E4M3_POS[lo] + _E4M3_POS[hi]) / 2.0
    take_hi = (a > mid) | ((a == mid) & (lo % 2 == 1))
    code = np.where((hi > lo) & take_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(v), code | np.uint8(0x80), code)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def bf16_round(x):
    """float32 values -> bfloat16 bit patterns (uint16), nearest, ties to even.

    A bfloat16 value is a float32 whose low 16 bits are zero.  The two
    candidates for x are its truncation toward zero and the next bfloat16
    away from zero; the float32 halfway between them is the truncation with
    the highest dropped bit set.  |x| above the halfway value takes the
    candidate away from zero, below it the truncation, and on it the
    candidate whose last kept bit is 0.  Stepping away from zero past the
    largest finite bfloat16 gives infinity, as IEEE rounding does.  NaN gives
    a quiet NaN of the same sign.
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lower = bits & np.uint32(0xFFFF0000)
    with np.errstate(invalid="ignore"):
        half = np.abs((lower | np.uint32(0x8000)).view(np.float32).astype(np.float64))
        a = np.abs(x.astype(np.float64))
        up = (a > half) | ((a == half) & (((lower >> 16) & 1) == 1))
    out = ((lower >> 16) + up.astype(np.uint32)).astype(np.uint16)
    return np.where(np.isnan(x), ((bits >> 16) | 0x40).astype(np.uint16), out).astype(np.uint16)


def quantize_groups(latent):
    """float32 [n, 512] -> (codes uint8 [n, 512], scales float32 [n, 4]).

    Per group g of 128 dimensions: amax = max |x| (exact in float32),
    scale = float32(amax / 448) or 1 when amax is 0, code = encode(float32(x /
    scale)).
    """
    x = np.asarray(latent, dtype=np.float32)
    n = x.shape[0]
    g = x.reshape(n, LATENT // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        scales = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
        q = (g / scales[:, :, None]).astype(np.float32)
    return e4m3fn_encode(q).reshape(n, LATENT), scales


def row_bytes_for(src_f32, kv_dtype):
    """One token's 576 float32 values -> its cache row (uint8 [row_bytes]).

    f32: 576 little-endian float32.  bf16: 576 bfloat16 (rounded from the
    float32 value; exact for a bfloat16 source).  fp8_ds: 512 codes, then the
    4 group scales as little-endian float32, then 64 rope values as bfloat16.
    """
    x = np.asarray(src_f32, dtype=np.float32).reshape(DK)
    if kv_dtype == "f32":
        return x.astype("<f4").view(np.uint8).copy()
    if kv_dtype == "bf16":
        return bf16_round(x).astype("<u2").view(np.uint8).copy()
    if kv_dtype != "fp8_ds":
        raise ValueError(kv_dtype)
    codes, scales = quantize_groups(x[:LATENT].reshape(1, LATENT))
    rope = bf16_round(x[LATENT:]).astype("<u2").view(np.uint8)
    return np.concatenate([codes.reshape(-1), scales.astype("<f4").view(np.uint8).reshape(-1), rope])


def dcp_slot_mapping(req_idx, positions, block_tables, shard_begin, shard_count, n_shards,
                     pool_blocks):
    """Cache slot of each new token, -1 where none of the shards writes it.

    block_tables [shard_count][B][max_blocks]: the tables of shards
    shard_begin .. shard_begin + shard_count - 1.  For token i with request b
    and global position p >= 0: owner s = p mod N, local j = p div N; if s is
    in the shard range, slot = block_tables[s - shard_begin][b][j div 64] * 64
    + j mod 64.  Returns (slots int64 [T], bad bool [T]): `bad` marks tokens
    whose table row is too narrow for j or whose block id falls outside the
    pool; their slot is -1 (nothing is written).  Padding tokens (p < 0 or b
    outside [0, B)) get -1 and are not bad.
    """
    req_idx = np.asarray(req_idx, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    bt = np.asarray(block_tables, dtype=np.int64)
    _, B, max_blocks = bt.shape
    T = positions.shape[0]
    slots = np.full(T, -1, dtype=np.int64)
    bad = np.zeros(T, dtype=bool)
    for i in range(T):
        b, p = int(req_idx[i]), int(positions[i])
        if p < 0 or b < 0 or b >= B:
            continue
        s, j = p % n_shards, p // n_shards
        if not (shard_begin <= s < shard_begin + shard_count):
            continue
        col = j // BLOCK
        if col >= max_blocks:
            bad[i] = True
            continue
        blk = int(bt[s - shard_begin, b, col])
        if blk < 0 or blk >= pool_blocks:
            bad[i] = True
            continue
        slots[i] = blk * BLOCK + j % BLOCK
    return slots, bad


def kv_write(pool, kv_dtype, src_f32, slots):
    """The pool after writing token i's row at slots[i] for every slots[i] >= 0.

    pool: uint8 [pool_blocks * 64 * row_bytes] (copied, not modified).
    src_f32: [T][576] float32 values of the new tokens (a bfloat16 source is
    passed widened, which is exact).  A negative slot writes nothing; a slot
    at or past the end of the pool writes nothing and is reported in the
    returned `bad` mask.  Slots must be distinct.
    """
    rb = ROW_BYTES[kv_dtype]
    out = np.array(pool, dtype=np.uint8, copy=True)
    rows = out.size // rb
    slots = np.asarray(slots, dtype=np.int64)
    bad = np.zeros(slots.shape[0], dtype=bool)
    src = np.asarray(src_f32, dtype=np.float32).reshape(-1, DK)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        if s >= rows:
            bad[i] = True
            continue
        out[s * rb:(s + 1) * rb] = row_bytes_for(src[i], kv_dtype)
    return out, bad
