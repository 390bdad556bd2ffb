"""Pins of the oracle's number-format decoders (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import codecs


def _ocp(golden_dir):
    with open(os.path.join(golden_dir, "ocp_e4m3fn.json")) as f:
        return json.load(f)


def test_e4m3fn_table_values(golden_dir):
    g = _ocp(golden_dir)
    for code, val in g["values"].items():
        got = codecs.e4m3fn_to_f64(np.uint8(int(code, 16)))
        assert got == val, code
        assert np.signbit(got) == np.signbit(val), code
    for code in g["nan"]:
        assert np.isnan(codecs.e4m3fn_to_f64(np.uint8(int(code, 16))))


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = codecs.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_e4m3fn_is_monotone_and_symmetric():
    pos = codecs.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = codecs.e4m3fn_to_f64(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def test_bf16_bits_match_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**16, size=100000, dtype=np.uint32).astype(np.uint16)
    mine = codecs.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_bf16_known_bits():
    assert codecs.bf16_bits_to_f64(np.uint16(0x3F80)) == 1.0
    assert codecs.bf16_bits_to_f64(np.uint16(0xC000)) == -2.0
    assert codecs.bf16_bits_to_f64(np.uint16(0x3F81)) == 1.0 + 2.0 ** -7
    assert np.isneginf(codecs.bf16_bits_to_f64(np.uint16(0xFF80)))


def test_fp8_ds_group_scales_land_on_their_groups():
    codes = np.full((2, 512), 0x38, dtype=np.uint8)  # every code is 1.0
    scales = np.array([[1, 2, 3, 4], [0.5, 0.25, 8, -1]], dtype=np.float32)
    v = codecs.fp8_ds_latent_to_f64(codes, scales)
    for g in range(4):
        assert np.all(v[:, g * 128:(g + 1) * 128] == scales[:, g:g + 1])
    codes[0, 127] = 0x40  # 2.0 at the last dim of group 0
    codes[0, 128] = 0x30  # 0.5 at the first dim of group 1
    v = codecs.fp8_ds_latent_to_f64(codes, scales)
    assert v[0, 127] == 2.0 and v[0, 128] == 1.0


@pytest.mark.parametrize("x", [0.1, -3.7, 447.9, 1e-4])
def test_fp8_decode_inverts_torch_encode(x):
    code = torch.tensor([x], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    v = codecs.e4m3fn_to_f64(code)[0]
    # nearest representable: relative error at most 2^-4 for normals
    assert abs(v - x) <= max(abs(x) * 2.0 ** -4, 2.0 ** -10)
