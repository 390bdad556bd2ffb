"""The tables and sums the pages print, against the oracle's arithmetic."""
import json
import os
from fractions import Fraction

import pytest

from oracle import capacity


@pytest.fixture(scope="module")
def tables(golden_dir):
    with open(os.path.join(golden_dir, "page_tables.json")) as f:
        return json.load(f)


def test_copy_geometry(tables):
    t = tables["copy_geometry"]
    for row in t["rows"]:
        assert capacity.cache_copies(t["tp"], row["dcp"]) == row["copies"]
        assert capacity.sequence_share(row["dcp"]) == float(Fraction(row["share"]))
        # measured share of the round-robin deal over a long context
        assert capacity.sequence_share(row["dcp"], 1048576) == float(Fraction(row["share"]))
        assert capacity.duplication_reduction(row["dcp"]) * 100 == pytest.approx(row["reduction_pct"])


def test_head_envelope(tables):
    t = tables["head_envelope"]
    for row in t["rows"]:
        got = capacity.head_envelope(t["global_heads"], t["tp"], row["dcp"])
        assert got == (row["local"], row["gathered"], row["local_pad"], row["gathered_pad"])


def test_row_bytes(tables):
    t = tables["mla_row_bytes"]
    assert capacity.kv_row_bytes("bf16") == t["bf16_row_bytes"]
    per = capacity.bytes_per_token_per_gpu(t["bf16_row_bytes"], t["layers"], t["gpus"])
    assert per == t["bytes_per_token_per_gpu"]
    assert round(per * t["tokens"] / 2**30, 2) == t["gib_per_gpu"]
    assert capacity.kv_row_bytes("fp8_ds") == 656
    assert capacity.kv_row_bytes("f32") == 2304


def test_reporter_concurrency(tables):
    t = tables["reporter_concurrency"]
    assert round(t["kv_tokens_per_gpu"] / t["request_tokens"], 4) == t["ratio"]


def test_million_token_share(tables):
    t = tables["million_token_share"]
    share = capacity.sequence_share(t["ranks"], t["context"])
    assert round(t["total_gib"] * share, 1) == t["per_gpu_gib_approx"]
