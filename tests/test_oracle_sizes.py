"""Pins the oracle's cache-size arithmetic to the figures printed on the pages
(tests/golden/kv_sizes.json holds each figure with its citation)."""

import json
import os

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_sizes.json")


def _entries():
    with open(GOLDEN) as f:
        data = json.load(f)
    return [(k, v) for k, v in data.items() if not k.startswith("_")]


@pytest.mark.parametrize("name,entry", _entries(), ids=[k for k, _ in _entries()])
def test_printed_cache_sizes(name, entry):
    a = entry["args"]
    if name.startswith("mha"):
        got = oracle.mha_cache_bytes(a["layers"], a["seq_len"], a["heads"], a["head_dim"],
                                     a["elem_bytes"])
    else:
        got = oracle.mla_cache_bytes_per_token(a["d_latent"], a["d_rope"], a["elem_bytes"],
                                               a["scale_bytes"]) * entry.get("layers", 1)
    assert got == entry["value"], entry["cite"]


def test_mla_vs_mha_ratio_v2_geometry():
    # DeepSeek-V2 geometry (snabindia page, section 3.1): the latent row is
    # 32768 / 576 = 56.9x smaller than the MHA K+V of one token and layer.
    mha = oracle.mha_cache_bytes(1, 1, 128, 128, 2)
    mla = oracle.mla_cache_bytes_per_token(512, 64, 2, 0)
    assert mha == 65536 and mla == 1152
    assert abs(mha / mla - 56.888) < 1e-2
