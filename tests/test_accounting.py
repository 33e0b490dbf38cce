"""Byte / FLOP accounting pinned to the numbers the pages print
(tests/golden/kv_bytes.json, each entry with its citation)."""
from __future__ import annotations

import json
import os

import pytest

from decode_attention_paged_slot_amd import accounting as acc

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_bytes.json")))


@pytest.mark.parametrize("row", G["bytes_per_token"], ids=lambda r: r["model"])
def test_bytes_per_token(row):
    got = acc.kv_bytes_per_token(row["layers"], row["n_kv"], row["d_h"], row["elem_bytes"])
    if "value" in row:
        assert got == row["value"]
    else:
        assert round(got / 1e6, 2) == row["value_mb_rounded"]


def test_mla_bytes_per_token():
    m = G["mla_bytes_per_token"]
    assert acc.mla_bytes_per_token(m["latent_dims"], m["layers"], m["elem_bytes"]) == m["value"]


@pytest.mark.parametrize("row", G["table_9_3_gib"]["rows"], ids=lambda r: r["design"])
def test_table_9_3(row):
    b = acc.kv_bytes_sequence(row["tokens"], 32, row["n_kv"], 128, row["elem_bytes"])
    assert acc.gib(b) == row["gib"]


def test_128k_70b_sequence():
    s = G["seq_128k_70b_gb"]
    b = acc.kv_bytes_sequence(s["tokens"], 80, 8, 128, 2)
    assert round(b / 1e9, 1) == s["value_gb"]


@pytest.mark.parametrize("row", G["table_9_1"]["rows"], ids=lambda r: f"B{r['B']}T{r['T']}")
def test_table_9_1(row):
    t = G["table_9_1"]
    kv = row["B"] * row["T"] * t["bytes_per_token"]
    assert round(kv / 1e9, 2 if kv < 1e10 else 1) == pytest.approx(row["kv_gb"], abs=0.051)
    if "floor_ms" in row:
        f = acc.decode_floor_seconds(t["weight_gb"] * 1e9, kv, t["bandwidth_tb_s"] * 1e12)
        assert round(f * 1e3, 1) == row["floor_ms"]


def test_intensity():
    i = G["intensity"]
    l8 = i["llama8b_layer"]
    flops = acc.attention_flops(l8["n_q"], l8["d_h"], 1)
    kv = acc.kv_bytes_per_token(1, l8["n_kv"], l8["d_h"], l8["elem_bytes"])
    assert flops / kv == l8["flop_per_byte"]
    assert acc.attention_intensity(l8["n_q"] // l8["n_kv"], 2) == l8["flop_per_byte"]
    assert acc.attention_intensity(i["mha_bf16"]["g"], 2) == i["mha_bf16"]["flop_per_byte"]
    assert acc.attention_intensity(i["gqa8_bf16"]["g"], 2) == i["gqa8_bf16"]["flop_per_byte"]
    sf = i["softmax_fraction_dh128_percent"]
    assert round(100 * acc.softmax_fraction(sf["d_h"]), 2) == sf["value"]


@pytest.mark.parametrize("row", G["rate_ceiling_mtok_s"]["rows"], ids=lambda r: r["device"])
def test_rate_ceiling(row):
    assert round(acc.rate_ceiling(row["tb_s"] * 1e12, 327680) / 1e6, 1) == row["value"]


@pytest.mark.parametrize("row", G["ridge_flop_per_byte"], ids=lambda r: r["device"])
def test_ridge(row):
    assert round(acc.ridge_point(row["tflops"] * 1e12, row["tb_s"] * 1e12)) == row["value"]


def test_step_bytes_70b_layer():
    sb = acc.step_bytes([32768] * 8, n_q=64, n_kv=8, d_h=128, block_size=16, kv_dtype=1,
                        q_dtype=1)
    assert sb.kv_read == 1_073_741_824
    assert sb.table_read == 8 * 2048 * 4
    assert sb.out_write == 8 * 64 * 128 * 4


def test_step_bytes_shared_prefix_unique():
    ctx = [3000, 2048, 100]
    sb = acc.step_bytes(ctx, n_q=32, n_kv=8, d_h=128, block_size=16, kv_dtype=2, q_dtype=1,
                        shared_prefix_blocks=128)
    # rows share min(128, blocks-1) blocks: 128, 127, 6 -> duplicates 127 + 6 blocks
    dup = (127 + 6) * 16 * 8 * 128 * 2
    assert sb.kv_read - sb.kv_read_unique == dup


def test_window_accounting():
    """A 4096-token window with 4 sinks on a 32k row reads 4100 positions in
    257 + 1 blocks; short rows are read whole."""
    assert acc.attended_tokens(32768, 4096, 4) == 4100
    assert acc.attended_blocks(32768, 16, 4096, 4) == 1 + 256
    assert acc.attended_tokens(4000, 4096, 4) == 4000
    assert acc.attended_blocks(4000, 16, 4096, 4) == 250
    # window start in the middle of a block: that block counts once
    assert acc.attended_blocks(100, 16, 30, 0) == 3      # positions 70..99 -> blocks 4, 5, 6
    # sinks and window sharing a block
    assert acc.attended_blocks(40, 16, 20, 5) == 3       # 0..4 -> block 0; 20..39 -> blocks 1, 2
    assert acc.attended_blocks(40, 16, 30, 5) == 3       # 0..4 and 10..39 share block 0


def test_int4_accounting():
    """4-bit cache with a residual window: half a byte per K and V element of
    the encoded blocks (SoK paper section 2.3, w_q = w / 4 for bf16), a 4-B
    value scale per encoded token and KV head, bf16 residual tokens, the
    per-channel key scales once."""
    sb = acc.step_bytes([20], n_q=4, n_kv=1, d_h=128, block_size=16, kv_dtype=4, q_dtype=1)
    # 16 encoded tokens: 2 * 16 * 128 * 0.5 = 2048 B; 4 residual: 2 * 4 * 128 * 2 = 2048 B
    assert sb.kv_read == 4096
    assert sb.scales_read == 16 * 4 + 128 * 4
    assert sb.table_read == 4                       # one encoded block
    sb = acc.step_bytes([32, 15], n_q=8, n_kv=2, d_h=64, block_size=16, kv_dtype=4, q_dtype=1)
    assert sb.kv_read == 2 * 2 * 64 * (32 // 2) + 2 * 2 * 64 * 15 * 2
    assert sb.table_read == 8
