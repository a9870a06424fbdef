"""Pins for the byte formulas against the tables the pages print."""

import pytest

from oracle import accounting as acc

GiB = 1 << 30
MiB = 1 << 20


def test_fp_bytes_per_token_llama_8b(golden):
    g = golden["kv_memory_by_context_llama31_8b"]
    L, H, d = g["layers"], g["kv_heads"], g["head_dim"]
    per = acc.fp_bytes_per_token(L, H, d, 2)
    for row in g["rows"]:
        assert per * row["context"] / GiB == pytest.approx(row["fp16_GiB"], abs=0.05)
    # FP8: 1 byte per scalar
    assert acc.fp_bytes_per_token(L, H, d, 1) * 8192 / MiB == g["rows"][0]["fp8_MiB"]


def test_tq_memory_tables(golden):
    g = golden["kv_memory_by_context_llama31_8b"]
    L, H, d = g["layers"], g["kv_heads"], g["head_dim"]
    row = g["rows"][0]  # 8K, exact MiB values
    for bits, key in [(4, "tq4_MiB"), (3, "tq3_MiB"), (2, "tq2_MiB")]:
        total = 2 * L * H * acc.record_bytes(d, bits) * row["context"]
        assert total / MiB == row[key]
    for row in g["rows"][1:]:
        for bits, key in [(4, "tq4_GiB"), (3, "tq3_GiB"), (2, "tq2_GiB")]:
            total = 2 * L * H * acc.record_bytes(d, bits) * row["context"]
            assert total / GiB == pytest.approx(row[key], abs=0.05)
    for row in golden["kv_memory_by_model_32k"]["rows"]:
        Lm, Hm = row["layers"], row["kv_heads"]
        assert acc.fp_bytes_per_token(Lm, Hm, 128, 2) * 32768 / GiB == pytest.approx(row["fp16_GiB"], abs=0.05)
        for bits, key in [(4, "tq4_GiB"), (3, "tq3_GiB"), (2, "tq2_GiB")]:
            assert 2 * Lm * Hm * acc.record_bytes(128, bits) * 32768 / GiB == pytest.approx(row[key], abs=0.05)


def test_compression_ratios(golden):
    g = golden["compression_ratios"]
    for bits, nb, r16, r8 in zip(g["bits"], g["bytes_per_vector"], g["vs_fp16"], g["vs_fp8"]):
        assert acc.record_bytes(128, bits) == nb
        assert round(256 / nb, 1) == r16
        assert round(128 / nb, 1) == r8


def test_design_study_bpc(golden):
    g = golden["design_study_bpc"]
    P, H, d = g["page_tokens"], g["kv_heads"], g["head_dim"]
    hdr = acc.all_in_bpc(0, 0, 0, d, P, H)
    assert hdr == pytest.approx(g["header_bpc_about"], abs=0.0005)
    assert acc.all_in_bpc(3, 8, 0, d, 10**12, H) == pytest.approx(3 + g["u8_norm_bpc"])
    assert acc.all_in_bpc(3, 0, 24, d, 10**12, H) == pytest.approx(3 + g["sidecar_entry_bpc"])
    c = golden["design_study_compression"]
    assert acc.memory_compression(c["key_bits"], c["value_bits"]) == pytest.approx(c["r_mem_about"], abs=0.005)
    cap = golden["design_study_capacity"]
    # L*H_kv*d = 16384 reproduces "about 64 KiB per token" and "about 2 GiB at 32,768"
    per = acc.fp_bytes_per_token(16, 8, 128, 2)
    assert per == cap["bytes_per_token_KiB"] * 1024
    assert per * cap["tokens"] / GiB == pytest.approx(cap["total_GiB_about"])


def test_windowed_payload():
    # T <= W: everything FP16 (4 bytes per channel for K+V)
    assert acc.payload_bytes_windowed(1, 1, 128, 100, 128, 3, 4) == 100 * 128 * 4
    # T > W: compressed part at (bK+bV)/8 bytes per channel
    assert acc.payload_bytes_windowed(2, 8, 128, 1000, 128, 4, 4) == 2 * 8 * 128 * (872 * 1 + 128 * 4)


def test_decode_bytes_target_shape():
    # B=16, H_kv=8, T=32768, K 3-bit+QJL (72 B), V 4-bit (68 B), W=128
    assert acc.record_bytes(128, 3, qjl=True) == 72
    assert acc.record_bytes(128, 4) == 68
    assert acc.decode_algorithmic_bytes([32768] * 16, 8, 128, 3, True, 4, 128) == 593_297_408
