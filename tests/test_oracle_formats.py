"""Pins for the oracle's number formats and MXFP4 layout (CPU only).

T1 decode over every byte and scale code against the published E2M1 table;
T2 nibble order by a one-hot construction; T3 the pages' packed shapes;
T4 the pages' parameter and byte counts; T5 the pages' group statistic;
bf16 conversions at hand-checked values.
"""
import json
import os

import numpy as np
import pytest

from oracle import mxfp4, numerics
from oracle.mxfp4 import decode, decode_glu_record, split_glu_record
from workload import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    with open(os.path.join(GOLD, "k3_pages_facts.json")) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


def _e2m1_ocp():
    with open(os.path.join(GOLD, "e2m1_ocp.json")) as f:
        return np.array(json.load(f)["values"])


def test_t1_decode_every_byte_and_scale():
    table = _e2m1_ocp()
    for code in (119, 120, 121, 122, 123, 127, 1, 254):
        packed = np.arange(256, dtype=np.uint8).reshape(16, 16)     # 16 rows x 32 values
        scales = np.full((16, 1), code, dtype=np.uint8)
        got = decode(packed, scales, 16, 32)
        scale = 2.0 ** (code - 127)
        for b in range(256):
            r, j = divmod(b, 16)
            assert got[r, 2 * j] == table[b & 0xF] * scale
            assert got[r, 2 * j + 1] == table[b >> 4] * scale
            # signed zero of code 8 is kept
            if (b & 0xF) == 8:
                assert np.signbit(got[r, 2 * j])


def test_t1_table_matches_bitfield_definition():
    # E2M1: sign | 2-bit exponent (bias 1) | 1 mantissa bit; exponent 0 is subnormal (0.5*m)
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m)
        assert numerics.e2m1_value(code) == (-mag if s else mag)
    assert numerics.e2m1_value(1) == 0.5          # the subnormal is not flushed
    assert np.isnan(numerics.e8m0_value(255))
    assert numerics.e8m0_value(127) == 1.0 and numerics.e8m0_value(0) == 2.0 ** -127


def test_t2_low_nibble_is_first_element():
    packed = np.zeros((1, 16), dtype=np.uint8)
    scales = np.full((1, 1), 127, dtype=np.uint8)
    packed[0, 0] = 0x02                      # low nibble = code 2 = 1.0, high nibble = 0
    got = decode(packed, scales, 1, 32)
    assert got[0, 0] == 1.0 and np.all(got[0, 1:] == 0.0)
    packed[0, 0] = 0x70                      # high nibble = code 7 = 6.0
    got = decode(packed, scales, 1, 32)
    assert got[0, 1] == 6.0 and got[0, 0] == 0.0 and np.all(got[0, 2:] == 0.0)


def test_t2_scale_group_is_32_consecutive_weights_of_a_row():
    packed = np.full((2, 32), 0x22, dtype=np.uint8)    # every weight 1.0, 64 per row
    scales = np.array([[120, 121], [122, 123]], dtype=np.uint8)
    got = decode(packed, scales, 2, 64)
    assert np.all(got[0, :32] == 2.0 ** -7) and np.all(got[0, 32:] == 2.0 ** -6)
    assert np.all(got[1, :32] == 2.0 ** -5) and np.all(got[1, 32:] == 2.0 ** -4)


def test_t3_page_shapes_decode_to_dense_shapes():
    f = _facts()
    c = gen.named_config("decode16")
    packed, scales = gen.make_expert(c, 0, 0)
    (p1, s1), (p3, s3), (p2, s2) = split_glu_record(packed, scales, c.latent, c.inter)
    assert p1.reshape(f["w1_packed_shape"]).shape == tuple(f["w1_packed_shape"])
    assert s1.reshape(f["w1_scale_shape"]).shape == tuple(f["w1_scale_shape"])
    assert p2.reshape(f["w2_packed_shape"]).shape == tuple(f["w2_packed_shape"])
    assert s2.reshape(f["w2_scale_shape"]).shape == tuple(f["w2_scale_shape"])
    w1, w3, w2 = decode_glu_record(packed, scales, c.latent, c.inter)
    assert w1.shape == tuple(f["w13_dense_shape"]) == w3.shape
    assert w2.shape == tuple(f["w2_dense_shape"])
    # 1792 bytes at 4 bits = 3584 values; 112 scales x 32 = 3584
    assert f["w1_packed_shape"][1] * 2 == f["w1_scale_shape"][1] * 32 == f["latent"]


def test_t4_parameter_and_byte_counts():
    f = _facts()
    c = gen.named_config("decode16")
    params = 3 * c.inter * c.latent
    assert params == 33_030_144
    assert round(params / 1e6, 1) == f["params_per_expert_M_1dp"]
    assert round(params / 1e6, 2) == f["params_per_expert_M_2dp"]
    assert abs(round(f["params_per_expert_M_2dp"] * 1e6) * 896 / 1e9 - f["routed_params_B_per_layer"]) < 1e-3
    assert round(92 * 896 * params / 1e12, 2) == f["routed_params_T_all_layers"]
    assert round(92 * 896 * params / 1e12, 3) == f["routed_params_T_review"]
    naive = 3 * c.inter * c.hidden
    assert round(naive / 1e6, 2) == f["params_per_expert_no_latent_M"]
    assert round(92 * 896 * naive / 1e12, 2) == f["routed_params_no_latent_T"]
    rec = gen.expert_record_bytes(c) + gen.expert_scale_bytes(c)
    assert rec == 17_547_264
    assert round(rec / 1e6, 1) == f["expert_record_MB"]
    assert round(rec / 2 ** 20, 1) == f["expert_record_MiB_as_shipped"]
    assert f["n_experts_all_layers"] == 92 * 896
    # the page multiplies its rounded 17.5 MB by 82,432 (exact bytes give 1.4465 TB)
    assert round(round(rec / 1e6, 1) * f["n_experts_all_layers"] / 1e6, 2) == f["routed_TB_all"]
    assert abs(rec * f["n_experts_all_layers"] / 1e12 - f["routed_TB_all"]) < 0.01
    assert rec * 8 / params == f["bits_per_weight"]
    assert 896 * rec == 15_722_348_544
    sh = gen.shared_record_bytes(c) + gen.shared_scale_bytes(c)
    assert sh == 3 * c.shared_inter * c.hidden * 4.25 / 8 == 70_189_056
    assert c.shared_inter == f["shared_merged_inter"]
    assert [c.hidden, c.shared_inter] == f["gguf_shared_shape"]


def test_t5_group_amax_over_scale_statistic():
    """Every decoded group has amax/scale <= 6 (the largest E2M1 magnitude); the pages'
    (3, 6] statistic holds for real groups, and for uniform synthetic codes it fails
    only when all 32 codes have magnitude <= 3, probability 0.75**32 ~ 1e-4."""
    lo, hi = _facts()["group_amax_over_scale_interval"]
    c = gen.LayerConfig("t5", T=1, hidden=256, latent=256, inter=256, n_experts=1, topk=1)
    packed, scales = gen.make_expert(c, 0, 0)
    w1, w3, w2 = decode_glu_record(packed, scales, c.latent, c.inter)
    (_, s1), _, _ = split_glu_record(packed, scales, c.latent, c.inter)
    amax = np.abs(w1).reshape(-1, 32).max(axis=1)
    ratio = amax / numerics.e8m0_value(s1)
    assert np.all(ratio <= hi)
    inside = np.mean((ratio > lo) & (ratio <= hi))
    assert inside > 0.995


@pytest.mark.parametrize("value,expected_bits", [
    (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000),
    (1.0 + 2.0 ** -8, 0x3F80),            # exact tie -> even (mantissa 0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie between 0x3F81 and 0x3F82 -> even 0x3F82
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie -> up
    (3.0e38 * 2, 0x7F80),                 # overflow -> +inf
    (2.0 ** -133, 0x0001),                # smallest bf16 subnormal
    (2.0 ** -134, 0x0000),                # half of it: tie -> even (zero)
    (3 * 2.0 ** -134, 0x0002),            # 1.5 quanta: tie -> even (2 quanta)
])
def test_bf16_rounding_cases(value, expected_bits):
    assert int(numerics.f64_to_bf16(np.array([value]))[0]) == expected_bits


def test_bf16_roundtrip_exact():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = numerics.bf16_to_f64(bits)
    fin = np.isfinite(v)
    back = numerics.f64_to_bf16(v[fin])
    # every finite bf16 value maps back to itself (-0 keeps its sign bit)
    assert np.array_equal(back, bits[fin])
