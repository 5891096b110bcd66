"""Pins for the E4M3 (OCP FP8 E4M3FN) latent-pool path of the oracle and of the
seeded input generator.

The decode is pinned to the format's definition (sign, 4-bit exponent with bias 7,
3-bit mantissa, subnormals at exponent 0, one NaN pattern per sign, no infinity,
largest finite value 448), the generator's rounding to a brute-force nearest search
with ties to the even code, and the fp8 oracle to the bf16 oracle on a pool whose
dequantized values are exactly bf16 (a power-of-two scale).
"""
import numpy as np
import pytest

from oracle import E4M3Pool, bf16_bits_to_f64, e4m3_bits_to_f64, mla_attention_folded
from mla_latent_kv_16_amd.workloads import (
    E4M3_NAN, f32_to_bf16_bits, f32_to_e4m3_bits, make_workload)

ALL = np.arange(256, dtype=np.uint8)


def test_e4m3_fixed_points():
    v = e4m3_bits_to_f64(ALL)
    assert v[0x00] == 0.0 and not np.signbit(v[0x00])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x38] == 1.0          # exponent 7 = bias, mantissa 0
    assert v[0x39] == 1.125
    assert v[0x40] == 2.0
    assert v[0x08] == 2.0 ** -6    # smallest normal
    assert v[0x07] == 7 * 2.0 ** -9  # largest subnormal
    assert v[0x01] == 2.0 ** -9    # smallest subnormal
    assert v[0x7E] == 448.0        # largest finite
    assert v[0xFE] == -448.0
    assert v[0x77] == 240.0        # 1.875 * 2^7
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v[E4M3_NAN])


def test_e4m3_structure():
    v = e4m3_bits_to_f64(ALL)
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # strictly increasing codes
    assert np.array_equal(v[0x80:0xFF], -pos)            # sign bit mirrors
    assert np.isnan(v).sum() == 2
    assert np.allclose(np.diff(pos[:9]), 2.0 ** -9)      # uniform subnormal spacing
    for e in range(1, 16):                               # binade e: 8 evenly spaced values
        codes = [(e << 3) | m for m in range(8) if (e << 3) | m < 0x7F]
        d = np.diff(v[codes])
        assert np.allclose(d, 2.0 ** (e - 7) / 8)


def test_quantizer_nearest_with_ties_to_even():
    table = e4m3_bits_to_f64(ALL[:0x7F])
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000) * 50, rng.uniform(-500, 500, 2000),
                        rng.standard_normal(1000) * 0.01]).astype(np.float32)
    q = f32_to_e4m3_bits(x)
    got = e4m3_bits_to_f64(q)
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    dist = np.abs(table[None, :] - a[:, None])
    best = dist.min(axis=1)
    assert np.isfinite(got).all()
    assert np.allclose(np.abs(np.abs(got) - a), best, rtol=0, atol=0)
    assert np.array_equal(np.signbit(got), np.signbit(x))
    # exact midpoints go to the even code
    assert f32_to_e4m3_bits(np.float32(1.0625)) == 0x38
    assert f32_to_e4m3_bits(np.float32(1.1875)) == 0x3A
    assert f32_to_e4m3_bits(np.float32(-1.0625)) == 0xB8
    # saturation
    assert f32_to_e4m3_bits(np.float32(1000.0)) == 0x7E
    assert f32_to_e4m3_bits(np.float32(-1e6)) == 0xFE


def test_quantizer_round_trips_every_finite_code():
    v = e4m3_bits_to_f64(ALL)
    fin = ~np.isnan(v)
    assert np.array_equal(f32_to_e4m3_bits(v[fin].astype(np.float32)), ALL[fin])


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_oracle_equals_bf16_oracle_on_exact_values(causal):
    """kv_scale = 2^-6: every dequantized value is exactly a bf16 value, so the fp8
    pool and the bf16 pool holding those values give the same fp64 result."""
    w = make_workload("tiny", seed=31, B=2, Sq=3, H=4, lens=("uniform", 70, 200),
                      kv_format="e4m3", kv_scale=2.0 ** -6, causal=causal)
    deq = e4m3_bits_to_f64(w.kv_pool) * w.kv_scale
    stray = np.isnan(deq)
    bf = f32_to_bf16_bits(np.where(stray, np.nan, deq).astype(np.float32))
    assert np.array_equal(bf16_bits_to_f64(bf)[~stray], deq[~stray])
    O8, l8 = mla_attention_folded(w.q_nope, w.q_rope, E4M3Pool(w.kv_pool, w.kv_scale),
                                  w.block_table, w.seq_lens, w.scale, w.causal)
    Ob, lb = mla_attention_folded(w.q_nope, w.q_rope, bf, w.block_table, w.seq_lens,
                                  w.scale, w.causal)
    assert np.isfinite(O8).all()
    assert np.array_equal(O8, Ob) and np.array_equal(l8, lb)


def test_fp8_workload_is_the_quantized_bf16_workload():
    """Same seed: the E4M3 pool holds the bf16 workload's draws divided by the scale
    and rounded (checked within the rounding of both formats)."""
    wb = make_workload("tiny", seed=32, B=1, Sq=1, H=2, lens=("fixed", 130))
    w8 = make_workload("tiny", seed=32, B=1, Sq=1, H=2, lens=("fixed", 130),
                       kv_format="e4m3", kv_scale=0.02)
    assert np.array_equal(wb.block_table, w8.block_table)
    vb = bf16_bits_to_f64(wb.kv_pool)
    v8 = e4m3_bits_to_f64(w8.kv_pool) * 0.02
    live = ~np.isnan(vb)
    assert np.array_equal(live, ~np.isnan(v8))
    rel = np.abs(v8[live] - vb[live]) / np.maximum(np.abs(vb[live]), 2.0 ** -6 * 0.02)
    assert rel.max() <= 2.0 ** -4 + 2.0 ** -8
