"""Pins of the KV-append oracle and of its E4M3 quantizer."""
import numpy as np

from oracle import e4m3_bits_to_f64, e4m3_quantize, kv_append, gather_latent_rows
from mla_latent_kv_16_amd.workloads import make_workload


def test_quantizer_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = e4m3_bits_to_f64(codes).astype(np.float32)
    q = e4m3_quantize(vals)
    assert np.array_equal(q, codes)


def test_quantizer_fixed_points_and_saturation():
    cases = {0.0: 0x00, 1.0: 0x38, -1.0: 0xB8, 448.0: 0x7E, 1e9: 0x7E, -1e9: 0xFE,
             464.0: 0x7E, 2.0 ** -9: 0x01, 2.0 ** -6: 0x08, 1.75: 0x3E, 0.5: 0x30}
    for x, c in cases.items():
        assert int(e4m3_quantize(np.float32(x))) == c, x


def test_quantizer_ties_go_to_even_codes():
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38
    assert int(e4m3_quantize(np.float32(1.0625))) == 0x38
    # 1.1875 is halfway between 1.125 (0x39) and 1.25 (0x3A): even code 0x3A
    assert int(e4m3_quantize(np.float32(1.1875))) == 0x3A
    # halfway between the two smallest subnormals 2^-9 (0x01) and 2^-8 (0x02)
    assert int(e4m3_quantize(np.float32(1.5 * 2.0 ** -9))) == 0x02
    # just off the tie the nearest wins
    assert int(e4m3_quantize(np.nextafter(np.float32(1.0625), np.float32(2)))) == 0x39


def test_quantizer_is_nearest_on_random_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * 64).astype(np.float32)
    q = e4m3_quantize(x)
    back = e4m3_bits_to_f64(q)
    allv = e4m3_bits_to_f64(np.arange(127, dtype=np.uint8))
    err = np.abs(np.minimum(np.abs(x.astype(np.float64)), 448.0) - np.abs(back))
    best = np.abs(np.minimum(np.abs(x.astype(np.float64)), 448)[:, None] - allv).min(axis=1)
    assert np.allclose(err, best, rtol=0, atol=0)


def test_append_writes_exactly_the_draft_rows():
    w = make_workload("tiny", seed=701, B=3, Sq=5, H=2, lens=("uniform", 60, 200))
    rng = np.random.default_rng(1)
    new = rng.integers(0, 1 << 16, size=(w.B, w.Sq, 576), dtype=np.uint16)
    out = kv_append(w.kv_pool, w.block_table, w.seq_lens, new)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        # read back through the block table: the last Sq rows are the new ones
        phys = w.block_table[b, (np.arange(L) // 64)]
        rows = out[phys, np.arange(L) % 64]
        assert np.array_equal(rows[L - w.Sq:], new[b])
        assert np.array_equal(rows[:L - w.Sq], w.kv_pool[phys, np.arange(L) % 64][:L - w.Sq])
    # nothing else in the pool changed
    touched = np.zeros(w.kv_pool.shape[:2], dtype=bool)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for j in range(L - w.Sq, L):
            touched[w.block_table[b, j // 64], j % 64] = True
    assert np.array_equal(out[~touched], w.kv_pool[~touched])
