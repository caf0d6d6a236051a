"""Pins for the oracle's FP8 (E4M3) codec and its quantized paths (CPU only).

The pages fix no FP8 format; the oracle's reading is OCP E4M3 with one float32
scale per cache. These tests pin the codec to the format's closed forms and to
a brute-force nearest-value search that shares nothing with the encoder's bit
arithmetic, and the quantized attention to the bf16 path it approximates.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W

ALL = np.arange(256, dtype=np.uint8)


def test_closed_forms():
    v = oracle.fp8_value(ALL)
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and math.copysign(1, v[0x80]) < 0
    assert v[0x38] == 1.0                          # exponent field 7 = bias
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0  # largest finite
    assert v[0x08] == 2.0 ** -6                    # smallest normal
    assert v[0x01] == 2.0 ** -9                    # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                # largest subnormal
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2
    pos = v[:0x7F]
    assert (np.diff(pos) > 0).all()                # codes 0x00..0x7E are increasing
    assert np.array_equal(v[0x80:0xFF], -pos)      # sign bit mirrors


def test_round_trip_every_code():
    v = oracle.fp8_value(ALL)
    finite = ~np.isnan(v)
    back = oracle.fp8_encode(v[finite].astype(np.float32))
    assert np.array_equal(back, ALL[finite])


def _nearest(x):
    """Brute force: the finite code nearest to float32 x, ties to the even code
    (even mantissa), magnitudes past 448 saturating."""
    vals = oracle.fp8_value(ALL[:0x7F])
    a = min(abs(float(x)), 448.0)
    d = np.abs(vals - a)
    best = np.flatnonzero(d == d.min())
    c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
    return c | (0x80 if math.copysign(1.0, float(x)) < 0 else 0)


def test_encode_is_nearest_ties_to_even():
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * np.float32(2.0) ** rng.integers(-12, 10, 3000),
        # every midpoint between neighbouring codes, and a hair either side
        *(np.array([m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))], np.float32)
          for m in ((oracle.fp8_value(ALL[1:0x7F]) + oracle.fp8_value(ALL[:0x7E])) / 2).astype(np.float32)),
        np.array([448, 463.99, 464, 465, 1e6, 3e38, -500, 2.0 ** -10, 2.0 ** -11, -(2.0 ** -10)], np.float32),
    ])
    got = oracle.fp8_encode(xs)
    want = np.array([_nearest(x) for x in xs], np.uint8)
    assert np.array_equal(got, want)


def test_specials():
    c = oracle.fp8_encode(np.array([np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0], np.float32))
    assert list(c[:2]) == [0x7E, 0xFE]
    assert c[2] & 0x7F == 0x7F and c[3] & 0x7F == 0x7F
    assert list(c[4:]) == [0x00, 0x80]


def test_quantize_error_bound():
    # Within the normal range the stored value is within half a code spacing:
    # |x - value| <= 2^-4 |x| (3 mantissa bits), times the scale.
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000).astype(np.float32)
    for scale in (1.0, 1 / 64, 0.0125):
        q = oracle.quantize(x, scale)
        back = oracle.dequantize(q, scale)
        t = x.astype(np.float64) / np.float32(scale)
        normal = (np.abs(t) >= 2.0 ** -6) & (np.abs(t) <= 448)
        err = np.abs(back - x.astype(np.float64))
        assert (err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6) + 1e-12).all()


def test_fp8_decode_is_attention_on_dequantized_values():
    """The quantized decode equals plain attention on value(code) * scale, and
    stays close to the bf16 answer it approximates."""
    cfg = W.small_case("fp8", 3, 8, 2, 64, "bf16", ("uniform", 5, 60), seed=9, num_blocks=20)
    inp = W.make_inputs(cfg)
    ks, vs = 1 / 32, 1 / 16
    kq = oracle.quantize(inp.key_cache, ks)
    vq = oracle.quantize(inp.value_cache, vs)
    out, lse = oracle.paged_decode_fp8(inp.query, kq, vq, inp.block_tables, inp.context_lens, cfg.scale, ks, vs)
    Kd, Vd = oracle.dequantize(kq, ks), oracle.dequantize(vq, vs)
    q = oracle.decode_values(inp.query, "bf16")
    for i in range(cfg.num_seqs):
        n = int(inp.context_lens[i])
        Kc, Vc = oracle.gather_context(Kd, Vd, inp.block_tables[i], n, 16)
        for h in range(cfg.num_heads):
            kvh = h // (cfg.num_heads // cfg.num_kv_heads)
            s = cfg.scale * Kc[:, kvh] @ q[i, h]
            p = np.exp(s - s.max())
            assert np.allclose(out[i, h], (p / p.sum()) @ Vc[:, kvh], atol=1e-12)
            assert np.isclose(lse[i, h], s.max() + np.log(p.sum()), atol=1e-12)
    ref, _ = oracle.paged_decode(inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                                 inp.context_lens, cfg.scale, "bf16")
    assert np.abs(out - ref).max() < 0.15


def test_reshape_fp8_writes_codes_and_skips_padding():
    cfg = W.small_case("fp8r", 2, 4, 2, 64, "bf16", ("uniform", 1, 20), seed=10, num_blocks=8)
    inp = W.make_inputs(cfg)
    kc = np.zeros((8, 16, 2, 64), np.uint8)
    vc = np.zeros_like(kc)
    slots = np.array([5, -1, 8 * 16, 17], np.int64)
    key = np.repeat(inp.new_key[:1], 4, 0)
    val = np.repeat(inp.new_value[:1], 4, 0)
    k2, v2 = oracle.reshape_and_cache_fp8(key, val, kc, vc, slots, 0.5, 0.25)
    assert np.array_equal(k2[0, 5], oracle.quantize(key[0], 0.5))
    assert np.array_equal(v2[1, 1], oracle.quantize(val[3], 0.25))
    touched = np.zeros((8, 16), bool)
    touched[0, 5] = touched[1, 1] = True
    assert (k2[~touched] == 0).all() and (v2[~touched] == 0).all()
