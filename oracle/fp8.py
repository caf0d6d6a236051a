"""FP8 KV cache: codec and quantized paths (test infrastructure only).

The pages name an FP8 KV cache only as a way to enlarge the pool
(llm-stack-book 7.3 "vLLM: Architecture, PagedAttention & Internals",
"The knobs that actually matter", item 5; modernaiengineering.com lesson 13.15,
"Memory efficiency") and fix no format, so this module takes its own reading,
the plainest one:

* codes are OCP 8-bit floats E4M3 ("FN"): 1 sign bit, 4 exponent bits (bias
  7), 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; there is no
  infinity, S.1111.111 is NaN, and the largest finite magnitude is 448;
* a cache has one float32 scale (k_scale for keys, v_scale for values); a
  value x is stored as code(float32(x) / scale) with the float32 quotient
  rounded to the nearest code, ties to an even mantissa, magnitudes above 448
  (infinities included) saturating to 448 and NaN kept as NaN (sign kept);
* a code reads back as value(code) * scale; attention then runs on those
  values exactly as for bf16 caches.

Pinned in ``tests/test_oracle_fp8.py`` by the format's closed forms and by a
brute-force nearest-value search over all codes.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import attention_contiguous, decode_values, gather_context

FP8_MAX = 448.0


def fp8_value(codes) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def fp8_encode(x) -> np.ndarray:
    """E4M3 code of each float32 value: nearest, ties to even, saturating."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), FP8_MAX)                     # saturate (inf included)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    # Exponent field of the result's binade; subnormals share the bottom one.
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    step = np.exp2(e - 3)                                 # spacing of codes in this binade
    q = np.rint(a / step)                                 # round half to even (exact quotient)
    mag = q * step
    # From mantissa index q (8..16 within a normal binade, 0..8 for subnormals)
    # back to the bit fields; q == 16 carries into the next binade.
    sub = a < 2.0 ** -6
    code = np.where(sub, q, (e + 7) * 8 + (q - 8))
    code = np.where(~sub & (q == 16), (e + 8) * 8, code)
    code = np.where(mag == 0, 0, code)
    code = code.astype(np.int64) | np.where(neg, 0x80, 0)
    code = np.where(nan, 0x7F | np.where(neg, 0x80, 0), code)
    return code.astype(np.uint8)


def quantize(x, scale: float) -> np.ndarray:
    """Codes of the values ``x`` (bf16 bits as uint16, or float32) under ``scale``."""
    xf = decode_values(x, "bf16" if np.asarray(x).dtype == np.uint16 else "f32").astype(np.float32)
    return fp8_encode(xf / np.float32(scale))


def dequantize(codes, scale: float) -> np.ndarray:
    return fp8_value(codes) * np.float64(np.float32(scale))


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale: float, v_scale: float,
                          block_size: int = 16):
    """The quantizing scatter: each token's K/V codes go to its slot; padding
    (negative) and out-of-pool slots are skipped. Returns new caches."""
    kc, vc = key_cache.copy(), value_cache.copy()
    qk, qv = quantize(key, k_scale), quantize(value, v_scale)
    total = kc.shape[0] * block_size
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if 0 <= slot < total:
            kc[slot // block_size, slot % block_size] = qk[t]
            vc[slot // block_size, slot % block_size] = qv[t]
    return kc, vc


def paged_decode_fp8(query, key_cache, value_cache, block_tables, context_lens, scale: float,
                     k_scale: float, v_scale: float, q_dtype: str = "bf16", block_size: int = 16, seqs=None):
    """Paged decode over FP8 caches: each sequence's codes are gathered through
    its block table, read as code value times scale, and attended in float64
    (only the blocks a sequence owns are decoded, so pools of any size fit).
    ``seqs`` optionally restricts the work to some sequences (the rest: NaN)."""
    S, Hq, d = query.shape
    out = np.full((S, Hq, d), np.nan)
    lse = np.full((S, Hq), np.nan)
    for i in (range(S) if seqs is None else seqs):
        n = int(context_lens[i])
        Kc, Vc = gather_context(key_cache, value_cache, block_tables[i], n, block_size)
        out[i], lse[i] = attention_contiguous(decode_values(query[i], q_dtype), dequantize(Kc, k_scale),
                                              dequantize(Vc, v_scale), scale)
    return out, lse
