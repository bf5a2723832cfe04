"""INT4 latent-cache quantiser of the oracle (test infrastructure only).

Source: the QuantMLA abstract on the "Multi-Head Latent Attention" topic page
(thelatestinai.com) quantises both cache paths of MLA, the content latent and
the decoupled rotary key, to INT4, and dequantises them inside attention.  The
page does not give the number format; the workload fixes "symmetric, fp16
scale per 32-element group" for c_kv and "one fp16 scale per token" for
k_rope.  The remaining choices are readings shared with the HIP path:

* scale  s = fp16_round_to_nearest_even( fp32(amax) / 7.0f )
* code   q = clamp( round_half_even( fp32(x) / fp32(s) ), -8, 7 ), IEEE fp32 divide;
           a zero scale gives all-zero codes
* value  x_hat = q * s   (exact: |q| <= 8 and s has an 11-bit significand)
* packing: element 2j in the low nibble, 2j+1 in the high nibble, two's complement

All arithmetic is float32 NumPy so that the decisions (the integer codes) are
taken in the precision the kernel takes them in.
"""
from __future__ import annotations

import numpy as np


def quantize_groups(x, group: int):
    """Quantise the last axis in groups of ``group`` elements.

    ``x``: float array whose values are exactly representable in float32
    (the bf16-rounded cache values).  Returns (codes int8 [..., n], scales
    float16 [..., n // group]).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    assert n % group == 0
    g = x.reshape(x.shape[:-1] + (n // group, group))
    amax = np.max(np.abs(g), axis=-1)
    scale16 = (amax / np.float32(7.0)).astype(np.float16)
    s = scale16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(g / s)
    q = np.where(s == 0, np.float32(0), q)
    q = np.clip(q, -8, 7).astype(np.int8)
    return q.reshape(x.shape), scale16


def dequantize_groups(codes, scales, group: int):
    """Exact values q * s as float64 (last axis grouped by ``group``)."""
    codes = np.asarray(codes)
    n = codes.shape[-1]
    q = codes.astype(np.float64).reshape(codes.shape[:-1] + (n // group, group))
    s = np.asarray(scales).astype(np.float64)[..., None]
    return (q * s).reshape(codes.shape)


def pack_nibbles(codes):
    """int8 codes in [-8, 7], even length on the last axis -> uint8 bytes."""
    c = np.asarray(codes).astype(np.int16)
    assert c.shape[-1] % 2 == 0
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """uint8 bytes -> int8 codes (low nibble first), sign-extended."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo = b & 0xF
    hi = b >> 4
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


def quantize_cache_rows(rows, d_c: int, group: int = 32):
    """Quantise cache rows ``[..., d_c + d_r]`` (bf16 values).

    Returns dict with
      codes  uint8 [..., (d_c + d_r) / 2]  content codes then rotary codes
      cscale float16 [..., d_c / group]    per-group content scales
      rscale float16 [...]                 per-token rotary scale
      values float64 [..., d_c + d_r]      dequantised row values
    """
    rows = np.asarray(rows)
    c = rows[..., :d_c]
    r = rows[..., d_c:]
    qc, sc = quantize_groups(c, group)
    qr, sr = quantize_groups(r, r.shape[-1])
    values = np.concatenate(
        [dequantize_groups(qc, sc, group), dequantize_groups(qr, sr, r.shape[-1])], axis=-1)
    codes = np.concatenate([pack_nibbles(qc), pack_nibbles(qr)], axis=-1)
    return {"codes": codes, "cscale": sc, "rscale": sr[..., 0], "values": values}


def dequantize_cache_rows(codes, cscale, rscale, d_c: int, group: int = 32):
    """Inverse of the storage: packed bytes + scales -> float64 row values."""
    q = unpack_nibbles(codes)
    qc, qr = q[..., :d_c], q[..., d_c:]
    c = dequantize_groups(qc, cscale, group)
    r = dequantize_groups(qr, np.asarray(rscale)[..., None], qr.shape[-1])
    return np.concatenate([c, r], axis=-1)
