"""Low-bit (INT4, INT2) latent-cache quantiser of the oracle (test
infrastructure only).

Source: the QuantMLA abstract on the "Multi-Head Latent Attention" topic page
(thelatestinai.com) quantises both cache paths of MLA, the content latent and
the decoupled rotary key, to INT4 and dequantises them inside attention; the
same abstract reports a deeper variant with the content latent in INT2 and the
rotary key in INT4.  The page does not give the number format; the workload
fixes "symmetric, fp16 scale per 32-element group" for c_kv and "one fp16
scale per token" for k_rope.  The remaining choices are readings shared with
the HIP path, written for b bits (qmax = 2^(b-1) - 1, qmin = -2^(b-1)):

* scale  s = fp16_round_to_nearest_even( fp32(amax) / qmax )   (INT4: amax / 7,
           INT2: amax / 1)
* code   q = clamp( round_half_even( fp32(x) / fp32(s) ), qmin, qmax ), IEEE
           fp32 divide; a zero scale gives all-zero codes (INT2: |x / s| <= 1,
           so the codes are -1, 0, 1)
* value  x_hat = q * s   (exact: |q| <= 8 and s has an 11-bit significand)
* packing, two's complement, element order from the low bits up: INT4 element
  2j in the low nibble of byte j; INT2 element 4j + k in bits 2k .. 2k + 1
* row layout: content codes (d_c * b / 8 bytes) then the INT4 rotary codes
  (d_r / 2 bytes)

All arithmetic is float32 NumPy so that the decisions (the integer codes) are
taken in the precision the kernel takes them in.
"""
from __future__ import annotations

import numpy as np


def group_scale(amax, bits: int = 4):
    """fp16 scale of a group whose largest magnitude is ``amax`` (float32):
    fp16_round_to_nearest_even(amax / qmax)."""
    qmax = (1 << (bits - 1)) - 1
    return (np.asarray(amax, np.float32) / np.float32(qmax)).astype(np.float16)


def codes_for(x, scale16, bits: int = 4):
    """Codes of float32 values ``x`` under fp16 scales ``scale16`` (broadcast):
    clamp(round_half_even(x / s)), and 0 where the scale is 0."""
    qmax = (1 << (bits - 1)) - 1
    qmin = -(1 << (bits - 1))
    s = np.asarray(scale16).astype(np.float32)
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(x / s)
    q = np.where(s == 0, np.float32(0), q)
    return np.clip(q, qmin, qmax).astype(np.int8)


def quantize_groups(x, group: int, bits: int = 4):
    """Quantise the last axis in groups of ``group`` elements to ``bits``-bit
    symmetric codes.

    ``x``: float array whose values are exactly representable in float32
    (the bf16-rounded cache values).  Returns (codes int8 [..., n], scales
    float16 [..., n // group]).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    assert n % group == 0
    g = x.reshape(x.shape[:-1] + (n // group, group))
    scale16 = group_scale(np.max(np.abs(g), axis=-1), bits)
    q = codes_for(g, scale16[..., None], bits)
    return q.reshape(x.shape), scale16


def admissible_groups(lo, hi, group: int, bits: int = 4):
    """Bounds on the codes and scales of ``quantize_groups`` when each input
    element may be any value in [lo, hi] (float32-exact arrays, lo <= hi).

    The scale is non-decreasing in the group maximum and the code of a fixed
    value is monotone in the value and in the scale, so the extremes are
    reached at the interval ends.  Returns (code_min, code_max int8 [..., n],
    scale_min, scale_max float16 [..., n // group])."""
    lo = np.asarray(lo, np.float32)
    hi = np.asarray(hi, np.float32)
    n = lo.shape[-1]
    shp = lo.shape[:-1] + (n // group, group)
    glo, ghi = lo.reshape(shp), hi.reshape(shp)
    small = np.where((glo <= 0) & (ghi >= 0), np.float32(0), np.minimum(np.abs(glo), np.abs(ghi)))
    big = np.maximum(np.abs(glo), np.abs(ghi))
    s_min = group_scale(np.max(small, axis=-1), bits)
    s_max = group_scale(np.max(big, axis=-1), bits)
    cands = [codes_for(x, s[..., None], bits) for x in (glo, ghi) for s in (s_min, s_max)]
    c_min = np.minimum.reduce(cands)
    c_max = np.maximum.reduce(cands)
    # a group that may be all zero may also take the smallest non-zero scales,
    # under which any non-zero value clamps: no bound but the code range
    wide = ((s_min == 0) & (s_max != 0))[..., None]
    c_min = np.where(wide & (glo < 0), np.int8(-(1 << (bits - 1))), c_min)
    c_max = np.where(wide & (ghi > 0), np.int8((1 << (bits - 1)) - 1), c_max)
    return c_min.reshape(lo.shape), c_max.reshape(lo.shape), s_min, s_max


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


def pack_crumbs(codes):
    """int8 codes in [-2, 1], length a multiple of 4 on the last axis -> uint8
    bytes (element 4j + k in bits 2k .. 2k + 1 of byte j)."""
    c = np.asarray(codes).astype(np.int16)
    assert c.shape[-1] % 4 == 0
    out = np.zeros(c.shape[:-1] + (c.shape[-1] // 4,), dtype=np.int16)
    for k in range(4):
        out |= (c[..., k::4] & 0x3) << (2 * k)
    return out.astype(np.uint8)


def unpack_crumbs(packed):
    """uint8 bytes -> int8 2-bit codes (lowest bits first), sign-extended."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 4,), dtype=np.int16)
    for k in range(4):
        out[..., k::4] = (b >> (2 * k)) & 0x3
    out = np.where(out >= 2, out - 4, out)
    return out.astype(np.int8)


def _pack(codes, bits):
    return pack_nibbles(codes) if bits == 4 else pack_crumbs(codes)


def _unpack(packed, bits):
    return unpack_nibbles(packed) if bits == 4 else unpack_crumbs(packed)


def quantize_cache_rows(rows, d_c: int, group: int = 32, content_bits: int = 4):
    """Quantise cache rows ``[..., d_c + d_r]`` (bf16 values): the content
    latent to ``content_bits`` (4 or 2) in groups of ``group``, the rotary key
    to INT4 with one scale per row.

    Returns dict with
      codes  uint8 [..., d_c * content_bits / 8 + d_r / 2]  content then rotary codes
      cscale float16 [..., d_c / group]                     per-group content scales
      rscale float16 [...]                                  per-token rotary scale
      values float64 [..., d_c + d_r]                       dequantised row values
    """
    rows = np.asarray(rows)
    c = rows[..., :d_c]
    r = rows[..., d_c:]
    qc, sc = quantize_groups(c, group) if content_bits == 4 else quantize_groups(c, group, content_bits)
    qr, sr = quantize_groups(r, r.shape[-1])
    values = np.concatenate(
        [dequantize_groups(qc, sc, group), dequantize_groups(qr, sr, r.shape[-1])], axis=-1)
    codes = np.concatenate([_pack(qc, content_bits), pack_nibbles(qr)], axis=-1)
    return {"codes": codes, "cscale": sc, "rscale": sr[..., 0], "values": values}


def dequantize_cache_rows(codes, cscale, rscale, d_c: int, group: int = 32, content_bits: int = 4):
    """Inverse of the storage: packed bytes + scales -> float64 row values."""
    codes = np.asarray(codes)
    nb = d_c * content_bits // 8
    qc = _unpack(codes[..., :nb], content_bits)
    qr = unpack_nibbles(codes[..., nb:])
    c = dequantize_groups(qc, cscale, group)
    r = dequantize_groups(qr, np.asarray(rscale)[..., None], qr.shape[-1])
    return np.concatenate([c, r], axis=-1)
