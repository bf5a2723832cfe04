"""Deterministic synthetic inputs.

Each array ("part") is drawn from its own PCG64 stream seeded by
``(seed, part index)``, so any subset of parts can be generated in any order
with identical results.  Values are float32 standard normals times the stated
standard deviation; for bf16 workloads they are then rounded to bfloat16 (round
to nearest, ties to even) and returned as uint16 bit patterns.

Recipe (standard deviations follow "weights ~ N(0, 1/fan_in)", with fan_in the
width of the vector each weight multiplies):

=========  =======================  ===========================  =============
part       shape                    meaning                      std
=========  =======================  ===========================  =============
w_dkr      [d_c + d_r, d_model]     rows 0..d_c-1: content       1/sqrt(d_model)
                                    down-projection; rows d_c..:
                                    rotary-key projection
w_uk       [H, d_c, d_nope]         per head, the key            1/sqrt(d_c)
                                    up-projection transposed
w_uv       [H, d_v, d_c]            per head, the value          1/sqrt(d_c)
                                    up-projection
w_o        [d_model, H * d_v]       output projection            1/sqrt(H*d_v)
x          [B, n_frames, P, d_model] hidden states, frame-major  1
cache_c    [B, (n_frames-1) * P, d_c] given content latents      1
cache_r    [B, (n_frames-1) * P, d_r] given (already rotated)    1
                                    rotary keys
x_new      [B, 1, P, d_model]       hidden state of the newest   1
                                    frame, appended by the step
q_nope     [B, n_q, H, d_nope]      content queries              1
q_rope     [B, n_q, H, d_r]         rotary queries (unrotated)   1
c_q        [B, n_q, d_cq]           low-rank query latents       1
                                    (optional part)
w_uq       [H * d_nope, d_cq]       query up-projection,         1/sqrt(d_cq)
                                    output-feature major
                                    (optional part)
=========  =======================  ===========================  =============

``x`` is only drawn for workloads that build their cache by appending frames.
Optional parts (``c_q``, ``w_uq``) are drawn only when asked for by name.
Decode workloads are given the cache of every earlier position
(``cache_c``/``cache_r``) and append only the newest token from ``x_new``.
"""
from __future__ import annotations

import numpy as np

from .configs import MLAConfig

_PART_IDS = {
    "w_dkr": 1, "w_uk": 2, "w_uv": 3, "w_o": 4, "x": 5,
    "cache_c": 6, "cache_r": 7, "q_nope": 8, "q_rope": 9, "x_new": 10,
    "c_q": 11, "w_uq": 12,
}
OPTIONAL_PARTS = ("c_q", "w_uq")


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exactly equal float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def part_shapes(cfg: MLAConfig) -> dict:
    B, H, P = cfg.batch, cfg.n_heads, cfg.tokens_per_frame
    shapes = {
        "w_uk": ((H, cfg.d_c, cfg.d_nope), 1.0 / np.sqrt(cfg.d_c)),
        "w_uv": ((H, cfg.d_v, cfg.d_c), 1.0 / np.sqrt(cfg.d_c)),
        "w_o": ((cfg.d_model, H * cfg.d_v), 1.0 / np.sqrt(H * cfg.d_v)),
        "q_nope": ((B, cfg.n_q, H, cfg.d_nope), 1.0),
        "q_rope": ((B, cfg.n_q, H, cfg.d_r), 1.0),
    }
    shapes["w_dkr"] = ((cfg.d_c + cfg.d_r, cfg.d_model), 1.0 / np.sqrt(cfg.d_model))
    shapes["c_q"] = ((B, cfg.n_q, cfg.d_cq), 1.0)
    shapes["w_uq"] = ((H * cfg.d_nope, cfg.d_cq), 1.0 / np.sqrt(cfg.d_cq))
    if cfg.cache_given:
        L = (cfg.n_frames - 1) * P
        shapes["cache_c"] = ((B, L, cfg.d_c), 1.0)
        shapes["cache_r"] = ((B, L, cfg.d_r), 1.0)
        shapes["x_new"] = ((B, 1, P, cfg.d_model), 1.0)
    else:
        shapes["x"] = ((B, cfg.n_frames, P, cfg.d_model), 1.0)
    return shapes


def make_part(cfg: MLAConfig, name: str, seed: int = 0) -> np.ndarray:
    shape, std = part_shapes(cfg)[name]
    rng = np.random.default_rng([seed, _PART_IDS[name]])
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if cfg.dtype == "bf16":
        return bf16_bits_from_f32(a)
    return a


def make_workload(cfg: MLAConfig, seed: int = 0, parts=None) -> dict:
    """Return {part name: array}; float32 arrays or bf16 bit patterns (uint16)."""
    names = [n for n in part_shapes(cfg) if n not in OPTIONAL_PARTS] if parts is None else list(parts)
    return {n: make_part(cfg, n, seed) for n in names}
