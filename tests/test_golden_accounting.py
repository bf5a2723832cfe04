"""Byte accounting of the cache row against the widths the pages print."""
import json
import os

import numpy as np

import oracle.mla as om
from mla_inputs import CONFIGS, EXTRA_CONFIGS

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cache_widths.json")))


def _row_bytes(cfg):
    st = om.new_cache(cfg.replace(batch=1, window=1, grid_h=1, grid_w=1, n_frames=1, q_first=0, q_frames=1))
    if cfg.cache_fmt in ("int4", "int2"):
        return st["codes"].shape[-1] + 2 * st["cscale"].shape[-1] + 2
    return st["values"].shape[-1] * (2 if cfg.dtype == "bf16" else 4)


def test_videomla_row_width():
    g = GOLD["videomla_shared_cache"]
    assert g["content_latent_dims"] + g["position_key_dims"] == g["per_token_dims"]
    cfg = CONFIGS[4]          # long-horizon video: 512 latent + 512 positional dims
    assert (cfg.d_c, cfg.d_r) == (g["content_latent_dims"], g["position_key_dims"])
    assert om.new_cache(cfg.replace(window=1, grid_h=1, grid_w=1, n_frames=1, q_first=0, q_frames=1))["values"].shape[-1] == 1024
    assert _row_bytes(cfg) == 2048
    # the per-head layout it replaces: 32 heads x 128 dims for K and again for V
    ph = g["per_head_layout"]
    assert 2 * ph["heads"] * ph["dims_per_head"] == 8192


def test_latent_plus_rope_row():
    g = GOLD["mla_cache_is_latent_plus_rope"]
    cfg = CONFIGS[2]
    assert (cfg.d_c, cfg.d_r, cfg.n_heads, cfg.d_nope) == (g["d_c"], g["d_r"], g["n_h"], g["d_h"])
    assert _row_bytes(cfg) == 2 * (g["d_c"] + g["d_r"]) == 1152
    assert g["d_c"] + g["d_r"] < 2 * g["n_h"] * g["d_h"]


def test_int4_row_bytes_and_ratio():
    cfg = CONFIGS[5]
    assert _row_bytes(cfg) == 256 + 32 + 32 + 2 == 322
    ratio = _row_bytes(CONFIGS[3]) / _row_bytes(cfg)
    assert abs(ratio - GOLD["quantmla_compression"]["ratio"]) / GOLD["quantmla_compression"]["ratio"] < 0.01
    assert np.isclose(ratio, 1152 / 322)


def test_int2_row_bytes():
    # 2-bit content codes (128 B) + 4-bit rotary codes (32 B) + 16 fp16 group
    # scales + one fp16 token scale; the pages print no INT2 ratio to pin
    cfg = EXTRA_CONFIGS[6]
    assert _row_bytes(cfg) == 128 + 32 + 32 + 2 == 194
    assert np.isclose(_row_bytes(CONFIGS[3]) / _row_bytes(cfg), 1152 / 194)
