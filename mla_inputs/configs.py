"""Workload shapes for MLA over a shared per-token latent cache.

Every cached token holds one row ``[c_kv (d_c) | k_rope (d_r)]`` shared by all
heads (VideoMLA review, "Core Mechanism"; praveentn MLA concept page, "The RoPE
problem, and the decoupled fix").  Video workloads keep a sliding window of
whole frames in a ring buffer (VideoMLA review, "The Gap"); the language-model
decode workload is the same geometry with one token per frame.

The five named workloads are the headline shapes; ``SMALL_CONFIGS`` are reduced
shapes with the same latent widths that the CPU oracle finishes in seconds and
that still span several kernel tiles, ragged tails and a wrapped ring.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class MLAConfig:
    name: str
    batch: int
    n_heads: int
    d_model: int
    d_nope: int          # per-head content query/key width (= d_v here)
    d_v: int             # per-head value width
    d_c: int             # shared content latent width
    d_r: int             # shared decoupled rotary key width
    rope_dims: int       # 1: one band over the token position; 3: bands over (t, h, w)
    bands: tuple         # rotary band widths in order (t, h, w) or (d_r,); sum == d_r
    theta: float
    grid_h: int          # tokens per frame = grid_h * grid_w (1 x 1 for language models)
    grid_w: int
    window: int          # frames held by the ring buffer; capacity = window * P
    frames_per_block: int  # block-causal granularity in frames
    n_frames: int        # frames appended 0 .. n_frames-1 (cache length for decode)
    q_first: int         # absolute frame index of the first query frame
    q_frames: int        # number of consecutive query frames
    dtype: str           # "f32" or "bf16": storage/I-O type, fp32 accumulate
    cache_fmt: str = "dense"   # "dense", "int4", or "int2" (INT2 content latent, INT4 rotary key)
    cache_given: bool = False  # decode: earlier positions' rows are given; only the
                               # newest frame is appended
    d_cq: int = 1536     # low-rank query latent width (load-time fold of W^UQ and W^UK)
    qk_norm: bool = False  # QK-normalised attention (RMSNorm of all heads' content query / key)
    qk_eps: float = 1e-6

    # ---- derived -------------------------------------------------------
    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def capacity(self) -> int:
        return self.window * self.tokens_per_frame

    @property
    def n_q(self) -> int:
        return self.q_frames * self.tokens_per_frame

    @property
    def d_qk(self) -> int:
        return self.d_c + self.d_r

    @property
    def newest(self) -> int:
        return self.n_frames - 1

    def replace(self, **kw) -> "MLAConfig":
        return dataclasses.replace(self, **kw)

    def __post_init__(self):
        assert sum(self.bands) == self.d_r, (self.name, self.bands, self.d_r)
        assert len(self.bands) == self.rope_dims
        assert all(b % 2 == 0 for b in self.bands)
        assert self.dtype in ("f32", "bf16")
        assert self.cache_fmt in ("dense", "int4", "int2")
        assert 0 <= self.q_first and self.q_first + self.q_frames <= self.n_frames


# --------------------------------------------------------------------------
# the five headline workloads
# --------------------------------------------------------------------------
TINY_VIDEO = MLAConfig(
    name="tiny_video_f32", batch=1, n_heads=4, d_model=128, d_nope=32, d_v=32,
    d_c=64, d_r=16, rope_dims=3, bands=(4, 6, 6), theta=10000.0,
    grid_h=4, grid_w=4, window=3, frames_per_block=1,
    n_frames=3, q_first=2, q_frames=1, dtype="f32", d_cq=40)

LLM_DECODE = MLAConfig(
    name="llm_decode_bf16", batch=32, n_heads=128, d_model=16384, d_nope=128,
    d_v=128, d_c=512, d_r=64, rope_dims=1, bands=(64,), theta=10000.0,
    grid_h=1, grid_w=1, window=4096, frames_per_block=1,
    n_frames=4096, q_first=4095, q_frames=1, dtype="bf16", cache_given=True)

VIDEO_CHUNK = MLAConfig(
    name="video_chunk_bf16", batch=1, n_heads=32, d_model=4096, d_nope=128,
    d_v=128, d_c=512, d_r=64, rope_dims=3, bands=(16, 24, 24), theta=10000.0,
    grid_h=30, grid_w=52, window=12, frames_per_block=1,
    n_frames=12, q_first=11, q_frames=1, dtype="bf16")

LONG_VIDEO = MLAConfig(
    name="long_video_bf16", batch=2, n_heads=32, d_model=4096, d_nope=128,
    d_v=128, d_c=512, d_r=512, rope_dims=3, bands=(128, 192, 192), theta=10000.0,
    grid_h=30, grid_w=52, window=48, frames_per_block=1,
    n_frames=48, q_first=45, q_frames=3, dtype="bf16")

INT4_VIDEO = VIDEO_CHUNK.replace(name="int4_video_chunk", cache_fmt="int4")

CONFIGS = {1: TINY_VIDEO, 2: LLM_DECODE, 3: VIDEO_CHUNK, 4: LONG_VIDEO, 5: INT4_VIDEO}

# the deeper low-bit variant: INT2 content latent, INT4 rotary key (video-chunk shape)
INT2_VIDEO = VIDEO_CHUNK.replace(name="int2_video_chunk", cache_fmt="int2")
EXTRA_CONFIGS = {6: INT2_VIDEO}

# --------------------------------------------------------------------------
# reduced shapes (same latent widths) for whole-output parity against the oracle
# --------------------------------------------------------------------------
SMALL_CONFIGS = {
    1: TINY_VIDEO,
    # 300 written of 320 slots: poisoned unwritten tail, ragged key tiles
    2: LLM_DECODE.replace(name="llm_decode_small", batch=3, d_model=256,
                          window=320, n_frames=300, q_first=299, d_cq=200),
    # 35-token frames, ring of 4 frames wrapped once (frames 0..5 appended)
    3: VIDEO_CHUNK.replace(name="video_chunk_small", d_model=512, grid_h=5,
                           grid_w=7, window=4, n_frames=6, q_first=5, d_cq=264),
    # frame-causal 3-frame chunk over a wrapped 6-frame ring, d_r = 512
    4: LONG_VIDEO.replace(name="long_video_small", n_heads=8, d_model=512,
                          grid_h=3, grid_w=5, window=6, n_frames=9, q_first=6),
    # 36-token frames: capacity 144 (a multiple of 8, ragged last key tile)
    5: VIDEO_CHUNK.replace(name="int4_video_small", d_model=512, grid_h=6,
                           grid_w=6, window=4, n_frames=6, q_first=5,
                           cache_fmt="int4"),
    # INT2 content latent (INT4 rotary key), same shape as the INT4 case
    6: VIDEO_CHUNK.replace(name="int2_video_small", d_model=512, grid_h=6,
                           grid_w=6, window=4, n_frames=6, q_first=5,
                           cache_fmt="int2"),
}


def get_config(key) -> MLAConfig:
    if isinstance(key, MLAConfig):
        return key
    if isinstance(key, int):
        return CONFIGS[key] if key in CONFIGS else EXTRA_CONFIGS[key]
    for c in list(CONFIGS.values()) + list(EXTRA_CONFIGS.values()) + list(SMALL_CONFIGS.values()):
        if c.name == key:
            return c
    raise KeyError(key)
