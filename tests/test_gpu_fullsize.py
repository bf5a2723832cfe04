"""Parity at the full workload sizes, through the same C-ABI calls, shapes and
kernels that the benchmark times, on outputs the oracle can afford to compute:
a sample of sequences (decode), of query tokens (video chunk), of tokens and
heads (long horizon)."""
import numpy as np
import pytest

import gpu_path as gp
import oracle.mla as om
from mla_inputs import CONFIGS, get_config, make_workload

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def test_fullsize_llm_decode(gpu_lib):
    """Batch 32, 128 heads, 4096-token cache: three whole sequences."""
    cfg = CONFIGS[2]
    _case(cfg.name)
    inp = make_workload(cfg, seed=0)
    got = gp.run_gpu(cfg, inp)
    for b in (0, 13, 31):
        sub_cfg = cfg.replace(batch=1)
        sub = {k: (v[b:b + 1] if k in ("q_nope", "q_rope", "cache_c", "cache_r", "x_new") else v)
               for k, v in inp.items()}
        ref = om.run(sub_cfg, sub)
        gp.compare("cache", got["cache"][b], ref["cache"]["values"][0], cfg.dtype)
        gp.compare("q_abs", got["q_abs"][b], ref["q_abs"][0], cfg.dtype)
        gp.compare("o_lat", got["o_lat"][b], ref["o_lat"].reshape(cfg.n_q, cfg.n_heads, cfg.d_c), cfg.dtype)
        gp.compare("lse", got["lse"][b], ref["lse"].reshape(cfg.n_q, cfg.n_heads), cfg.dtype)
        gp.compare("o_heads", got["o_heads"][b], ref["o_heads"].reshape(cfg.n_q, cfg.n_heads, cfg.d_v),
                   cfg.dtype)
        gp.compare("y", got["y"][b], ref["y"].reshape(cfg.n_q, cfg.d_model), cfg.dtype)


@pytest.mark.parametrize("key", [3, 5, 6])
def test_fullsize_video_chunk(gpu_lib, key):
    """1560 query tokens x 32 heads over 18,720 keys (dense, INT4 and INT2
    content cache): the whole cache, every absorbed query, and five query
    tokens end to end."""
    cfg = get_config(key)
    _case(cfg.name)
    inp = make_workload(cfg, seed=0)
    got = gp.run_gpu(cfg, inp)
    st = om.build_cache(cfg, inp)
    if cfg.cache_fmt in ("int4", "int2"):
        written = om.slot_frames(cfg, st["newest"]) >= 0
        same = gp.check_lowbit_codes(cfg, got["codes"], got["cscale"], got["rscale"], st, written)
        print(f"low-bit code bytes equal to the oracle's: {same:.5f}", flush=True)
    else:
        gp.compare("cache", got["cache"], st["values"], cfg.dtype)
    toks = [(0, t) for t in (0, 51, 777, 1200, cfg.n_q - 1)]
    ref = om.run(cfg, inp, tokens=toks, st=st)
    gp.compare("q_abs", got["q_abs"], ref["q_abs"], cfg.dtype)
    idx = [t for _, t in toks]
    gp.compare("o_lat", got["o_lat"][0, idx], ref["o_lat"], cfg.dtype)
    gp.compare("lse", got["lse"][0, idx], ref["lse"], cfg.dtype)
    gp.compare("o_heads", got["o_heads"][0, idx], ref["o_heads"], cfg.dtype)
    gp.compare("y", got["y"][0, idx], ref["y"], cfg.dtype)


def test_fullsize_long_video(gpu_lib):
    """Batch 2, 4680 query tokens x 32 heads over 74,880 keys of 1024-wide
    rows: sampled cache rows, every absorbed query, and attention for sampled
    (token, head) pairs of all three query frames against the oracle's own
    cache (frames 45 and 46 see a frame-causal part of the window: the masked
    key tiles of the benchmark's split plan), and two tokens end to end over
    every head."""
    cfg = CONFIGS[4]
    _case(cfg.name)
    inp = make_workload(cfg, seed=0)
    got = gp.run_gpu(cfg, inp)
    P = cfg.tokens_per_frame
    st = om.build_cache(cfg, inp)
    # cache rows: every written slot of both sequences against the oracle's projection
    gp.compare("cache", got["cache"], st["values"], cfg.dtype)
    del got["cache"]
    # absorbed queries of every token
    w_uk = om.as_f64(inp["w_uk"])
    q_ref = om.absorb_query(cfg, om.as_f64(inp["q_nope"]), om.as_f64(inp["q_rope"]), w_uk, cfg.q_first)
    gp.compare("q_abs", got["q_abs"], q_ref, cfg.dtype)
    # attention for tokens of query frames 45, 46 and 47 (both sequences)
    toks = [(0, 5), (1, 777), (0, P + 3), (1, P + 1111), (0, 2 * P + 5), (1, 2 * P + 900), (1, cfg.n_q - 1)]
    heads = [0, 13, 31]
    _, o_lat, lse = om.attend(cfg, st, om.as_f64(inp["q_nope"]), q_ref[..., cfg.d_c:], w_uk,
                              om.as_f64(inp["w_uv"]), cfg.q_first, tokens=toks, heads=heads)
    mask = om.mask_matrix(cfg, cfg.q_first, st["newest"])
    for i, (b, t) in enumerate(toks):
        frame = cfg.q_first + t // P
        n_vis = int(mask[t].sum())
        _case(f"long video b={b} t={t} frame={frame} visible keys={n_vis}")
        gp.compare("o_lat", got["o_lat"][b, t, heads], o_lat[i, heads], cfg.dtype)
        gp.compare("lse", got["lse"][b, t, heads], lse[i, heads], cfg.dtype)
    # two tokens (frames 45 and 47) end to end over every head: attention,
    # then the un-absorb of the oracle's own latent output
    full = [(0, 5), (1, cfg.n_q - 1)]
    _, o_lat, lse = om.attend(cfg, st, om.as_f64(inp["q_nope"]), q_ref[..., cfg.d_c:], w_uk,
                              om.as_f64(inp["w_uv"]), cfg.q_first, tokens=full)
    for i, (b, t) in enumerate(full):
        _case(f"long video end to end b={b} t={t}")
        gp.compare("o_lat", got["o_lat"][b, t], o_lat[i], cfg.dtype)
        gp.compare("lse", got["lse"][b, t], lse[i], cfg.dtype)
        o_heads, y = om.unabsorb(o_lat[i], om.as_f64(inp["w_uv"]), om.as_f64(inp["w_o"]))
        gp.compare("o_heads", got["o_heads"][b, t], o_heads, cfg.dtype)
        gp.compare("y", got["y"][b, t], y, cfg.dtype)
