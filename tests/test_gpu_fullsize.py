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
        same = np.mean(got["codes"] == st["codes"])
        assert same > 0.99, f"only {same:.4f} of low-bit code bytes agree"
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
    rows: sampled cache rows, the absorbed queries of the last query frame,
    attention for sampled (token, head) pairs given the stored cache, and the
    un-absorb of sampled tokens."""
    cfg = CONFIGS[4]
    _case(cfg.name)
    inp = make_workload(cfg, seed=0)
    got = gp.run_gpu(cfg, inp)
    P = cfg.tokens_per_frame
    w_dkr = om.as_f64(inp["w_dkr"])
    # cache rows against the oracle's projection and rotation
    for b in (0, 1):
        for f in (0, 23, cfg.n_frames - 1):
            toks = np.array([0, 777, P - 1])
            rows = om.project_rows(cfg, om.as_f64(inp["x"][b, f, toks]), w_dkr, f, toks)
            slots = om.slot_index(cfg, f, toks)
            gp.compare("cache rows", got["cache"][b, slots], om.round_to_storage(rows, cfg.dtype), cfg.dtype)
    # absorbed queries of the last query frame
    last = cfg.q_frames - 1
    sl = slice(last * P, (last + 1) * P)
    cfg1 = cfg.replace(q_frames=1)
    q_ref = om.absorb_query(cfg1, om.as_f64(inp["q_nope"][:, sl]), om.as_f64(inp["q_rope"][:, sl]),
                            om.as_f64(inp["w_uk"]), cfg.q_first + last)
    gp.compare("q_abs", got["q_abs"][:, sl], q_ref, cfg.dtype)
    # attention on the stored cache for sampled tokens (of the last frame) and heads
    st = {"values": got["cache"], "newest": cfg.newest}
    q_nope = np.zeros((cfg.batch, cfg.n_q, cfg.n_heads, cfg.d_nope))
    q_rot = np.zeros((cfg.batch, cfg.n_q, cfg.n_heads, cfg.d_r))
    q_nope[:, sl] = om.as_f64(inp["q_nope"][:, sl])
    q_rot[:, sl] = q_ref[..., cfg.d_c:]
    toks = [(0, last * P + 5), (1, last * P + 900), (1, cfg.n_q - 1)]
    heads = [0, 13, 31]
    _, o_lat, lse = om.attend(cfg, st, q_nope, q_rot, om.as_f64(inp["w_uk"]), om.as_f64(inp["w_uv"]),
                              cfg.q_first, tokens=toks, heads=heads)
    for i, (b, t) in enumerate(toks):
        gp.compare("o_lat", got["o_lat"][b, t, heads], o_lat[i, heads], cfg.dtype)
        gp.compare("lse", got["lse"][b, t, heads], lse[i, heads], cfg.dtype)
    # un-absorb of sampled tokens from the path's own latent output
    for b, t in toks:
        o_heads, y = om.unabsorb(got["o_lat"][b, t], om.as_f64(inp["w_uv"]), om.as_f64(inp["w_o"]))
        gp.compare("o_heads", got["o_heads"][b, t], o_heads, cfg.dtype)
        gp.compare("y", got["y"][b, t], y, cfg.dtype)
