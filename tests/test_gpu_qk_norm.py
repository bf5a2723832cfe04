"""QK-normalised MLA on the HIP path (static weights folded at load time,
per-slot key inverse RMS, query inverse RMS, the content score scaled in
attention) against the oracle's materialised definition, through the C-ABI."""
import numpy as np
import pytest

import gpu_path as gp
import oracle.mla as om
from mla_inputs import SMALL_CONFIGS, bf16_bits_from_f32, make_workload

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _weights(cfg, seed):
    rng = np.random.default_rng(seed)
    g = [rng.uniform(0.5, 1.5, (cfg.n_heads, cfg.d_nope)).astype(np.float32) for _ in range(2)]
    if cfg.dtype == "bf16":
        return [bf16_bits_from_f32(x) for x in g]
    return g


def run_qkn(cfg, inp, g_q, g_k, fill=None):
    """Append (and store every row's key inverse RMS), absorb with the folded
    weight, attend.  Returns host arrays and device tensors."""
    import torch
    from head_latent_attention_cache_amd import api
    dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
    B, H, P = cfg.batch, cfg.n_heads, cfg.tokens_per_frame
    dt = api.torch_dtype(dims)
    cache, aux = api.new_cache(dims, geom, fill=fill)
    w_uk = gp.to_device(inp["w_uk"])
    w_fold = torch.empty_like(w_uk)
    gram = torch.empty((cfg.d_c, cfg.d_c), dtype=torch.float32, device="cuda")
    api.qk_norm_prepare(dims, w_uk, gp.to_device(g_q), gp.to_device(g_k), w_fold, gram)
    w_dkr = gp.to_device(inp["w_dkr"])
    ws = torch.empty(max(16, api.append_workspace_bytes(dims, geom, P)), dtype=torch.uint8, device="cuda")
    if cfg.cache_given:
        L = inp["cache_c"].shape[1]
        cache[:, :L, :cfg.d_c] = gp.to_device(inp["cache_c"])
        cache[:, :L, cfg.d_c:] = gp.to_device(inp["cache_r"])
        api.cache_key_norm(dims, geom, L, gp.int_tensor([0] * B), gram, cache, aux)
        f_new = gp.int_tensor([cfg.n_frames - 1] * B)
        api.cache_append(dims, geom, gp.to_device(inp["x_new"]).reshape(B, P, cfg.d_model), f_new, w_dkr,
                         cache, aux, workspace=ws)
        api.cache_key_norm(dims, geom, P, f_new, gram, cache, aux)
    else:
        x = gp.to_device(inp["x"])
        for f in range(cfg.n_frames):
            ft = gp.int_tensor([f] * B)
            api.cache_append(dims, geom, x[:, f].contiguous(), ft, w_dkr, cache, aux, workspace=ws)
            api.cache_key_norm(dims, geom, P, ft, gram, cache, aux)
    q_first = gp.int_tensor([cfg.q_first] * B)
    q_abs = torch.empty((B, cfg.n_q, H, cfg.d_qk), dtype=dt, device="cuda")
    api.absorb_q(dims, geom, gp.to_device(inp["q_nope"]), gp.to_device(inp["q_rope"]), q_first, w_fold, q_abs)
    o_lat = torch.empty((B, cfg.n_q, H, cfg.d_c), dtype=dt, device="cuda")
    lse = torch.empty((B, cfg.n_q, H), dtype=torch.float32, device="cuda")
    api.attention(dims, geom, q_abs, q_first, gp.int_tensor([cfg.newest] * B), cache, aux, o_lat, lse)
    torch.cuda.synchronize()
    return {"o_lat": gp.to_host(o_lat), "lse": gp.to_host(lse), "dims": dims, "geom": geom, "cache": cache,
            "aux": aux, "gram": gram}


# decode (bf16), video chunk (bf16), INT4 and INT2 chunks (narrow MFMA kernel),
# the fp32 tiny video (generic kernel), the d_r = 512 long video (wide-row
# kernel; capacity 90 reads the key statistic one value at a time) and a
# 4 x 5 grid of the long video (capacity 120, a multiple of 4: the wide-row
# kernel's 16-byte reads of the key statistic, with a ragged last tile)
QKN_CASES = {key: SMALL_CONFIGS[key] for key in (2, 3, 5, 6, 1, 4)}
QKN_CASES["4x5"] = SMALL_CONFIGS[4].replace(name="long_video_small_4x5", grid_h=4, grid_w=5)
# the long video with 4 of 6 ring frames written, the other slots (and their
# key statistics) NaN bit patterns: masked tiles of the wide-row kernel
QKN_CASES["4_partial"] = SMALL_CONFIGS[4].replace(name="long_video_small_partial", n_frames=4, q_first=1)
# a longer key loop for the wide-row kernel: 30 key tiles per row block (the
# key-scale slots rotate through many steps), 48-token frames, a wrapped
# 20-frame ring, frame-causal 3-frame chunk
QKN_CASES["4_medium"] = SMALL_CONFIGS[4].replace(name="long_video_medium", grid_h=6, grid_w=8, window=20, n_frames=23,
                                                 q_first=20)


@pytest.mark.parametrize("key", list(QKN_CASES))
def test_qk_norm_matches_oracle(gpu_lib, key):
    import torch
    from head_latent_attention_cache_amd import api
    cfg = QKN_CASES[key].replace(qk_norm=True, qk_eps=EPS)
    if key == "4x5":
        assert cfg.capacity % 4 == 0 and cfg.capacity % 32 != 0
    _case(f"qk norm {cfg.name}")
    inp = make_workload(cfg, seed=41)
    g_q, g_k = _weights(cfg, 42)
    got = run_qkn(cfg, inp, g_q, g_k, fill=0xFF if cfg.cache_given or key == "4_partial" else None)
    st = om.build_cache(cfg, inp)
    w_uk, w_uv = om.as_f64(inp["w_uk"]), om.as_f64(inp["w_uv"])
    q_nope = om.as_f64(inp["q_nope"])
    q_rot = om.absorb_query(cfg, q_nope, om.as_f64(inp["q_rope"]), w_uk, cfg.q_first)[..., cfg.d_c:]
    _, o_lat, lse = om.attend_qk_norm(cfg, st, q_nope, q_rot, w_uk, w_uv, om.as_f64(g_q), om.as_f64(g_k), EPS,
                                      cfg.q_first)
    B, n_q, H = cfg.batch, cfg.n_q, cfg.n_heads
    gp.compare("o_lat", got["o_lat"], o_lat.reshape(B, n_q, H, cfg.d_c), cfg.dtype)
    gp.compare("lse", got["lse"], lse.reshape(B, n_q, H), cfg.dtype)
    # the stored key inverse RMS against its definition on the oracle's cache
    # (the two caches' latents differ at most by storage rounding, which moves
    # a statistic over H * d_nope values far less than the bound)
    ks = api.key_scales(got["dims"], got["geom"], got["aux"])
    torch.cuda.synchronize()
    written = om.slot_frames(cfg, cfg.newest) >= 0
    k = np.einsum("bsc,hci->bshi", st["values"][:, written, :cfg.d_c], w_uk)
    want = 1.0 / np.sqrt(np.mean(k * k, axis=(2, 3)) + EPS)
    have = ks.cpu().numpy().astype(np.float64)[:, written]
    assert np.max(np.abs(have - want) / want) < 5e-4
    # the Gram matrix of the key up-projection
    gram = np.einsum("hai,hbi->ab", w_uk, w_uk)
    assert np.max(np.abs(got["gram"].cpu().numpy() - gram)) <= 1e-4 * np.max(np.abs(gram))


def test_qk_norm_full_decode_shape_sampled(gpu_lib):
    """Batch 32, 128 heads, 4096 keys: three whole sequences."""
    from mla_inputs import CONFIGS
    cfg = CONFIGS[2].replace(qk_norm=True, qk_eps=EPS)
    _case(f"qk norm {cfg.name}")
    inp = make_workload(cfg, seed=43)
    g_q, g_k = _weights(cfg, 44)
    got = run_qkn(cfg, inp, g_q, g_k)
    for b in (0, 17, 31):
        sub_cfg = cfg.replace(batch=1)
        sub = {k: (v[b:b + 1] if k in ("q_nope", "q_rope", "cache_c", "cache_r", "x_new") else v)
               for k, v in inp.items()}
        st = om.build_cache(sub_cfg, sub)
        w_uk, w_uv = om.as_f64(inp["w_uk"]), om.as_f64(inp["w_uv"])
        q_nope = om.as_f64(sub["q_nope"])
        q_rot = om.absorb_query(sub_cfg, q_nope, om.as_f64(sub["q_rope"]), w_uk, cfg.q_first)[..., cfg.d_c:]
        _, o_lat, lse = om.attend_qk_norm(sub_cfg, st, q_nope, q_rot, w_uk, w_uv, om.as_f64(g_q), om.as_f64(g_k),
                                          EPS, cfg.q_first)
        gp.compare("o_lat", got["o_lat"][b], o_lat.reshape(cfg.n_q, cfg.n_heads, cfg.d_c), cfg.dtype)
        gp.compare("lse", got["lse"][b], lse.reshape(cfg.n_q, cfg.n_heads), cfg.dtype)
