"""A step's four library calls captured in a HIP graph (as the benchmark
times them): every replay reproduces the direct-call results bit for bit,
with eager work (the outputs overwritten) and synchronisations between the
replays."""
import numpy as np
import pytest

import gpu_path as gp
from mla_inputs import SMALL_CONFIGS, make_workload

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


@pytest.mark.parametrize("key", [2, 3, 5, 6])
def test_graph_replay_matches_direct_calls(gpu_lib, key):
    import torch
    from head_latent_attention_cache_amd import api

    cfg = SMALL_CONFIGS[key]
    print(f"[case] graph replay, workload {cfg.name}", flush=True)
    inp = make_workload(cfg, seed=3)
    dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
    B, H, P = cfg.batch, cfg.n_heads, cfg.tokens_per_frame
    dt = api.torch_dtype(dims)
    dev = "cuda"
    w_dkr, w_uk, w_uv, w_o = (gp.to_device(inp[k]) for k in ("w_dkr", "w_uk", "w_uv", "w_o"))
    q_nope, q_rope = gp.to_device(inp["q_nope"]), gp.to_device(inp["q_rope"])

    # cache state before the step; the step appends the newest frame(s)
    step_frames = 1 if cfg.cache_given else cfg.n_frames - cfg.q_first
    first = cfg.n_frames - step_frames
    cache, aux = api.new_cache(dims, geom, fill=0xFF if cfg.cache_given else None)
    ws_app = torch.empty(max(16, api.append_workspace_bytes(dims, geom, step_frames * P),
                             api.append_workspace_bytes(dims, geom, P)), dtype=torch.uint8, device=dev)
    if cfg.cache_given:
        L = inp["cache_c"].shape[1]
        cache[:, :L, :cfg.d_c] = gp.to_device(inp["cache_c"])
        cache[:, :L, cfg.d_c:] = gp.to_device(inp["cache_r"])
        x_step = gp.to_device(inp["x_new"]).reshape(B, P, cfg.d_model)
    else:
        x = gp.to_device(inp["x"])
        for f in range(first):
            api.cache_append(dims, geom, x[:, f].contiguous(), gp.int_tensor([f] * B), w_dkr, cache, aux,
                             workspace=ws_app)
        x_step = x[:, first:].reshape(B, step_frames * P, cfg.d_model).contiguous()
    frame_t = gp.int_tensor([first] * B)
    q_first = gp.int_tensor([cfg.q_first] * B)
    newest = gp.int_tensor([cfg.newest] * B)
    outs = {"q_abs": torch.empty((B, cfg.n_q, H, cfg.d_qk), dtype=dt, device=dev),
            "o_lat": torch.empty((B, cfg.n_q, H, cfg.d_c), dtype=dt, device=dev),
            "lse": torch.empty((B, cfg.n_q, H), dtype=torch.float32, device=dev),
            "o_heads": torch.empty((B, cfg.n_q, H * cfg.d_v), dtype=dt, device=dev),
            "y": torch.empty((B, cfg.n_q, cfg.d_model), dtype=dt, device=dev)}
    ws_attn = torch.empty(max(16, api.attention_workspace_bytes(dims, geom, cfg.n_q)), dtype=torch.uint8,
                          device=dev)

    def step():
        api.cache_append(dims, geom, x_step, frame_t, w_dkr, cache, aux, workspace=ws_app)
        api.absorb_q(dims, geom, q_nope, q_rope, q_first, w_uk, outs["q_abs"])
        api.attention(dims, geom, outs["q_abs"], q_first, newest, cache, aux, outs["o_lat"], outs["lse"],
                      workspace=ws_attn)
        api.unabsorb_out(dims, geom, outs["o_lat"], w_uv, w_o, outs["o_heads"], outs["y"])

    step()
    torch.cuda.synchronize()
    ref = {k: _bits(v).clone() for k, v in outs.items()}
    ref["cache"] = _bits(cache).clone()
    ref["aux"] = aux.clone() if aux is not None else None
    # finite direct-call results (their parity with the oracle is tested elsewhere)
    got = {k: gp.to_host(v) for k, v in outs.items()}
    assert np.isfinite(got["o_lat"]).all() and np.isfinite(got["y"]).all()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():
            _bits(v).fill_(-1)          # eager work between replays: clobber every output
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(_bits(v), ref[k]), f"replay {rep}: {k} differs from the direct calls"
        assert torch.equal(_bits(cache), ref["cache"]), f"replay {rep}: cache differs"
        if aux is not None:
            assert torch.equal(aux, ref["aux"]), f"replay {rep}: cache scales differ"
