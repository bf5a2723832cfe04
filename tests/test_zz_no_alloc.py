"""mla_attention_noalloc (the attention call with the library's static
scratch instead of a caller workspace, for callers that cannot allocate)
against mla_attention on the same inputs, through the C-ABI: two calls in a
row, the second one smaller, then a call too large for the scratch."""
import numpy as np
import pytest

import gpu_path as gp
from mla_inputs import CONFIGS, SMALL_CONFIGS, make_workload

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _noalloc_matches(cfg, seed):
    import torch
    from head_latent_attention_cache_amd import api
    inp = make_workload(cfg, seed=seed)
    got = gp.run_gpu(cfg, inp, fill=0xFF if cfg.cache_given else None, keep_device=True)
    dev = got["_dev"]
    need = api.attention_workspace_bytes(dev["dims"], dev["geom"], cfg.n_q)
    assert 0 < need <= (64 << 20), need          # the call uses the scratch
    o_lat = torch.full_like(dev["o_lat"], 7.0)
    lse = torch.full_like(dev["lse"], 7.0)
    api.attention_noalloc(dev["dims"], dev["geom"], dev["q_abs"], dev["q_first"], dev["newest"], dev["cache"],
                          dev["aux"], o_lat, lse)
    torch.cuda.synchronize()
    # the same kernels and split plan as the workspace call: identical bits
    assert torch.equal(o_lat.view(torch.int16), dev["o_lat"].view(torch.int16))
    assert torch.equal(lse.view(torch.int32), dev["lse"].view(torch.int32))
    # and within the path's tolerance of the workspace call's values
    gp.compare("o_lat", gp.to_host(o_lat), got["o_lat"], cfg.dtype)


def test_noalloc_matches_workspace_call_twice_second_smaller(gpu_lib):
    _case("decode batch 32 x 128 heads x 4096 keys")
    _noalloc_matches(CONFIGS[2], seed=31)
    _case("decode batch 3 x 128 heads x 300 keys (after the larger call)")
    _noalloc_matches(SMALL_CONFIGS[2], seed=32)
    _case("video chunk small (after both)")
    _noalloc_matches(SMALL_CONFIGS[3], seed=33)
    _case("INT4 video chunk small: the packed cache dequantised into the scratch too")
    _noalloc_matches(SMALL_CONFIGS[5], seed=34)
    _case("long video small (d_r 512, wide-row kernel, split partials in the scratch)")
    _noalloc_matches(SMALL_CONFIGS[4], seed=35)


def test_noalloc_rejects_a_call_beyond_the_scratch(gpu_lib):
    import torch
    from head_latent_attention_cache_amd import api
    from head_latent_attention_cache_amd._lib import MLA_ERR_WORKSPACE, MLAError
    cfg = CONFIGS[3]
    _case(f"{cfg.name}: partials beyond the static scratch")
    dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
    assert api.attention_workspace_bytes(dims, geom, cfg.n_q) > (64 << 20)
    B, H = cfg.batch, cfg.n_heads
    cache, aux = api.new_cache(dims, geom)
    q_abs = torch.zeros((B, cfg.n_q, H, cfg.d_qk), dtype=torch.bfloat16, device="cuda")
    o_lat = torch.full((B, cfg.n_q, H, cfg.d_c), 3.0, dtype=torch.bfloat16, device="cuda")
    idx = gp.int_tensor([cfg.q_first] * B)
    with pytest.raises(MLAError) as ei:
        api.attention_noalloc(dims, geom, q_abs, idx, gp.int_tensor([cfg.newest] * B), cache, aux, o_lat)
    assert ei.value.status == MLA_ERR_WORKSPACE and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool(torch.all(o_lat == 3.0))          # nothing was launched
