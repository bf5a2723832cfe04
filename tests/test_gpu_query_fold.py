"""Load-time fold of the query and key up-projections and the folded
absorbed query, through the C-ABI, against the oracle: the folded weight, the
absorbed queries, and attention driven by them against the materialised-head
definition with q_nope = W^UQ c_q; sampled heads at the full decode shape."""
import numpy as np
import pytest

import gpu_path as gp
import oracle.mla as om
from mla_inputs import CONFIGS, SMALL_CONFIGS, make_workload

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _fold_gpu(cfg, inp):
    import torch
    from head_latent_attention_cache_amd import api
    dims = api.dims_from_config(cfg)
    w_fold = torch.empty((cfg.n_heads, cfg.d_c, cfg.d_cq), dtype=api.torch_dtype(dims), device="cuda")
    api.fold_query_weights(dims, gp.to_device(inp["w_uq"]), gp.to_device(inp["w_uk"]), w_fold)
    return w_fold


@pytest.mark.parametrize("key", [1, 2, 3])
def test_fold_and_folded_absorb_match_oracle(gpu_lib, key):
    import torch
    from head_latent_attention_cache_amd import api
    cfg = SMALL_CONFIGS[key]
    _case(f"fold {cfg.name} d_cq {cfg.d_cq}")
    inp = make_workload(cfg, seed=31, parts=("w_uq", "w_uk", "c_q", "q_rope"))
    w_fold = _fold_gpu(cfg, inp)
    torch.cuda.synchronize()
    ref_fold = om.fold_query_weights(cfg, om.as_f64(inp["w_uq"]), om.as_f64(inp["w_uk"]))
    gp.compare("w_fold", gp.to_host(w_fold), ref_fold, cfg.dtype)
    dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
    B, H = cfg.batch, cfg.n_heads
    q_abs = torch.empty((B, cfg.n_q, H, cfg.d_qk), dtype=api.torch_dtype(dims), device="cuda")
    api.absorb_q_folded(dims, geom, gp.to_device(inp["c_q"]), gp.to_device(inp["q_rope"]),
                        gp.int_tensor([cfg.q_first] * B), w_fold, q_abs)
    torch.cuda.synchronize()
    ref = om.absorb_query_folded(cfg, om.as_f64(inp["c_q"]), om.as_f64(inp["q_rope"]), ref_fold, cfg.q_first)
    gp.compare("q_abs", gp.to_host(q_abs), ref, cfg.dtype)


@pytest.mark.parametrize("key", [2, 3])
def test_folded_query_attention_end_to_end(gpu_lib, key):
    """Attention on the path's cache with folded queries against the oracle's
    materialised heads with q_nope = W^UQ c_q."""
    import torch
    from head_latent_attention_cache_amd import api
    cfg = SMALL_CONFIGS[key]
    _case(f"folded attention {cfg.name}")
    inp = make_workload(cfg, seed=32)
    inp.update(make_workload(cfg, seed=32, parts=("w_uq", "c_q")))
    got = gp.run_gpu(cfg, inp, fill=0xFF if cfg.cache_given else None, keep_device=True)
    dev = got["_dev"]
    w_fold = _fold_gpu(cfg, inp)
    q_abs = torch.empty_like(dev["q_abs"])
    api.absorb_q_folded(dev["dims"], dev["geom"], gp.to_device(inp["c_q"]), gp.to_device(inp["q_rope"]),
                        dev["q_first"], w_fold, q_abs)
    o_lat = torch.empty_like(dev["o_lat"])
    lse = torch.empty_like(dev["lse"])
    api.attention(dev["dims"], dev["geom"], q_abs, dev["q_first"], dev["newest"], dev["cache"], dev["aux"],
                  o_lat, lse)
    torch.cuda.synchronize()
    q_nope = om.query_up(cfg, om.as_f64(inp["c_q"]), om.as_f64(inp["w_uq"]))
    st = om.build_cache(cfg, inp)
    q_rot = om.absorb_query(cfg, np.zeros_like(q_nope), om.as_f64(inp["q_rope"]), om.as_f64(inp["w_uk"]),
                            cfg.q_first)[..., cfg.d_c:]
    _, ref_o, ref_l = om.attend(cfg, st, q_nope, q_rot, om.as_f64(inp["w_uk"]), om.as_f64(inp["w_uv"]),
                                cfg.q_first)
    B, n_q, H = cfg.batch, cfg.n_q, cfg.n_heads
    gp.compare("o_lat", gp.to_host(o_lat), ref_o.reshape(B, n_q, H, cfg.d_c), cfg.dtype)
    gp.compare("lse", gp.to_host(lse), ref_l.reshape(B, n_q, H), cfg.dtype)


def test_fold_full_decode_shape_sampled(gpu_lib):
    """128 heads, d_c 512, d_nope 128, d_cq 1536: sampled heads of the fold and
    of the absorbed queries of the 32 sequences."""
    import torch
    from head_latent_attention_cache_amd import api
    cfg = CONFIGS[2]
    _case(f"fold {cfg.name} d_cq {cfg.d_cq}")
    inp = make_workload(cfg, seed=33, parts=("w_uq", "w_uk", "c_q", "q_rope"))
    w_fold = _fold_gpu(cfg, inp)
    dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
    B, H = cfg.batch, cfg.n_heads
    q_abs = torch.empty((B, cfg.n_q, H, cfg.d_qk), dtype=torch.bfloat16, device="cuda")
    api.absorb_q_folded(dims, geom, gp.to_device(inp["c_q"]), gp.to_device(inp["q_rope"]),
                        gp.int_tensor([cfg.q_first] * B), w_fold, q_abs)
    torch.cuda.synchronize()
    heads = [0, 77, 127]
    wq = om.as_f64(inp["w_uq"]).reshape(H, cfg.d_nope, cfg.d_cq)
    wk = om.as_f64(inp["w_uk"])
    got_fold = gp.to_host(w_fold[heads])
    got_q = gp.to_host(q_abs)
    cq = om.as_f64(inp["c_q"])
    for i, h in enumerate(heads):
        ref = wk[h] @ wq[h]
        gp.compare(f"w_fold[{h}]", got_fold[i], ref, "bf16")
        gp.compare(f"q_lat[:, :, {h}]", got_q[:, :, h, :cfg.d_c], np.einsum("btj,cj->btc", cq, ref), "bf16")
