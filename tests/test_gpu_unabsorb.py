"""Un-absorb with at most 32 rows and long head concatenations (K = H * d_v
>= 4096, the decode output projection's regime), including ragged tails in
M, N and K, against the oracle's definition."""
import numpy as np
import pytest

import gpu_path as gp
import oracle.mla as om
from mla_inputs.generate import bf16_bits_from_f32, bf16_bits_to_f32

pytestmark = pytest.mark.gpu

# (rows M, heads H, d_v, d_c, d_model)
SHAPES = [(5, 41, 104, 64, 1000),      # K = 4264 (K % 64 = 40), N % 64 = 40, M < 32
          (32, 32, 128, 512, 4096),    # K = N = 4096, full tiles
          (17, 64, 72, 128, 200),      # K = 4608, N = 200 (3 blocks + tail)
          (5, 64, 128, 64, 8232),      # K = 8192, N = 8232 (ragged last column block)
          (32, 128, 128, 64, 16384)]   # the decode output projection's shape (K = N = 16384)


def _inputs(M, H, d_v, d_c, d_model, seed):
    rng = np.random.default_rng(seed)
    o_lat = bf16_bits_from_f32(rng.standard_normal((M, 1, H, d_c)).astype(np.float32))
    w_uv = bf16_bits_from_f32((rng.standard_normal((H, d_v, d_c)) / np.sqrt(d_c)).astype(np.float32))
    w_o = bf16_bits_from_f32((rng.standard_normal((d_model, H * d_v)) / np.sqrt(H * d_v)).astype(np.float32))
    return o_lat, w_uv, w_o


def _run(M, H, d_v, d_c, d_model, seed=0):
    import torch
    from head_latent_attention_cache_amd import api
    dims = api.make_dims(H, d_model, 32, d_v, d_c, 16, 1, [16])
    geom = api.make_geom(M, 1, 1, 16)
    o_lat, w_uv, w_o = _inputs(M, H, d_v, d_c, d_model, seed)
    o_heads = torch.empty((M, 1, H * d_v), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, 1, d_model), dtype=torch.bfloat16, device="cuda")
    api.unabsorb_out(dims, geom, gp.to_device(o_lat), gp.to_device(w_uv), gp.to_device(w_o), o_heads, y)
    torch.cuda.synchronize()
    return gp.to_host(o_heads), gp.to_host(y), (o_lat, w_uv, w_o)


@pytest.mark.parametrize("shape", SHAPES)
def test_unabsorb_streaming_shapes(gpu_lib, shape):
    M, H, d_v, d_c, d_model = shape
    print(f"[case] unabsorb M={M} H={H} d_v={d_v} d_c={d_c} d_model={d_model}", flush=True)
    o_heads, y, (o_lat, w_uv, w_o) = _run(*shape)
    ref_heads, ref_y = om.unabsorb(bf16_bits_to_f32(o_lat), bf16_bits_to_f32(w_uv), bf16_bits_to_f32(w_o))
    gp.compare("o_heads", o_heads, ref_heads.reshape(M, 1, H * d_v), "bf16")
    gp.compare("y", y, ref_y.reshape(M, 1, d_model), "bf16")

