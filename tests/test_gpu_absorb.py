"""The absorbed query (mla_absorb_q) against the oracle on shapes of the
decode-time path, where the content product and the rotary half share one
launch (bf16, at most 32 query rows): several query tokens per sequence,
a different first position per sequence, 1D and 3D rotary coordinates, and
exactly 32 rows; plus a 40-row shape that takes the two-launch path.  Every
call goes through the C-ABI."""
import numpy as np
import pytest

import gpu_path as gp
import oracle.mla as om
from mla_inputs import SMALL_CONFIGS
from mla_inputs.generate import bf16_bits_from_f32, bf16_bits_to_f32

pytestmark = pytest.mark.gpu

# (name, base workload, batch, query frames, grid (h, w), per-sequence first frame)
CASES = [("1d_b3_q5", 2, 3, 5, (1, 1), [0, 7, 300]),
         ("3d_b2_2frames", 3, 2, 2, (2, 3), [3, 5]),
         ("1d_b4_q8_32rows", 2, 4, 8, (1, 1), [11, 0, 250, 64]),
         ("1d_b5_q8_40rows", 2, 5, 8, (1, 1), [1, 2, 3, 4, 5])]


@pytest.mark.parametrize("name,key,B,qf,grid,firsts", CASES)
def test_absorb_matches_oracle(gpu_lib, name, key, B, qf, grid, firsts):
    import torch
    from head_latent_attention_cache_amd import api
    base = SMALL_CONFIGS[key]
    cfg = base.replace(name=f"absorb_{name}", batch=B, n_heads=8, grid_h=grid[0], grid_w=grid[1],
                       window=max(firsts) + qf, n_frames=max(firsts) + qf, q_first=0, q_frames=qf)
    n_q, H = cfg.n_q, cfg.n_heads
    print(f"[case] absorb {cfg.name} rows {B * n_q}", flush=True)
    rng = np.random.default_rng(77)
    q_nope = bf16_bits_from_f32(rng.standard_normal((B, n_q, H, cfg.d_nope)).astype(np.float32))
    q_rope = bf16_bits_from_f32(rng.standard_normal((B, n_q, H, cfg.d_r)).astype(np.float32))
    w_uk = bf16_bits_from_f32((rng.standard_normal((H, cfg.d_c, cfg.d_nope)) / np.sqrt(cfg.d_nope)).astype(np.float32))
    dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
    q_abs = torch.empty((B, n_q, H, cfg.d_qk), dtype=torch.bfloat16, device="cuda")
    api.absorb_q(dims, geom, gp.to_device(q_nope), gp.to_device(q_rope), gp.int_tensor(firsts),
                 gp.to_device(w_uk), q_abs)
    torch.cuda.synchronize()
    got = gp.to_host(q_abs)
    ref = np.concatenate([om.absorb_query(cfg, bf16_bits_to_f32(q_nope[b:b + 1]), bf16_bits_to_f32(q_rope[b:b + 1]),
                                          bf16_bits_to_f32(w_uk), firsts[b]) for b in range(B)])
    gp.compare("q_abs", got, ref, "bf16")
