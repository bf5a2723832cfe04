"""The fixed-reference softmax of the MFMA attention kernels and its rerun.

Both MFMA kernels exponentiate scores against a fixed per-row reference (the
maximum of the row's first visible key tile) and never rescale their output
accumulators; when a later tile's maximum exceeds the reference by more than
a threshold (64 log2 units), the work-group discards its accumulators and runs
the key loop again with the final maxima as references.

Two kinds of cases, each in a child process with the kernel overrides in its
environment (the library reads them once):

* threshold 0 (MLA_SOFTMAX_RERUN_SLACK=0): every row whose maximum is not in
  its first visible tile reruns, so every kernel variant (dense, INT4, INT2,
  d_r = 512, QK normalisation) takes the second pass on ordinary inputs;
* planted keys: cache rows aligned with one (token, head) query so that
  its score is ~52 nats, more than the 44.4 nats (64 log2 units) above the
  first tile's maximum, placed in a later tile of a split (the rerun fires on
  its own) or in the first visible tile (no rerun, a large spread).

Planted cases attend over a cache written by the oracle (copied to the
device) with the oracle's absorbed queries rounded to bf16, so both sides
see identical operands; the expected values come from the oracle's textbook
masked softmax over those rows (the absorbed form, pinned against the
materialised heads by the oracle's own tests).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SLACK_CHILD = r'''
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {here!r})
import gpu_path as gp
import oracle.mla as om
from mla_inputs import SMALL_CONFIGS, make_workload
cfg = SMALL_CONFIGS[{key}]
B, n_q, H = cfg.batch, cfg.n_q, cfg.n_heads
if {qkn}:
    import test_gpu_qk_norm as tq
    cfg = cfg.replace(qk_norm=True, qk_eps=tq.EPS)
    inp = make_workload(cfg, seed=21)
    g_q, g_k = tq._weights(cfg, 22)
    got = tq.run_qkn(cfg, inp, g_q, g_k, fill=0xFF if cfg.cache_given else None)
    st = om.build_cache(cfg, inp)
    w_uk, w_uv = om.as_f64(inp["w_uk"]), om.as_f64(inp["w_uv"])
    q_nope = om.as_f64(inp["q_nope"])
    q_rot = om.absorb_query(cfg, q_nope, om.as_f64(inp["q_rope"]), w_uk, cfg.q_first)[..., cfg.d_c:]
    _, o_lat, lse = om.attend_qk_norm(cfg, st, q_nope, q_rot, w_uk, w_uv, om.as_f64(g_q), om.as_f64(g_k),
                                      tq.EPS, cfg.q_first)
else:
    inp = make_workload(cfg, seed=21)
    got = gp.run_gpu(cfg, inp, fill=0xFF if cfg.cache_given else None)
    ref = om.run(cfg, inp)
    o_lat, lse = ref["o_lat"], ref["lse"]
gp.compare("o_lat", got["o_lat"], o_lat.reshape(B, n_q, H, cfg.d_c), cfg.dtype)
gp.compare("lse", got["lse"], lse.reshape(B, n_q, H), cfg.dtype)
print("child ok", flush=True)
'''

PLANT_CHILD = r'''
import sys
import numpy as np
sys.path.insert(0, {root!r}); sys.path.insert(0, {here!r})
import torch
import gpu_path as gp
import oracle.int4 as oi
import oracle.mla as om
from mla_inputs import SMALL_CONFIGS, make_workload, bf16_bits_from_f32
import head_latent_attention_cache_amd as mla
from head_latent_attention_cache_amd import api
mla.load()
cfg = SMALL_CONFIGS[{key}]
plants = {plants!r}          # (b, slot, query token, head, score in nats)
B, n_q, H, DC = cfg.batch, cfg.n_q, cfg.n_heads, cfg.d_c
inp = make_workload(cfg, seed=23)
st = om.build_cache(cfg, inp)
w_uk = om.as_f64(inp["w_uk"])
q_abs = om.round_bf16(om.absorb_query(cfg, om.as_f64(inp["q_nope"]), om.as_f64(inp["q_rope"]), w_uk,
                                      cfg.q_first))
scale = om.softmax_scale(cfg)
lowbit = cfg.cache_fmt in ("int4", "int2")
for b, s, t, h, score in plants:
    q = q_abs[b, t, h]
    row = om.round_to_storage(q * (score / (scale * float(q @ q))), cfg.dtype)
    if lowbit:
        qz = oi.quantize_cache_rows(row[None], DC, 32, om.content_bits(cfg))
        st["codes"][b, s] = qz["codes"][0]
        st["cscale"][b, s] = qz["cscale"][0]
        st["rscale"][b, s] = qz["rscale"][0]
        row = qz["values"][0]
    st["values"][b, s] = row
dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
cache, aux = api.new_cache(dims, geom)
if lowbit:
    cache.copy_(torch.from_numpy(st["codes"]))
    aux.copy_(torch.from_numpy(np.concatenate([st["cscale"].reshape(-1), st["rscale"].reshape(-1)])))
else:
    cache.copy_(gp.to_device(bf16_bits_from_f32(st["values"].astype(np.float32))))
o_lat = torch.empty((B, n_q, H, DC), dtype=torch.bfloat16, device="cuda")
lse = torch.empty((B, n_q, H), dtype=torch.float32, device="cuda")
api.attention(dims, geom, gp.to_device(bf16_bits_from_f32(q_abs.astype(np.float32))),
              gp.int_tensor([cfg.q_first] * B), gp.int_tensor([cfg.newest] * B), cache, aux, o_lat, lse)
torch.cuda.synchronize()
# the oracle's textbook masked softmax over the same rows and queries
mask = om.mask_matrix(cfg, cfg.q_first, st["newest"])
ref_o = np.zeros((B, n_q, H, DC))
ref_l = np.zeros((B, n_q, H))
for b in range(B):
    K = st["values"][b]
    for h in range(H):
        o, _, l = om.attention_core(q_abs[b, :, h], K, K[:, :DC], mask, scale)
        ref_o[b, :, h] = o
        ref_l[b, :, h] = l
planted = {{(b, s) for b, s, _, _, _ in plants}}
for b, s, t, h, score in plants:
    assert mask[t, s], ("planted key not visible", b, s, t)
    # the planted key outscores every other visible key of its row by more
    # than 64 log2 units (44.4 nats): a split whose first tile does not hold
    # it reruns
    sc = scale * (st["values"][b] @ q_abs[b, t, h])
    others = [sc[k] for k in np.flatnonzero(mask[t]) if (b, k) not in planted]
    assert sc[s] - max(others) > 64.0 / np.log2(np.e) + 0.5, ("planted score too small", sc[s], max(others))
gp.compare("o_lat", gp.to_host(o_lat), ref_o, "bf16")
gp.compare("lse", gp.to_host(lse), ref_l, "bf16")
print("child ok", flush=True)
'''


def _child(code, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    print(f"[case] env {env_extra}", flush=True)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


# every small workload family: narrow MFMA kernel (decode, chunk, INT4, INT2),
# wide-row kernel (d_r = 512); with and without QK normalisation; one split and
# two splits (partials merged)
@pytest.mark.parametrize("key", [2, 3, 4, 5, 6])
@pytest.mark.parametrize("qkn", [False, True])
@pytest.mark.parametrize("splits", [1, 2])
def test_rerun_pass_on_every_row(gpu_lib, key, qkn, splits):
    code = SLACK_CHILD.format(root=ROOT, here=HERE, key=key, qkn=qkn)
    _child(code, {"MLA_SOFTMAX_RERUN_SLACK": "0", "MLA_ATTN_SPLITS": str(splits)})


# (workload, plants, splits): keys in a later tile of a split (the rerun fires
# by itself), two of them close in score so the second pass mixes their
# values; and keys in the first visible tile (no rerun, large spread)
PLANTS = [
    # decode, 10 tiles, two splits of 5: slots 150 (tile 4) and 290 (tile 9)
    (2, [(0, 150, 0, 5, 52.0), (0, 290, 0, 5, 51.5), (2, 100, 0, 77, 52.0)], 2),
    # decode: the planted key in the first tile of each split
    (2, [(1, 3, 0, 9, 52.0), (1, 165, 0, 100, 52.0)], 2),
    # video chunk, 5 tiles, two splits (tiles 0-2, 3-4): slots 90, 138 and 139
    (3, [(0, 90, 7, 3, 52.0), (0, 139, 7, 3, 51.5), (0, 138, 30, 31, 52.0)], 2),
    (3, [(0, 10, 7, 3, 52.0)], 1),
    # long video (d_r = 512, wide-row kernel), 3 tiles: slots 70 and 89 for a
    # token of the last query frame; slot 20 (frame 7) for the middle frame
    (4, [(0, 70, 40, 2, 52.0), (0, 89, 40, 2, 51.5), (1, 89, 20, 7, 52.0), (1, 20, 20, 0, 52.0)], 1),
    (4, [(0, 5, 40, 2, 52.0)], 1),
    # INT4 and INT2 caches, 5 tiles (the last one ragged)
    (5, [(0, 100, 11, 4, 52.0), (0, 143, 11, 4, 51.5)], 1),
    # (the 2-bit content codes keep only the sign pattern of the planted row:
    # larger targets keep its score above the margin)
    (6, [(0, 100, 11, 4, 58.0), (0, 143, 11, 4, 57.5)], 1),
    (6, [(0, 2, 11, 4, 58.0)], 2),
]


@pytest.mark.parametrize("key,plants,splits", PLANTS)
def test_planted_outlier_keys(gpu_lib, key, plants, splits):
    code = PLANT_CHILD.format(root=ROOT, here=HERE, key=key, plants=plants)
    _child(code, {"MLA_ATTN_SPLITS": str(splits)})
