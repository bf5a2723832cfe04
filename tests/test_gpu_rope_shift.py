"""Re-rotation of cached rotary keys (mla_cache_rope_shift) against the
oracle's definition, applied to the oracle's own stored cache (uploaded) so
that only the shift's arithmetic is compared; untouched columns and slots bit for bit; a zero
shift leaves every byte; attention is unchanged when the keys and the query
move by the same time shift.  Every call goes through the C-ABI."""
import numpy as np
import pytest

import gpu_path as gp
import oracle.int4 as oi
import oracle.mla as om
from mla_inputs import SMALL_CONFIGS, make_workload

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _snapshot(cfg, dev):
    import torch
    return dev["cache"].view(torch.uint8).clone(), (dev["aux"].clone() if dev["aux"] is not None else None)


# (workload key, slot_begin, n_slots or None for "to the end", per-sequence shifts)
CASES = [(1, 0, None, [[3, -1, 2]]),                       # fp32, 3D, every slot
         (3, 5, 37, [[-4, 2, -3]]),                        # bf16, 3D, a ragged range
         (2, 0, None, [[7, 0, 0], [0, 0, 0], [-300, 5, 5]]),   # bf16, 1D, one zero shift
         (5, 17, 100, [[2, 1, 0]]),                        # INT4
         (6, 0, None, [[1, -2, 3]])]                       # INT2


@pytest.mark.parametrize("key,begin,count,delta", CASES)
def test_shift_matches_oracle(gpu_lib, key, begin, count, delta):
    import torch
    from head_latent_attention_cache_amd import api
    cfg = SMALL_CONFIGS[key]
    count = cfg.capacity - begin if count is None else count
    delta = np.array(delta, np.int64)[:cfg.batch]
    _case(f"rope shift {cfg.name} slots [{begin}, {begin + count}) delta {delta.tolist()}")
    inp = make_workload(cfg, seed=21)
    st = om.build_cache(cfg, inp)
    dev = gp.upload_oracle_cache(cfg, st)
    before, aux_before = _snapshot(cfg, dev)
    written = om.slot_frames(cfg, cfg.newest) >= 0
    api.cache_rope_shift(dev["dims"], dev["geom"], gp.int_tensor(delta.reshape(-1)), begin, count,
                         dev["cache"], dev["aux"])
    torch.cuda.synchronize()
    om.rope_shift(st, cfg, delta, begin, count)
    after = dev["cache"].view(torch.uint8)
    rng_mask = np.zeros(cfg.capacity, bool)
    rng_mask[begin:begin + count] = True
    # slots outside the range: every byte unchanged
    b_out = torch.from_numpy(~rng_mask).to(after.device)
    assert torch.equal(after[:, b_out], before[:, b_out])
    # sequences with a zero shift: every byte unchanged
    for b in range(cfg.batch):
        if not np.any(delta[b, :cfg.rope_dims]):
            assert torch.equal(after[b], before[b])
    sel = rng_mask & written
    if cfg.cache_fmt in ("int4", "int2"):
        nb = cfg.d_c * om.content_bits(cfg) // 8
        assert torch.equal(after[..., :nb], before[..., :nb]), "content codes changed"
        codes = after.cpu().numpy()
        ng = cfg.d_c // 32
        aux = dev["aux"].cpu().numpy()
        cscale = aux[:cfg.batch * cfg.capacity * ng].reshape(cfg.batch, cfg.capacity, ng)
        rscale = aux[cfg.batch * cfg.capacity * ng:].reshape(cfg.batch, cfg.capacity)
        same = gp.check_lowbit_codes(cfg, codes, cscale, rscale, st, sel)
        print(f"rotary code bytes equal to the oracle's: {same:.5f}", flush=True)
        out = torch.empty((cfg.batch, cfg.capacity, cfg.d_qk), dtype=torch.float32, device="cuda")
        api.cache_dequant(dev["dims"], dev["geom"], dev["cache"], dev["aux"], out)
        torch.cuda.synchronize()
        vals = out.cpu().numpy().astype(np.float64)
        assert torch.equal(dev["aux"][:cfg.batch * cfg.capacity * ng], aux_before[:cfg.batch * cfg.capacity * ng])
    else:
        vals = gp.to_host(dev["cache"])
        elem = 2 if cfg.dtype == "bf16" else 4
        assert torch.equal(after[..., :cfg.d_c * elem], before[..., :cfg.d_c * elem]), "content changed"
        if cfg.dtype == "bf16":
            # every rotated key is one of the two bf16 values next to the
            # oracle's unrounded rotation (float32 sin / cos of an fp64-reduced
            # angle err by far less than half a bf16 step of the pair's norm)
            pre = st["pre"][:, sel, cfg.d_c:]
            pair = np.sqrt(pre[..., 0::2] ** 2 + pre[..., 1::2] ** 2)
            err = np.repeat(pair, 2, axis=-1) * 2.0 ** -20
            lo, _ = om.bf16_bracket(pre - err)
            _, hi = om.bf16_bracket(pre + err)
            v = vals[:, sel, cfg.d_c:]
            outside = (v < lo) | (v > hi)
            assert not outside.any(), f"{int(outside.sum())} rotated keys outside their bf16 bracket"
    gp.compare("rotary keys", vals[:, sel, cfg.d_c:], st["values"][:, sel, cfg.d_c:], cfg.dtype)


@pytest.mark.parametrize("key", [2, 3, 5, 6])
def test_zero_shift_leaves_every_byte(gpu_lib, key):
    import torch
    from head_latent_attention_cache_amd import api
    cfg = SMALL_CONFIGS[key]
    _case(f"zero shift {cfg.name}")
    got = gp.run_gpu(cfg, make_workload(cfg, seed=22), fill=0xFF if cfg.cache_given else None, keep_device=True)
    dev = got["_dev"]
    before, aux_before = _snapshot(cfg, dev)
    d = np.zeros((cfg.batch, 3), np.int64)
    if cfg.rope_dims == 1:
        d[:, 1:] = 5        # ignored by a 1D embedding
    api.cache_rope_shift(dev["dims"], dev["geom"], gp.int_tensor(d.reshape(-1)), 0, cfg.capacity,
                         dev["cache"], dev["aux"])
    torch.cuda.synchronize()
    assert torch.equal(dev["cache"].view(torch.uint8), before)
    if aux_before is not None:
        assert torch.equal(dev["aux"], aux_before)


@pytest.mark.parametrize("key,shift", [(3, 5), (2, -1000), (1, 2)])
def test_attention_invariant_under_common_shift(gpu_lib, key, shift):
    """Keys moved by `shift` frames (1D: positions) and queries absorbed
    `shift` further along give the attention of the unshifted cache."""
    import torch
    from head_latent_attention_cache_amd import api
    cfg = SMALL_CONFIGS[key]
    _case(f"shift invariance {cfg.name} by {shift}")
    inp = make_workload(cfg, seed=23)
    got = gp.run_gpu(cfg, inp, fill=0xFF if cfg.cache_given else None, keep_device=True)
    dev = got["_dev"]
    B = cfg.batch
    api.cache_rope_shift(dev["dims"], dev["geom"], gp.int_tensor([shift, 0, 0] * B), 0, cfg.capacity,
                         dev["cache"], dev["aux"])
    q_abs = torch.empty_like(dev["q_abs"])
    # rotary positions of the queries moved by the same shift (1D: P = 1, so
    # a frame shift is a position shift)
    api.absorb_q(dev["dims"], dev["geom"], gp.to_device(inp["q_nope"]), gp.to_device(inp["q_rope"]),
                 gp.int_tensor([cfg.q_first + shift] * B), gp.to_device(inp["w_uk"]), q_abs)
    o_lat = torch.empty_like(dev["o_lat"])
    lse = torch.empty_like(dev["lse"])
    api.attention(dev["dims"], dev["geom"], q_abs, dev["q_first"], dev["newest"], dev["cache"], dev["aux"],
                  o_lat, lse)
    torch.cuda.synchronize()
    gp.compare("o_lat", gp.to_host(o_lat), got["o_lat"], cfg.dtype)
    gp.compare("lse", gp.to_host(lse), got["lse"], cfg.dtype)
