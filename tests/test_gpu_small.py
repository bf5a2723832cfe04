"""HIP path vs the CPU oracle on reduced workloads (whole outputs), plus the
bit-exact checks of cache indexing, masking and low-bit (INT4, INT2) storage.

Every call goes through the C-ABI (via the ctypes binding)."""
import numpy as np
import pytest

import gpu_path as gp
import oracle.int4 as oi
import oracle.mla as om
from mla_inputs import SMALL_CONFIGS, make_workload

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _check_all(cfg, got, ref, report=None):
    st = ref["cache"]
    written = om.slot_frames(cfg, st["newest"]) >= 0
    if cfg.cache_fmt in ("int4", "int2"):
        # codes may differ by one step where the two paths' bf16 cache values differ
        import torch
        from head_latent_attention_cache_amd import api
        dev = got["_dev"]
        out = torch.empty((cfg.batch, cfg.capacity, cfg.d_qk), dtype=torch.float32, device="cuda")
        api.cache_dequant(dev["dims"], dev["geom"], dev["cache"], dev["aux"], out)
        gp.compare("cache", gp.to_host(out)[:, written], st["values"][:, written], cfg.dtype, report)
        same = gp.check_lowbit_codes(cfg, got["codes"], got["cscale"], got["rscale"], st, written)
        print(f"low-bit code bytes equal to the oracle's: {same:.5f}", flush=True)
    else:
        gp.compare("cache", got["cache"][:, written], st["values"][:, written], cfg.dtype, report)
    B, n_q, H = cfg.batch, cfg.n_q, cfg.n_heads
    gp.compare("q_abs", got["q_abs"], ref["q_abs"], cfg.dtype, report)
    gp.compare("o_lat", got["o_lat"], ref["o_lat"].reshape(B, n_q, H, cfg.d_c), cfg.dtype, report)
    gp.compare("lse", got["lse"], ref["lse"].reshape(B, n_q, H), cfg.dtype, report)
    gp.compare("o_heads", got["o_heads"], ref["o_heads"].reshape(B, n_q, H, cfg.d_v), cfg.dtype, report)
    gp.compare("y", got["y"], ref["y"].reshape(B, n_q, cfg.d_model), cfg.dtype, report)


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5, 6])
def test_small_workload_end_to_end(gpu_lib, key):
    cfg = SMALL_CONFIGS[key]
    _case(cfg.name)
    inp = make_workload(cfg, seed=0)
    got = gp.run_gpu(cfg, inp, fill=0xFF if cfg.cache_given else None, keep_device=True)
    ref = om.run(cfg, inp)
    rep = {}
    _check_all(cfg, got, ref, rep)
    print({k: (f"{a:.2e}", f"{b:.2e}") for k, (a, b) in rep.items()}, flush=True)


@pytest.mark.parametrize("key", [3, 4])
def test_partially_filled_ring_with_poisoned_slots(gpu_lib, key):
    # video chunk: 2 of 4 ring frames written; long video (wide-row kernel,
    # whose rotary keys go straight from the cache into registers): 4 of 6;
    # the rest hold NaN bit patterns
    base = SMALL_CONFIGS[key]
    cfg = base.replace(name=f"ring_partial_{base.name}", n_frames=base.q_frames + 1, q_first=1)
    assert om.slot_frames(cfg, cfg.newest).min() < 0
    _case(cfg.name)
    inp = make_workload(cfg, seed=1)
    got = gp.run_gpu(cfg, inp, fill=0xFF, keep_device=True)
    _check_all(cfg, got, om.run(cfg, inp))


@pytest.mark.parametrize("key", [5, 6])
def test_lowbit_partially_filled_ring_with_poisoned_slots(gpu_lib, key):
    # packed codes and scales of the unwritten slots are 0xFF bytes (NaN scales)
    cfg = SMALL_CONFIGS[key].replace(name=f"{SMALL_CONFIGS[key].cache_fmt}_ring_partial", n_frames=2, q_first=1)
    _case(cfg.name)
    inp = make_workload(cfg, seed=12)
    got = gp.run_gpu(cfg, inp, fill=0xFF, keep_device=True)
    ref = om.run(cfg, inp)
    _check_all(cfg, got, ref)


@pytest.mark.parametrize("key", [5, 6])
def test_lowbit_capacity_not_multiple_of_8(gpu_lib, key):
    # 35-token frames: capacity 140 takes the generic kernel's low-bit path
    cfg = SMALL_CONFIGS[key].replace(name=f"{SMALL_CONFIGS[key].cache_fmt}_cap140", grid_h=5, grid_w=7)
    _case(cfg.name)
    inp = make_workload(cfg, seed=13)
    got = gp.run_gpu(cfg, inp, keep_device=True)
    ref = om.run(cfg, inp)
    _check_all(cfg, got, ref)


def test_block_causal_two_frames_per_block(gpu_lib):
    cfg = SMALL_CONFIGS[4].replace(name="block2", frames_per_block=2, window=5, n_frames=8, q_first=5)
    _case(cfg.name)
    inp = make_workload(cfg, seed=2)
    got = gp.run_gpu(cfg, inp, keep_device=True)
    _check_all(cfg, got, om.run(cfg, inp))


def _one_hot_inputs(cfg, seed=4):
    inp = make_workload(cfg, seed=seed)
    B, F, P, D = cfg.batch, cfg.n_frames, cfg.tokens_per_frame, cfg.d_model
    x = np.zeros((B, F, P, D), np.float32)
    k = (np.arange(B * F * P) * 7) % D
    x.reshape(-1, D)[np.arange(B * F * P), k] = 1.0
    if cfg.dtype == "bf16":
        from mla_inputs import bf16_bits_from_f32
        x = bf16_bits_from_f32(x)
    inp["x"] = x
    return inp


@pytest.mark.parametrize("key", [3, 4])
def test_slot_indexing_bitexact(gpu_lib, key):
    # one-hot hidden states make every content latent an exact column of the
    # projection, so each slot's content identifies the (frame, token) it holds
    cfg = SMALL_CONFIGS[key]
    _case(f"slots {cfg.name}")
    inp = _one_hot_inputs(cfg)
    got = gp.run_gpu(cfg, inp)
    st = om.build_cache(cfg, inp)
    written = om.slot_frames(cfg, st["newest"]) >= 0
    assert np.array_equal(got["cache"][:, written, :cfg.d_c], st["values"][:, written, :cfg.d_c])


@pytest.mark.parametrize("key", [5, 6])
def test_lowbit_quantiser_bitexact(gpu_lib, key):
    cfg = SMALL_CONFIGS[key].replace(name=f"{SMALL_CONFIGS[key].cache_fmt}_nowrap", n_frames=4, q_first=3)
    _case(cfg.name)
    inp = _one_hot_inputs(cfg)
    got = gp.run_gpu(cfg, inp)
    st = om.build_cache(cfg, inp)
    ncb = cfg.d_c * om.content_bits(cfg) // 8          # content code bytes per row
    assert np.array_equal(got["codes"][..., :ncb], st["codes"][..., :ncb])
    assert np.array_equal(got["cscale"].view(np.uint16), st["cscale"].view(np.uint16))
    # rotary part at coordinate (0, 0, 0): rotation by zero is exact on both sides
    slot0 = int(om.slot_index(cfg, 0, 0))
    assert np.array_equal(got["codes"][:, slot0, ncb:], st["codes"][:, slot0, ncb:])
    assert np.array_equal(got["rscale"][:, slot0].view(np.uint16), st["rscale"][:, slot0].view(np.uint16))
    written = om.slot_frames(cfg, st["newest"]) >= 0
    gp.check_lowbit_codes(cfg, got["codes"], got["cscale"], got["rscale"], st, written)


@pytest.mark.parametrize("key", [5, 6])
def test_lowbit_unpack_bitexact_and_attention_on_oracle_cache(gpu_lib, key):
    # the oracle writes the packed cache; the GPU reads it
    import torch
    from head_latent_attention_cache_amd import api
    cfg = SMALL_CONFIGS[key]
    _case(f"{cfg.cache_fmt} unpack")
    inp = make_workload(cfg, seed=5)
    st = om.build_cache(cfg, inp)
    dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
    cache, aux = api.new_cache(dims, geom)
    cache.copy_(torch.from_numpy(st["codes"]))
    aux.copy_(torch.from_numpy(np.concatenate([st["cscale"].reshape(-1), st["rscale"].reshape(-1)])))
    out = torch.empty((cfg.batch, cfg.capacity, cfg.d_qk), dtype=torch.float32, device="cuda")
    api.cache_dequant(dims, geom, cache, aux, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), st["values"])
    # attention over the oracle's packed cache
    ref = om.run(cfg, inp, st=st)
    q_abs = gp.to_device(gp_bf16(ref["q_abs"]))
    o_lat = torch.empty((cfg.batch, cfg.n_q, cfg.n_heads, cfg.d_c), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((cfg.batch, cfg.n_q, cfg.n_heads), dtype=torch.float32, device="cuda")
    api.attention(dims, geom, q_abs, gp.int_tensor([cfg.q_first] * cfg.batch),
                  gp.int_tensor([cfg.newest] * cfg.batch), cache, aux, o_lat, lse)
    torch.cuda.synchronize()
    B, n_q, H = cfg.batch, cfg.n_q, cfg.n_heads
    gp.compare("o_lat", gp.to_host(o_lat), ref["o_lat"].reshape(B, n_q, H, cfg.d_c), "bf16")
    gp.compare("lse", gp.to_host(lse), ref["lse"].reshape(B, n_q, H), "bf16")


def gp_bf16(a):
    from mla_inputs import bf16_bits_from_f32
    return bf16_bits_from_f32(np.asarray(a, np.float32))


@pytest.mark.parametrize("key,q_shift", [(2, 0), (3, 0), (4, 0), (3, 1), (4, -2), (3, 4), (5, 0), (5, 1), (6, 0)])
def test_mask_counts_bitexact(gpu_lib, key, q_shift):
    """q_abs = 0 makes every visible score 0, so exp(lse) is the number of
    visible keys exactly (and rows with none give lse = -inf)."""
    import torch
    from head_latent_attention_cache_amd import api
    cfg = SMALL_CONFIGS[key]
    _case(f"mask {cfg.name} shift {q_shift}")
    inp = make_workload(cfg, seed=6)
    got = gp.run_gpu(cfg, inp, fill=0xFF if cfg.cache_given else None, keep_device=True)
    dev = got["_dev"]
    q_first = cfg.q_first + q_shift
    q0 = torch.zeros_like(dev["q_abs"])
    o_lat = torch.empty_like(dev["o_lat"])
    lse = torch.empty_like(dev["lse"])
    api.attention(dev["dims"], dev["geom"], q0, gp.int_tensor([q_first] * cfg.batch), dev["newest"],
                  dev["cache"], dev["aux"], o_lat, lse)
    torch.cuda.synchronize()
    mask = om.mask_matrix(cfg, q_first, cfg.newest)          # [n_q, capacity]
    n_vis = np.repeat(mask.sum(axis=1), cfg.n_heads).reshape(cfg.n_q, cfg.n_heads)
    got_lse = lse.cpu().numpy().astype(np.float64)
    for b in range(cfg.batch):
        none = n_vis == 0
        assert np.all(np.isneginf(got_lse[b][none]))
        assert np.array_equal(np.rint(np.exp(got_lse[b][~none])), n_vis[~none].astype(np.float64))
    if (n_vis == 0).any():
        o = gp.to_host(o_lat)
        assert np.all(o[:, n_vis == 0] == 0.0)


def test_fully_masked_rows(gpu_lib):
    import torch
    from head_latent_attention_cache_amd import api
    cfg = SMALL_CONFIGS[3]
    _case("fully masked")
    inp = make_workload(cfg, seed=7)
    got = gp.run_gpu(cfg, inp, keep_device=True)
    dev = got["_dev"]
    o_lat = torch.full_like(dev["o_lat"], 5.0)
    lse = torch.empty_like(dev["lse"])
    far = cfg.newest + cfg.window          # every written frame is outside this query's window
    api.attention(dev["dims"], dev["geom"], dev["q_abs"], gp.int_tensor([far] * cfg.batch),
                  dev["newest"], dev["cache"], dev["aux"], o_lat, lse)
    torch.cuda.synchronize()
    assert torch.all(o_lat == 0).item()
    assert torch.all(torch.isneginf(lse)).item()


@pytest.mark.parametrize("key", [2, 3, 5, 6])
def test_attention_is_deterministic(gpu_lib, key):
    import torch
    from head_latent_attention_cache_amd import api
    cfg = SMALL_CONFIGS[key]
    _case(f"determinism {cfg.name}")
    inp = make_workload(cfg, seed=8)
    got = gp.run_gpu(cfg, inp, keep_device=True)
    dev = got["_dev"]
    outs = []
    for _ in range(2):
        o_lat = torch.empty_like(dev["o_lat"])
        lse = torch.empty_like(dev["lse"])
        api.attention(dev["dims"], dev["geom"], dev["q_abs"], dev["q_first"], dev["newest"],
                      dev["cache"], dev["aux"], o_lat, lse)
        outs.append((o_lat.clone(), lse.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))


def test_ragged_batch_lengths(gpu_lib):
    """Sequences of one batch at different lengths (per-sequence newest)."""
    import torch
    from head_latent_attention_cache_amd import api
    cfg = SMALL_CONFIGS[2]
    _case("ragged decode")
    inp = make_workload(cfg, seed=9)
    got = gp.run_gpu(cfg, inp, fill=0xFF, keep_device=True)
    dev = got["_dev"]
    lens = [300, 77, 1][:cfg.batch]
    newest = gp.int_tensor([n - 1 for n in lens])
    q_first = gp.int_tensor([n - 1 for n in lens])
    refs = []
    for b, n in enumerate(lens):
        c = cfg.replace(batch=1, n_frames=n, q_first=n - 1)
        sub = {k: inp[k][b:b + 1] for k in ("q_nope", "q_rope")}
        sub.update({k: inp[k] for k in ("w_uk", "w_uv", "w_o")})
        # the GPU cache holds given rows at positions 0..298 and the appended
        # newest token at 299; a sequence of length n sees positions 0..n-1
        st = om.new_cache(c)
        L = inp["cache_c"].shape[1]
        m = min(n, L)
        om.given_cache(st, c, inp["cache_c"][b:b + 1, :m], inp["cache_r"][b:b + 1, :m])
        if n > L:
            om.append_frame(st, c, om.as_f64(inp["x_new"][b:b + 1, 0]), om.as_f64(inp["w_dkr"]), L)
        refs.append(om.run(c, sub, st=st))
    q_abs = torch.empty_like(dev["q_abs"])
    api.absorb_q(dev["dims"], dev["geom"], gp.to_device(inp["q_nope"]), gp.to_device(inp["q_rope"]),
                 q_first, gp.to_device(inp["w_uk"]), q_abs)
    o_lat = torch.empty_like(dev["o_lat"])
    lse = torch.empty_like(dev["lse"])
    api.attention(dev["dims"], dev["geom"], q_abs, q_first, newest, dev["cache"], dev["aux"], o_lat, lse)
    torch.cuda.synchronize()
    for b, r in enumerate(refs):
        gp.compare(f"q_abs[{b}]", gp.to_host(q_abs)[b:b + 1], r["q_abs"], "bf16")
        gp.compare(f"o_lat[{b}]", gp.to_host(o_lat)[b], r["o_lat"].reshape(cfg.n_q, cfg.n_heads, cfg.d_c), "bf16")
        gp.compare(f"lse[{b}]", gp.to_host(lse)[b], r["lse"].reshape(cfg.n_q, cfg.n_heads), "bf16")
