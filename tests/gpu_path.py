"""Runs the HIP path through the C-ABI binding on seeded inputs and compares
with the CPU oracle.  Used by the ``gpu``-marked tests, ``smoke()`` and the
bench's parity spot checks."""
from __future__ import annotations

import numpy as np

TOL_F32_ABS = 1e-4           # fp32 storage: max |gpu - oracle|
TOL_BF16_ABS = 2e-2          # bf16 storage: |d| <= abs + rel * |ref|
TOL_BF16_REL = 1e-2
TOL_BF16_L2 = 1e-2           # extra: ||d||_2 / ||ref||_2


def to_device(arr, device="cuda"):
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    raise TypeError(a.dtype)


def to_host(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def int_tensor(vals, device="cuda"):
    import torch
    return torch.tensor(list(vals), dtype=torch.int32, device=device)


def run_gpu(cfg, inp, fill=None, keep_device=False):
    """Append (or load the given cache), absorb, attend, un-absorb.

    Returns a dict of host float64 arrays (and the device tensors when
    ``keep_device``)."""
    import torch

    import head_latent_attention_cache_amd as mla
    from head_latent_attention_cache_amd import api

    mla.load()
    dims = api.dims_from_config(cfg)
    geom = api.geom_from_config(cfg)
    B, H, P = cfg.batch, cfg.n_heads, cfg.tokens_per_frame
    dt = api.torch_dtype(dims)
    cache, aux = api.new_cache(dims, geom, fill=fill)
    w_dkr = to_device(inp["w_dkr"])
    ws = torch.empty(max(16, api.append_workspace_bytes(dims, geom, P)), dtype=torch.uint8, device="cuda")
    if cfg.cache_given:
        # earlier positions are given rows (dense cache); the newest frame is appended
        L = inp["cache_c"].shape[1]
        cache[:, :L, :cfg.d_c] = to_device(inp["cache_c"])
        cache[:, :L, cfg.d_c:] = to_device(inp["cache_r"])
        api.cache_append(dims, geom, to_device(inp["x_new"]).reshape(B, P, cfg.d_model),
                         int_tensor([cfg.n_frames - 1] * B), w_dkr, cache, aux, workspace=ws)
    else:
        x = to_device(inp["x"])                        # [B, F, P, D]
        for f in range(cfg.n_frames):
            api.cache_append(dims, geom, x[:, f].contiguous(), int_tensor([f] * B), w_dkr, cache, aux,
                             workspace=ws)
    q_first = int_tensor([cfg.q_first] * B)
    newest = int_tensor([cfg.newest] * B)
    q_abs = torch.empty((B, cfg.n_q, H, cfg.d_qk), dtype=dt, device="cuda")
    api.absorb_q(dims, geom, to_device(inp["q_nope"]), to_device(inp["q_rope"]), q_first,
                 to_device(inp["w_uk"]), q_abs)
    o_lat = torch.empty((B, cfg.n_q, H, cfg.d_c), dtype=dt, device="cuda")
    lse = torch.empty((B, cfg.n_q, H), dtype=torch.float32, device="cuda")
    api.attention(dims, geom, q_abs, q_first, newest, cache, aux, o_lat, lse)
    o_heads = torch.empty((B, cfg.n_q, H * cfg.d_v), dtype=dt, device="cuda")
    y = torch.empty((B, cfg.n_q, cfg.d_model), dtype=dt, device="cuda")
    api.unabsorb_out(dims, geom, o_lat, to_device(inp["w_uv"]), to_device(inp["w_o"]), o_heads, y)
    torch.cuda.synchronize()
    out = {"q_abs": to_host(q_abs), "o_lat": to_host(o_lat), "lse": to_host(lse),
           "o_heads": to_host(o_heads).reshape(B, cfg.n_q, H, cfg.d_v), "y": to_host(y)}
    if cfg.cache_fmt in ("int4", "int2"):
        out["codes"] = cache.cpu().numpy()
        na = aux.numel()
        ng = cfg.d_c // 32
        a = aux.cpu().numpy()
        out["cscale"] = a[:B * cfg.capacity * ng].reshape(B, cfg.capacity, ng)
        out["rscale"] = a[B * cfg.capacity * ng:na].reshape(B, cfg.capacity)
    else:
        out["cache"] = to_host(cache)
    if keep_device:
        out["_dev"] = {"dims": dims, "geom": geom, "cache": cache, "aux": aux, "q_abs": q_abs,
                       "o_lat": o_lat, "lse": lse, "q_first": q_first, "newest": newest}
    return out


def compare(name, got, ref, dtype, report=None):
    """Assert the path's tolerance; returns (max_abs, rel_l2)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: finiteness differs"
    assert np.array_equal(got[~fin], ref[~fin]), f"{name}: non-finite values differ"
    d = np.abs(got[fin] - ref[fin])
    max_abs = float(d.max(initial=0.0))
    nrm = float(np.linalg.norm(ref[fin]))
    rel_l2 = float(np.linalg.norm(d) / nrm) if nrm > 0 else float(np.linalg.norm(d))
    if report is not None:
        report[name] = (max_abs, rel_l2)
    if dtype == "f32":
        assert max_abs <= TOL_F32_ABS, f"{name}: max |d| = {max_abs:.3g} > {TOL_F32_ABS}"
    else:
        bad = d > TOL_BF16_ABS + TOL_BF16_REL * np.abs(ref[fin])
        assert not bad.any(), (f"{name}: {int(bad.sum())} elements outside {TOL_BF16_ABS} + "
                               f"{TOL_BF16_REL}|ref| (max |d| {max_abs:.3g})")
        assert rel_l2 <= TOL_BF16_L2, f"{name}: relative L2 error {rel_l2:.3g} > {TOL_BF16_L2}"
    return max_abs, rel_l2


def check_lowbit_codes(cfg, codes, cscale, rscale, st, slots):
    """Every stored low-bit code and scale of ``slots`` (bool mask over ring
    slots) is one a correct computation can store: the oracle's row before
    storage rounding (``st["pre"]``), reached up to a float32 computation
    error, rounded to bf16 and quantised.  The error allowed is 2^-16 of the
    largest magnitude in the element's quantisation group (a code step is
    1/7 of it for INT4, all of it for INT2), far above float32 rounding of the
    projection and rotation and far below a code step, so every stored code
    and scale is held to its rounding boundaries.

    Returns the fraction of code bytes equal to the oracle's own."""
    import oracle.int4 as oi
    import oracle.mla as om
    assert cfg.dtype == "bf16"
    bits = om.content_bits(cfg)
    d_c = cfg.d_c
    ncb = d_c * bits // 8
    pre = st["pre"][:, slots]
    gmax_c = np.abs(pre[..., :d_c]).reshape(pre.shape[:-1] + (d_c // 32, 32)).max(axis=-1)
    gmax_r = np.abs(pre[..., d_c:]).max(axis=-1, keepdims=True)
    err = np.concatenate([np.repeat(gmax_c, 32, axis=-1), np.broadcast_to(gmax_r, pre[..., d_c:].shape)],
                         axis=-1) * 2.0 ** -16
    lo, _ = om.bf16_bracket(pre - err)
    _, hi = om.bf16_bracket(pre + err)
    got = np.asarray(codes)[:, slots]
    unpack = oi.unpack_nibbles if bits == 4 else oi.unpack_crumbs
    gc = unpack(got[..., :ncb])
    gr = oi.unpack_nibbles(got[..., ncb:])
    cmin, cmax, csmin, csmax = oi.admissible_groups(lo[..., :d_c], hi[..., :d_c], 32, bits)
    rmin, rmax, rsmin, rsmax = oi.admissible_groups(lo[..., d_c:], hi[..., d_c:], cfg.d_r, 4)
    gcs = np.asarray(cscale)[:, slots].astype(np.float64)
    grs = np.asarray(rscale)[:, slots].astype(np.float64)[..., None]
    for name, g, a, b in (("content codes", gc, cmin, cmax), ("rotary codes", gr, rmin, rmax),
                          ("content scales", gcs, csmin.astype(np.float64), csmax.astype(np.float64)),
                          ("rotary scales", grs, rsmin.astype(np.float64), rsmax.astype(np.float64))):
        out = (g < a) | (g > b)
        assert not out.any(), f"{name}: {int(out.sum())} of {out.size} outside the admissible bounds"
    return float(np.mean(got == st["codes"][:, slots]))


def upload_oracle_cache(cfg, st):
    """Device (dims, geom, cache, aux) holding exactly the oracle's stored cache
    ``st`` (dense values, or low-bit codes and fp16 scales)."""
    import torch

    from head_latent_attention_cache_amd import api
    from mla_inputs import bf16_bits_from_f32
    dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
    cache, aux = api.new_cache(dims, geom)
    if cfg.cache_fmt in ("int4", "int2"):
        cache.copy_(torch.from_numpy(st["codes"]))
        aux.copy_(torch.from_numpy(np.concatenate([st["cscale"].reshape(-1), st["rscale"].reshape(-1)])))
    elif cfg.dtype == "bf16":
        cache.copy_(to_device(bf16_bits_from_f32(st["values"].astype(np.float32))))
    else:
        cache.copy_(torch.from_numpy(st["values"].astype(np.float32)))
    return {"dims": dims, "geom": geom, "cache": cache, "aux": aux}
