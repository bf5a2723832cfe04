"""Thin torch-facing wrappers over the C-ABI (argument marshalling only).

PyTorch provides device memory and the current HIP stream; every step of the
MLA path runs in the library's HIP kernels.  Each wrapper checks device,
dtype, contiguity and element counts, then passes raw pointers through.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (MLA_BF16, MLA_CACHE_DENSE, MLA_CACHE_INT2, MLA_CACHE_INT4, MLA_F32, MlaDims, MlaGeom,
                   check, load, load_probe)

_TORCH_DTYPE = {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16}


def make_dims(n_heads, d_model, d_nope, d_v, d_c, d_r, rope_dims, bands, theta=10000.0,
              softmax_scale=0.0, dtype="bf16", cache_fmt="dense", qk_norm=False, qk_norm_eps=1e-6) -> MlaDims:
    d = MlaDims()
    d.n_heads, d.d_model, d.d_nope, d.d_v, d.d_c, d.d_r = n_heads, d_model, d_nope, d_v, d_c, d_r
    d.rope_dims = rope_dims
    b = list(bands) + [0] * (3 - len(bands))
    d.band[0], d.band[1], d.band[2] = b[0], b[1], b[2]
    d.rope_theta = theta
    d.softmax_scale = softmax_scale
    d.dtype = {"f32": MLA_F32, "bf16": MLA_BF16}[dtype] if isinstance(dtype, str) else dtype
    d.cache_fmt = ({"dense": MLA_CACHE_DENSE, "int4": MLA_CACHE_INT4, "int2": MLA_CACHE_INT2}[cache_fmt]
                   if isinstance(cache_fmt, str) else cache_fmt)
    d.qk_norm = int(bool(qk_norm))
    d.qk_norm_eps = qk_norm_eps
    return d


def make_geom(batch, grid_h, grid_w, window, frames_per_block=1) -> MlaGeom:
    g = MlaGeom()
    g.batch, g.grid_h, g.grid_w, g.window, g.frames_per_block = batch, grid_h, grid_w, window, frames_per_block
    return g


def dims_from_config(cfg) -> MlaDims:
    """Dimensions from any object with the workload attribute names."""
    return make_dims(cfg.n_heads, cfg.d_model, cfg.d_nope, cfg.d_v, cfg.d_c, cfg.d_r, cfg.rope_dims,
                     cfg.bands, cfg.theta, 0.0, cfg.dtype, cfg.cache_fmt, getattr(cfg, "qk_norm", False),
                     getattr(cfg, "qk_eps", 1e-6))


def geom_from_config(cfg, batch=None) -> MlaGeom:
    return make_geom(cfg.batch if batch is None else batch, cfg.grid_h, cfg.grid_w, cfg.window,
                     cfg.frames_per_block)


def torch_dtype(dims: MlaDims) -> torch.dtype:
    return _TORCH_DTYPE[dims.dtype]


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, numel=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _rd(d):
    return ctypes.byref(d)


# ---------------------------------------------------------------------------
# cache allocation helpers
# ---------------------------------------------------------------------------
def cache_nbytes(dims, geom):
    lib = load()
    return int(lib.mla_cache_bytes(_rd(dims), _rd(geom))), int(lib.mla_cache_aux_bytes(_rd(dims), _rd(geom)))


def new_cache(dims, geom, device="cuda", fill=None):
    """Allocate (cache, cache_aux) tensors.  ``fill``: optional byte value
    written into every byte (for poisoning unwritten slots in tests)."""
    nb, na = cache_nbytes(dims, geom)
    cap = geom.window * geom.grid_h * geom.grid_w
    dqk = dims.d_c + dims.d_r
    if dims.cache_fmt in (MLA_CACHE_INT4, MLA_CACHE_INT2):
        # low-bit: code bytes per row as the library sizes them; fp16 scales
        cache = torch.empty((geom.batch, cap, nb // max(1, geom.batch * cap)), dtype=torch.uint8, device=device)
    else:
        cache = torch.empty((geom.batch, cap, dqk), dtype=torch_dtype(dims), device=device)
    # fp16 scales (low-bit) and / or the per-slot key inverse RMS (QK normalisation)
    aux = torch.empty(na // 2, dtype=torch.float16, device=device) if na else None
    assert cache.numel() * cache.element_size() == nb
    if fill is not None:
        cache.view(torch.uint8).fill_(fill)
        if aux is not None:
            aux.view(torch.uint8).fill_(fill)
    else:
        cache.zero_()
        if aux is not None:
            aux.zero_()
    return cache, aux


def _check_cache(dims, geom, cache, cache_aux):
    nb, na = cache_nbytes(dims, geom)
    if dims.cache_fmt in (MLA_CACHE_INT4, MLA_CACHE_INT2):
        _need(cache, "cache", torch.uint8, nb)
    else:
        _need(cache, "cache", torch_dtype(dims), nb // (2 if dims.dtype == MLA_BF16 else 4))
    if na:
        _need(cache_aux, "cache_aux", torch.float16, na // 2)


def key_scales(dims, geom, cache_aux):
    """Float32 view [B, capacity] of the per-slot key inverse RMS held in
    cache_aux (QK normalisation)."""
    cap = geom.window * geom.grid_h * geom.grid_w
    rows = geom.batch * cap
    nb, na = cache_nbytes(dims, geom)
    off = na - 4 * rows
    return cache_aux.view(torch.uint8)[off:na].view(torch.float32).view(geom.batch, cap)


# ---------------------------------------------------------------------------
# the four path calls + inspection
# ---------------------------------------------------------------------------
def cache_append(dims, geom, x, frame, w_dkr, cache, cache_aux=None, workspace=None):
    """x [B, n_tokens, d_model]; frame int32 [B]; w_dkr [d_c + d_r, d_model]."""
    lib = load()
    dt = torch_dtype(dims)
    B = geom.batch
    n_tokens = x.shape[1] if x.dim() == 3 else 0
    _need(x, "x", dt, B * n_tokens * dims.d_model)
    _need(frame, "frame", torch.int32, B)
    _need(w_dkr, "w_dkr", dt, (dims.d_c + dims.d_r) * dims.d_model)
    _check_cache(dims, geom, cache, cache_aux)
    need = int(lib.mla_append_workspace_size(_rd(dims), _rd(geom), n_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    check(lib.mla_cache_append(_rd(dims), _rd(geom), _stream(), _ptr(x), n_tokens, _ptr(frame),
                               _ptr(w_dkr), _ptr(cache), _ptr(cache_aux), _ptr(workspace),
                               workspace.numel() * workspace.element_size()))


def append_workspace_bytes(dims, geom, n_tokens):
    return int(load().mla_append_workspace_size(_rd(dims), _rd(geom), n_tokens))


def absorb_q(dims, geom, q_nope, q_rope, q_first, w_uk, q_abs):
    """q_nope [B, n_q, H, d_nope]; q_rope [B, n_q, H, d_r] -> q_abs [B, n_q, H, d_c + d_r]."""
    lib = load()
    dt = torch_dtype(dims)
    B, H = geom.batch, dims.n_heads
    n_q = q_nope.shape[1]
    _need(q_nope, "q_nope", dt, B * n_q * H * dims.d_nope)
    _need(q_rope, "q_rope", dt, B * n_q * H * dims.d_r)
    _need(q_first, "q_first", torch.int32, B)
    _need(w_uk, "w_uk", dt, H * dims.d_c * dims.d_nope)
    _need(q_abs, "q_abs", dt, B * n_q * H * (dims.d_c + dims.d_r))
    check(lib.mla_absorb_q(_rd(dims), _rd(geom), _stream(), n_q, _ptr(q_nope), _ptr(q_rope),
                           _ptr(q_first), _ptr(w_uk), _ptr(q_abs)))


def fold_query_weights(dims, w_uq, w_uk, w_fold):
    """w_uq [H * d_nope, d_cq], w_uk [H, d_c, d_nope] -> w_fold [H, d_c, d_cq] (load time)."""
    lib = load()
    dt = torch_dtype(dims)
    H = dims.n_heads
    d_cq = w_uq.shape[-1]
    _need(w_uq, "w_uq", dt, H * dims.d_nope * d_cq)
    _need(w_uk, "w_uk", dt, H * dims.d_c * dims.d_nope)
    _need(w_fold, "w_fold", dt, H * dims.d_c * d_cq)
    check(lib.mla_fold_query_weights(_rd(dims), _stream(), d_cq, _ptr(w_uq), _ptr(w_uk), _ptr(w_fold)))


def absorb_q_folded(dims, geom, c_q, q_rope, q_first, w_fold, q_abs):
    """c_q [B, n_q, d_cq]; q_rope [B, n_q, H, d_r] -> q_abs [B, n_q, H, d_c + d_r]."""
    lib = load()
    dt = torch_dtype(dims)
    B, H = geom.batch, dims.n_heads
    n_q, d_cq = c_q.shape[1], c_q.shape[2]
    _need(c_q, "c_q", dt, B * n_q * d_cq)
    _need(q_rope, "q_rope", dt, B * n_q * H * dims.d_r)
    _need(q_first, "q_first", torch.int32, B)
    _need(w_fold, "w_fold", dt, H * dims.d_c * d_cq)
    _need(q_abs, "q_abs", dt, B * n_q * H * (dims.d_c + dims.d_r))
    check(lib.mla_absorb_q_folded(_rd(dims), _rd(geom), _stream(), n_q, d_cq, _ptr(c_q), _ptr(q_rope),
                                  _ptr(q_first), _ptr(w_fold), _ptr(q_abs)))


def qk_norm_prepare(dims, w_uk, g_q, g_k, w_uk_folded, gram):
    """Load time: w_uk_folded = w_uk * g_q * g_k (per head and content dim),
    gram [d_c, d_c] float = sum_h w_uk[h] w_uk[h]^T."""
    lib = load()
    dt = torch_dtype(dims)
    H = dims.n_heads
    _need(w_uk, "w_uk", dt, H * dims.d_c * dims.d_nope)
    _need(g_q, "g_q", dt, H * dims.d_nope)
    _need(g_k, "g_k", dt, H * dims.d_nope)
    _need(w_uk_folded, "w_uk_folded", dt, H * dims.d_c * dims.d_nope)
    _need(gram, "gram", torch.float32, dims.d_c * dims.d_c)
    check(lib.mla_qk_norm_prepare(_rd(dims), _stream(), _ptr(w_uk), _ptr(g_q), _ptr(g_k), _ptr(w_uk_folded),
                                  _ptr(gram)))


def key_norm_workspace_bytes(dims, geom, n_tokens):
    return int(load().mla_key_norm_workspace_size(_rd(dims), _rd(geom), int(n_tokens)))


def cache_key_norm(dims, geom, n_tokens, frame, gram, cache, cache_aux, workspace=None):
    """Key inverse RMS of the rows of n_tokens tokens written at frame[b]
    onwards (the arguments of the matching mla_cache_append)."""
    lib = load()
    _check_cache(dims, geom, cache, cache_aux)
    _need(frame, "frame", torch.int32, geom.batch)
    _need(gram, "gram", torch.float32, dims.d_c * dims.d_c)
    need = key_norm_workspace_bytes(dims, geom, n_tokens)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=cache.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib.mla_cache_key_norm(_rd(dims), _rd(geom), _stream(), int(n_tokens), _ptr(frame), _ptr(gram),
                                 _ptr(cache), _ptr(cache_aux), _ptr(workspace), nbytes))


def attention_workspace_bytes(dims, geom, n_q):
    return int(load().mla_attention_workspace_size(_rd(dims), _rd(geom), n_q))


def attention(dims, geom, q_abs, q_first, newest, cache, cache_aux, o_lat, lse=None, workspace=None):
    """q_abs [B, n_q, H, d_c + d_r] -> o_lat [B, n_q, H, d_c], lse [B, n_q, H] (optional)."""
    lib = load()
    dt = torch_dtype(dims)
    B, H = geom.batch, dims.n_heads
    n_q = q_abs.shape[1]
    _need(q_abs, "q_abs", dt, B * n_q * H * (dims.d_c + dims.d_r))
    _need(q_first, "q_first", torch.int32, B)
    _need(newest, "newest", torch.int32, B)
    _check_cache(dims, geom, cache, cache_aux)
    _need(o_lat, "o_lat", dt, B * n_q * H * dims.d_c)
    if lse is not None:
        _need(lse, "lse", torch.float32, B * n_q * H)
    need = attention_workspace_bytes(dims, geom, n_q)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_abs.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib.mla_attention(_rd(dims), _rd(geom), _stream(), n_q, _ptr(q_abs), _ptr(q_first),
                            _ptr(newest), _ptr(cache), _ptr(cache_aux), _ptr(o_lat), _ptr(lse),
                            _ptr(workspace), ws_bytes))


def attention_noalloc(dims, geom, q_abs, q_first, newest, cache, cache_aux, o_lat, lse=None):
    """mla_attention_noalloc: as ``attention`` with the library's static
    scratch instead of a workspace (nothing is allocated)."""
    lib = load()
    dt = torch_dtype(dims)
    B, H = geom.batch, dims.n_heads
    n_q = q_abs.shape[1]
    _need(q_abs, "q_abs", dt, B * n_q * H * (dims.d_c + dims.d_r))
    _need(q_first, "q_first", torch.int32, B)
    _need(newest, "newest", torch.int32, B)
    _check_cache(dims, geom, cache, cache_aux)
    _need(o_lat, "o_lat", dt, B * n_q * H * dims.d_c)
    if lse is not None:
        _need(lse, "lse", torch.float32, B * n_q * H)
    check(lib.mla_attention_noalloc(_rd(dims), _rd(geom), _stream(), n_q, _ptr(q_abs), _ptr(q_first),
                                    _ptr(newest), _ptr(cache), _ptr(cache_aux), _ptr(o_lat), _ptr(lse)))


def unabsorb_out(dims, geom, o_lat, w_uv, w_o, o_heads, y):
    """o_lat [B, n_q, H, d_c] -> o_heads [B, n_q, H * d_v], y [B, n_q, d_model]."""
    lib = load()
    dt = torch_dtype(dims)
    B, H = geom.batch, dims.n_heads
    n_q = o_lat.shape[1]
    _need(o_lat, "o_lat", dt, B * n_q * H * dims.d_c)
    _need(w_uv, "w_uv", dt, H * dims.d_v * dims.d_c)
    _need(w_o, "w_o", dt, dims.d_model * H * dims.d_v)
    _need(o_heads, "o_heads", dt, B * n_q * H * dims.d_v)
    _need(y, "y", dt, B * n_q * dims.d_model)
    check(lib.mla_unabsorb_out(_rd(dims), _rd(geom), _stream(), n_q, _ptr(o_lat), _ptr(w_uv),
                               _ptr(w_o), _ptr(o_heads), _ptr(y)))


def cache_dequant(dims, geom, cache, cache_aux, out):
    """Cache rows as float [B, capacity, d_c + d_r] (inspection utility)."""
    lib = load()
    _check_cache(dims, geom, cache, cache_aux)
    cap = geom.window * geom.grid_h * geom.grid_w
    _need(out, "out", torch.float32, geom.batch * cap * (dims.d_c + dims.d_r))
    check(lib.mla_cache_dequant(_rd(dims), _rd(geom), _stream(), _ptr(cache), _ptr(cache_aux), _ptr(out)))


def cache_rope_shift(dims, geom, delta, slot_begin, n_slots, cache, cache_aux):
    """Rotate the rotary keys of slots [slot_begin, slot_begin + n_slots) of
    every sequence by the coordinate shift delta [B, 3] int32 (device)."""
    lib = load()
    _check_cache(dims, geom, cache, cache_aux)
    _need(delta, "delta", torch.int32, geom.batch * 3)
    check(lib.mla_cache_rope_shift(_rd(dims), _rd(geom), _stream(), _ptr(delta), int(slot_begin), int(n_slots),
                                   _ptr(cache), _ptr(cache_aux)))


def probe_mfma(n_workgroups, iters, out, toggle=True):
    """Launch the bf16 MFMA rate probe (measurement only); returns the
    floating-point operations of the launch.  out: float32 device tensor of
    n_workgroups * 256 elements; toggle: alternate two pseudo-random operand
    pairs (True) or repeat one fixed pair (False)."""
    lib = load_probe()
    _need(out, "out", torch.float32, n_workgroups * 256)
    flops = ctypes.c_double(0.0)
    _check_probe(lib.mla_probe_mfma(_stream(), int(n_workgroups), int(iters), int(bool(toggle)), _ptr(out),
                                    ctypes.byref(flops)))
    return flops.value


def probe_hbm_read(src, n_workgroups, out):
    """Launch the streaming-read probe over the bytes of `src` (measurement
    only).  out: int32 device tensor of n_workgroups * 256 elements."""
    lib = load_probe()
    if not (src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous GPU tensor")
    _need(out, "out", torch.int32, n_workgroups * 256)
    n_bytes = src.numel() * src.element_size()
    _check_probe(lib.mla_probe_hbm_read(_stream(), _ptr(src), int(n_bytes), int(n_workgroups), _ptr(out)))
    return n_bytes


def _check_probe(status):
    if status != _lib.MLA_OK:
        raise _lib.MLAError(status, f"{load().mla_status_string(status).decode()}: "
                                    f"{load_probe().mla_probe_last_error().decode()}")


def raw_lib():
    """The loaded ctypes library (for callers passing their own pointers)."""
    return _lib.load()
