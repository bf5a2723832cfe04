"""Plain float64 definition of multi-head latent attention (MLA) over a shared
per-token latent cache, with per-head keys and values materialised.

Test infrastructure only (see the package docstring).

Pages cited (titles as printed; sections in brackets):
  [MLA concept]  "Multi-Head Latent Attention", praveentn.live concept page
  [MLA explainer] "Understanding Multi-Head Latent Attention and KV Compression"
  [VideoMLA review] "VideoMLA: Compressing Video Diffusion Memory by 92.7% with
                  Low-Rank Latent Attention", alanhou.org blog review
  [MLA topics]   "Multi-Head Latent Attention", thelatestinai.com topic page
                  (abstract cards: VideoMLA, QuantMLA, ...)

Conventions (row vectors, row-major arrays, last axis fastest):
  w_dkr [d_c + d_r, d_model]  rows 0..d_c-1 map h -> c_kv, rows d_c.. map h -> k_rope
  w_uk  [H, d_c, d_nope]      w_uk[h] is the transpose of W^UK_h (d_nope x d_c)
  w_uv  [H, d_v, d_c]         w_uv[h] is W^UV_h
  w_o   [d_model, H * d_v]    y = concat_h(o_h) . w_o^T
"""
from __future__ import annotations

import numpy as np

from . import int4

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
INT4_GROUP = 32


# ---------------------------------------------------------------------------
# input decoding and storage rounding
# ---------------------------------------------------------------------------
def as_f64(arr) -> np.ndarray:
    """Generator output (float32, or bf16 bit patterns as uint16) -> float64."""
    a = np.asarray(arr)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range; the
    smallest subnormal step is 2**-133.
    """
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(a / step) * step
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, a), r)


def bf16_bracket(a):
    """The two bfloat16 values next to each float64 value: (largest bf16 <= a,
    smallest bf16 >= a), equal where ``a`` is a bf16 value.  A computation that
    reaches ``a`` up to an error below half a bf16 step and then rounds to
    nearest lands on one of them."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.floor(a / step) * step, np.ceil(a / step) * step


def round_to_storage(a, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(a)
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# cache geometry: ring slots, positions, visibility
# [VideoMLA review, The Gap] and [MLA topics, VideoMLA abstract]: a fixed-size
# sliding window of recent frames; the workload's block-causal frame mask.
# ---------------------------------------------------------------------------
def token_coords(cfg, frame, tok) -> np.ndarray:
    """Rotary coordinates of token ``tok`` of frame ``frame``.

    3D: (t, h, w) = (frame, row, column) of the frame grid, tokens row-major.
    1D: the token position frame * P + tok (P = 1 for language models).
    """
    frame = np.asarray(frame, dtype=np.int64)
    tok = np.asarray(tok, dtype=np.int64)
    frame, tok = np.broadcast_arrays(frame, tok)
    if cfg.rope_dims == 3:
        return np.stack([frame, tok // cfg.grid_w, tok % cfg.grid_w], axis=-1).astype(np.float64)
    return (frame * cfg.tokens_per_frame + tok)[..., None].astype(np.float64)


def slot_index(cfg, frame, tok):
    """Ring slot of token ``tok`` of frame ``frame``: (frame mod W) * P + tok."""
    return (np.asarray(frame) % cfg.window) * cfg.tokens_per_frame + np.asarray(tok)


def slot_frames(cfg, newest: int) -> np.ndarray:
    """Frame held by every slot once frames 0..newest were appended; -1 if empty."""
    ring_pos = np.arange(cfg.capacity) // cfg.tokens_per_frame
    f = newest - np.mod(newest - ring_pos, cfg.window)
    return np.where(f >= 0, f, -1)


def visible(cfg, f_q, f_k):
    """Key frame f_k is visible to query frame f_q: written, not in a later
    block (block-causal), and inside the window."""
    f_q = np.asarray(f_q)
    f_k = np.asarray(f_k)
    fpb = cfg.frames_per_block
    return (f_k >= 0) & (f_k // fpb <= f_q // fpb) & (f_q - f_k < cfg.window)


def query_frames(cfg, q_first: int) -> np.ndarray:
    return q_first + np.arange(cfg.n_q) // cfg.tokens_per_frame


def mask_matrix(cfg, q_first: int, newest: int) -> np.ndarray:
    """[n_q, capacity] visibility of every slot to every query token."""
    fq = query_frames(cfg, q_first)
    fk = slot_frames(cfg, newest)
    return visible(cfg, fq[:, None], fk[None, :])


# ---------------------------------------------------------------------------
# rotary embedding: [MLA concept, The RoPE problem, and the decoupled fix]
# (a position-dependent rotation whose query/key product depends on the offset)
# and [VideoMLA review, Key Concepts] (3D-RoPE over time, height and width).
# Reading: interleaved pairs, per-band frequencies theta^(-2i/d_b), bands t|h|w.
# ---------------------------------------------------------------------------
def rope_frequencies(band: int, theta: float) -> np.ndarray:
    i = np.arange(band // 2, dtype=np.float64)
    return theta ** (-2.0 * i / band)


def rope_rotate(u, coords, cfg) -> np.ndarray:
    """Rotate ``u[..., d_r]`` at ``coords[..., rope_dims]`` (broadcastable)."""
    u = np.asarray(u, dtype=np.float64)
    coords = np.asarray(coords, dtype=np.float64)
    out = np.empty(np.broadcast_shapes(u.shape, coords.shape[:-1] + (u.shape[-1],)))
    off = 0
    for axis, band in enumerate(cfg.bands):
        ang = coords[..., axis:axis + 1] * rope_frequencies(band, cfg.theta)
        cos, sin = np.cos(ang), np.sin(ang)
        x0 = u[..., off:off + band:2]
        x1 = u[..., off + 1:off + band:2]
        out[..., off:off + band:2] = x0 * cos - x1 * sin
        out[..., off + 1:off + band:2] = x0 * sin + x1 * cos
        off += band
    return out


# ---------------------------------------------------------------------------
# cache append: [MLA concept, Low-rank joint compression] and [MLA explainer,
# Low-Rank Joint Compression] (down-project to one latent, cache only it),
# [MLA explainer, Decoupling RoPE] (the small rotary key is cached beside it).
# ---------------------------------------------------------------------------
def content_bits(cfg) -> int:
    """Bits per content-latent code of a low-bit cache (the rotary key is INT4)."""
    return {"int4": 4, "int2": 2}[cfg.cache_fmt]


def new_cache(cfg) -> dict:
    B, cap = cfg.batch, cfg.capacity
    # "pre": each slot's row before storage rounding (float64), kept so that
    # tests can bound the low-bit codes a correct computation may store
    st = {"values": np.zeros((B, cap, cfg.d_qk)), "pre": np.zeros((B, cap, cfg.d_qk)), "newest": -1}
    if cfg.cache_fmt in ("int4", "int2"):
        st["codes"] = np.zeros((B, cap, cfg.d_c * content_bits(cfg) // 8 + cfg.d_r // 2), np.uint8)
        st["cscale"] = np.zeros((B, cap, cfg.d_c // INT4_GROUP), np.float16)
        st["rscale"] = np.zeros((B, cap), np.float16)
    return st


def store_rows(st, cfg, slots, rows):
    """Round rows to the cache format and write them at ``slots``."""
    st["pre"][:, slots] = rows
    stored = round_to_storage(rows, cfg.dtype)
    if cfg.cache_fmt in ("int4", "int2"):
        q = int4.quantize_cache_rows(stored, cfg.d_c, INT4_GROUP, content_bits(cfg))
        st["codes"][:, slots] = q["codes"]
        st["cscale"][:, slots] = q["cscale"]
        st["rscale"][:, slots] = q["rscale"]
        stored = q["values"]
    st["values"][:, slots] = stored


def project_rows(cfg, x_rows, w_dkr, frames, toks) -> np.ndarray:
    """Cache rows [c | k] (before storage rounding) of hidden states
    ``x_rows [..., d_model]`` at (frame, token) positions ``frames``, ``toks``
    (broadcast against the leading axes): c = h W_DKV, k = RoPE(h W_KR)."""
    y = np.asarray(x_rows, np.float64) @ np.asarray(w_dkr, np.float64).T
    c = y[..., :cfg.d_c]
    k = rope_rotate(y[..., cfg.d_c:], token_coords(cfg, frames, toks), cfg)
    return np.concatenate([c, k], axis=-1)


def append_frame(st, cfg, x_frame, w_dkr, frame: int):
    """x_frame [B, P, d_model]; stores c = h W_DKV and k = RoPE(h W_KR)."""
    P = cfg.tokens_per_frame
    rows = project_rows(cfg, x_frame, w_dkr, frame, np.arange(P))
    store_rows(st, cfg, slot_index(cfg, frame, np.arange(P)), rows)
    st["newest"] = max(st["newest"], frame)


def given_cache(st, cfg, cache_c, cache_r):
    """Decode workload: frames 0..L/P-1 hold given (already rotated) rows."""
    L = cache_c.shape[1]
    P = cfg.tokens_per_frame
    rows = np.concatenate([as_f64(cache_c), as_f64(cache_r)], axis=-1)
    i = np.arange(L)
    store_rows(st, cfg, slot_index(cfg, i // P, i % P), rows)
    st["newest"] = max(st["newest"], L // P - 1)


# ---------------------------------------------------------------------------
# re-rotation of cached rotary keys: [MLA topics, Irminsul abstract] (an MLA
# row is a position-free content latent plus a small rotary key that a change
# of position corrects in closed form) and [MLA topics, the RedKnot
# head-aware reuse abstract] (relocating content computed at another
# position).  Rotations by angles
# proportional to the coordinate compose: R(p + d) = R(d) R(p), so a key
# stored at coordinates p is moved to p + d by rotating it with R(d).
# ---------------------------------------------------------------------------
def rope_shift(st, cfg, delta, slot_begin: int, n_slots: int):
    """Rotate the stored rotary keys of slots [slot_begin, slot_begin + n_slots)
    of every sequence b by the coordinate shift ``delta[b]`` ((t, h, w) for
    3D; 1D uses ``delta[b][0]``, a position shift), as if each of those
    tokens had been appended that much further along.  The rotated key is
    rounded to the cache format (low-bit: rounded to bf16, then re-quantised
    to INT4 with a new per-token scale); the content latent is untouched and a
    shift that is zero in the coordinates the embedding uses (1D: the first)
    leaves the rows unchanged."""
    delta = np.asarray(delta, dtype=np.int64).reshape(cfg.batch, 3)
    sl = slice(slot_begin, slot_begin + n_slots)
    for b in range(cfg.batch):
        d = delta[b, :cfg.rope_dims].astype(np.float64)
        if not np.any(d):
            continue
        k = rope_rotate(st["values"][b, sl, cfg.d_c:], d, cfg)
        if "pre" in st:
            st["pre"][b, sl, cfg.d_c:] = k
        k = round_to_storage(k, cfg.dtype)
        if cfg.cache_fmt in ("int4", "int2"):
            codes, scale = int4.quantize_groups(k, cfg.d_r)
            st["codes"][b, sl, cfg.d_c * content_bits(cfg) // 8:] = int4.pack_nibbles(codes)
            st["rscale"][b, sl] = scale[..., 0]
            k = int4.dequantize_groups(codes, scale, cfg.d_r)
        st["values"][b, sl, cfg.d_c:] = k


# ---------------------------------------------------------------------------
# absorbed query: [MLA concept, Low-rank joint compression] (q.(W^UK c) =
# ((W^UK)^T q).c, so W^UK folds into the query side)
# ---------------------------------------------------------------------------
def query_coords(cfg, q_first: int) -> np.ndarray:
    i = np.arange(cfg.n_q)
    P = cfg.tokens_per_frame
    return token_coords(cfg, q_first + i // P, i % P)


def absorb_query(cfg, q_nope, q_rope, w_uk, q_first: int) -> np.ndarray:
    """q_abs[b,t,h] = [ (W^UK_h)^T q_nope ; RoPE(q_rope) ]  -> [B, n_q, H, d_c + d_r]."""
    q_lat = np.einsum("bthi,hji->bthj", np.asarray(q_nope, np.float64), np.asarray(w_uk, np.float64))
    coords = query_coords(cfg, q_first)[None, :, None, :]
    q_rot = rope_rotate(q_rope, coords, cfg)
    return np.concatenate([q_lat, q_rot], axis=-1)


# ---------------------------------------------------------------------------
# low-rank query with the key up-projection folded in at load time:
# [MLA concept, Low-rank joint compression]: with a query latent c^Q and its
# up-projection W^UQ, q_t . k_s = (W^UQ c^Q_t) . (W^UK c^KV_s)
# = c^Q_t^T (W^UQ^T W^UK) c^KV_s, so the product of the two up-projections
# can be formed once when the weights are loaded.
# ---------------------------------------------------------------------------
def query_up(cfg, c_q, w_uq) -> np.ndarray:
    """Per-head content queries q_nope [..., H, d_nope] of query latents
    c_q [..., d_cq]: q_nope[.., h, i] = sum_j w_uq[h d_nope + i, j] c_q[.., j]."""
    q = np.asarray(c_q, np.float64) @ np.asarray(w_uq, np.float64).T
    return q.reshape(q.shape[:-1] + (cfg.n_heads, cfg.d_nope))


def fold_query_weights(cfg, w_uq, w_uk) -> np.ndarray:
    """w_fold [H, d_c, d_cq], w_fold[h] = w_uk[h] . W^UQ_h with W^UQ_h the
    rows h d_nope .. (h + 1) d_nope - 1 of w_uq (so that w_fold[h] . c_q is
    (W^UK_h)^T W^UQ_h c_q, the absorbed content query of head h)."""
    wq = np.asarray(w_uq, np.float64).reshape(cfg.n_heads, cfg.d_nope, -1)
    return np.matmul(np.asarray(w_uk, np.float64), wq)


def absorb_query_folded(cfg, c_q, q_rope, w_fold, q_first: int) -> np.ndarray:
    """q_abs[b,t,h] = [ w_fold[h] . c_q[b,t] ; RoPE(q_rope) ] -> [B, n_q, H, d_c + d_r]."""
    q_lat = np.einsum("btj,hcj->bthc", np.asarray(c_q, np.float64), np.asarray(w_fold, np.float64))
    coords = query_coords(cfg, q_first)[None, :, None, :]
    q_rot = rope_rotate(q_rope, coords, cfg)
    return np.concatenate([q_lat, q_rot], axis=-1)


# ---------------------------------------------------------------------------
# attention with materialised per-head keys/values (the plain definition):
# [MLA concept, The RoPE problem, and the decoupled fix] each head's query and
# key join a content part and the rotary part shared by all heads;
# [MLA explainer, On-the-Fly Reconstruction] K and V are up-projections of c.
# ---------------------------------------------------------------------------
def softmax_scale(cfg) -> float:
    """1/sqrt(d_nope + d_r): the textbook scale for the width of the
    materialised per-head key [k_nope ; k_rope] (the pages leave it open)."""
    return 1.0 / np.sqrt(cfg.d_nope + cfg.d_r)


def attention_core(q, K, V, mask, scale: float):
    """Textbook masked softmax attention.  A row with no visible key gives a
    zero output and log-sum-exp -inf."""
    s = (q @ K.T) * scale
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    safe_l = np.where(l > 0, l, 1.0)
    P = p / safe_l
    lse = np.where(l[:, 0] > 0, m[:, 0] + np.log(safe_l[:, 0]), -np.inf)
    return P @ V, P, lse


def materialize_head(cfg, cache_values_b, w_uk, w_uv, h: int):
    """K_h = [c W_UK_h^T ; k_rope] and V_h = c W_UV_h^T over all slots."""
    C = cache_values_b[:, :cfg.d_c]
    KR = cache_values_b[:, cfg.d_c:]
    K = np.concatenate([C @ w_uk[h], KR], axis=-1)
    V = C @ w_uv[h].T
    return K, V


def attend(cfg, st, q_nope, q_rope_rot, w_uk, w_uv, q_first: int, tokens=None, heads=None):
    """Per-head attention over the cache with materialised K/V.

    ``tokens``: optional list of (b, t) query tokens to evaluate; default:
    every query token.  ``heads``: optional list of heads to evaluate
    (default all; the others stay zero).  Returns o_heads [N, H, d_v], o_lat
    [N, H, d_c] (= sum_s p_s c_s with the same probabilities) and lse [N, H],
    where N is B * n_q in (b, t) order, or len(tokens).
    """
    B, H = cfg.batch, cfg.n_heads
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    q_nope = np.asarray(q_nope, np.float64)
    if tokens is None:
        tokens = [(b, t) for b in range(B) for t in range(cfg.n_q)]
    tokens = list(tokens)
    mask_all = mask_matrix(cfg, q_first, st["newest"])
    o_heads = np.zeros((len(tokens), H, cfg.d_v))
    o_lat = np.zeros((len(tokens), H, cfg.d_c))
    lse = np.zeros((len(tokens), H))
    for b in sorted({b for b, _ in tokens}):
        idx = [i for i, (bb, _) in enumerate(tokens) if bb == b]
        ts = np.array([tokens[i][1] for i in idx])
        C = st["values"][b, :, :cfg.d_c]
        mask = mask_all[ts]
        for h in (range(H) if heads is None else heads):
            K, V = materialize_head(cfg, st["values"][b], w_uk, w_uv, h)
            Q = np.concatenate([q_nope[b, ts, h], q_rope_rot[b, ts, h]], axis=-1)
            o, P, l = attention_core(Q, K, V, mask, softmax_scale(cfg))
            o_heads[idx, h] = o
            o_lat[idx, h] = P @ C
            lse[idx, h] = l
    return o_heads, o_lat, lse


# ---------------------------------------------------------------------------
# QK normalisation: [MLA topics, QK-Norm abstract]: RMSNorm of the projected
# query and key splits into a static per-dimension weight and one dynamic RMS
# statistic; in MLA every head's key comes from the one cached latent, so the
# key statistic is one scalar per token (one KV group).
# Reading: the norm covers the content part of the projected query, and of
# the projected key, of all heads together (H * d_nope values per token),
# with eps inside the root; the decoupled rotary parts are not normalised;
# the key is projected from the stored latent (what attention reads).
# ---------------------------------------------------------------------------
def rms_normalise(v, g, eps: float):
    """g * v / sqrt(mean(v^2) + eps) over the last two axes [.., H, d_nope]."""
    v = np.asarray(v, np.float64)
    d = np.sqrt(np.mean(v * v, axis=(-2, -1), keepdims=True) + eps)
    return np.asarray(g, np.float64) * v / np.where(d > 0, d, 1.0)   # (an all-zero v stays zero)


def attend_qk_norm(cfg, st, q_nope, q_rope_rot, w_uk, w_uv, g_q, g_k, eps: float, q_first: int,
                   tokens=None):
    """Per-head attention with explicit post-projection QK RMSNorm: every
    head's content key k_h = W^UK_h c and content query are normalised as
    above (weights g_q, g_k [H, d_nope]), joined with the unnormalised rotary
    parts, and attend with the textbook softmax.  Same outputs as ``attend``."""
    B, H = cfg.batch, cfg.n_heads
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    if tokens is None:
        tokens = [(b, t) for b in range(B) for t in range(cfg.n_q)]
    tokens = list(tokens)
    mask_all = mask_matrix(cfg, q_first, st["newest"])
    o_heads = np.zeros((len(tokens), H, cfg.d_v))
    o_lat = np.zeros((len(tokens), H, cfg.d_c))
    lse = np.zeros((len(tokens), H))
    for b in sorted({b for b, _ in tokens}):
        idx = [i for i, (bb, _) in enumerate(tokens) if bb == b]
        ts = np.array([tokens[i][1] for i in idx])
        C = st["values"][b, :, :cfg.d_c]
        KR = st["values"][b, :, cfg.d_c:]
        k_all = rms_normalise(np.matmul(C, w_uk).transpose(1, 0, 2), g_k, eps)  # [S, H, d_nope]
        q_all = rms_normalise(np.asarray(q_nope, np.float64)[b, ts], g_q, eps)  # [T, H, d_nope]
        mask = mask_all[ts]
        for h in range(H):
            K = np.concatenate([k_all[:, h], KR], axis=-1)
            V = C @ w_uv[h].T
            Q = np.concatenate([q_all[:, h], q_rope_rot[b, ts, h]], axis=-1)
            o, P, l = attention_core(Q, K, V, mask, softmax_scale(cfg))
            o_heads[idx, h] = o
            o_lat[idx, h] = P @ C
            lse[idx, h] = l
    return o_heads, o_lat, lse


# ---------------------------------------------------------------------------
# output: [MLA concept, Low-rank joint compression] (W^UV folds into the output
# projection) and [MLA explainer, On-the-Fly Reconstruction]
# ---------------------------------------------------------------------------
def output_projection(o_heads, w_o) -> np.ndarray:
    """y = concat_h(o_h) . w_o^T;  o_heads [..., H, d_v] -> [..., d_model]."""
    o = np.asarray(o_heads, np.float64)
    return o.reshape(o.shape[:-2] + (-1,)) @ np.asarray(w_o, np.float64).T


def unabsorb(o_lat, w_uv, w_o):
    """Definition of the un-absorb step from a given latent output:
    o_h = W^UV_h o_lat,h, then y = concat_h(o_h) . w_o^T."""
    o_heads = np.einsum("...hj,hvj->...hv", np.asarray(o_lat, np.float64), np.asarray(w_uv, np.float64))
    return o_heads, output_projection(o_heads, w_o)


# ---------------------------------------------------------------------------
# whole workload
# ---------------------------------------------------------------------------
def build_cache(cfg, inp) -> dict:
    st = new_cache(cfg)
    if cfg.cache_given:
        given_cache(st, cfg, inp["cache_c"], inp["cache_r"])
        append_frame(st, cfg, as_f64(inp["x_new"])[:, 0], as_f64(inp["w_dkr"]), cfg.n_frames - 1)
    else:
        x = as_f64(inp["x"])
        w = as_f64(inp["w_dkr"])
        for f in range(cfg.n_frames):
            append_frame(st, cfg, x[:, f], w, f)
    return st


def run(cfg, inp, tokens=None, st=None) -> dict:
    """Every intermediate the GPU path exposes, in float64.

    Returns cache state, q_abs [B, n_q, H, d_qk] (all tokens), and for the
    evaluated tokens: o_lat, lse, o_heads and y.
    """
    if st is None:
        st = build_cache(cfg, inp)
    w_uk, w_uv, w_o = as_f64(inp["w_uk"]), as_f64(inp["w_uv"]), as_f64(inp["w_o"])
    q_nope, q_rope = as_f64(inp["q_nope"]), as_f64(inp["q_rope"])
    q_abs = absorb_query(cfg, q_nope, q_rope, w_uk, cfg.q_first)
    q_rope_rot = q_abs[..., cfg.d_c:]
    o_heads, o_lat, lse = attend(cfg, st, q_nope, q_rope_rot, w_uk, w_uv, cfg.q_first, tokens)
    y = output_projection(o_heads, w_o)
    return {"cache": st, "q_abs": q_abs, "o_lat": o_lat, "lse": lse,
            "o_heads": o_heads, "y": y}
