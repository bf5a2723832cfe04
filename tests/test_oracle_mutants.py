"""Plants plausible mistakes into the CPU oracle and checks that the pins catch
each one.  This is evidence that the pins bind every part of the oracle, not
only that the oracle agrees with itself.  Runs on the CPU; the mistakes live
only inside the monkeypatched oracle of this test process."""
import numpy as np
import pytest

import oracle.int4 as oi
import oracle.mla as om
import pins

_orig = {
    "rope_rotate": om.rope_rotate, "rope_frequencies": om.rope_frequencies,
    "token_coords": om.token_coords, "visible": om.visible, "slot_frames": om.slot_frames,
    "query_frames": om.query_frames, "attention_core": om.attention_core,
    "materialize_head": om.materialize_head, "output_projection": om.output_projection,
    "absorb_query": om.absorb_query, "round_bf16": om.round_bf16,
    "softmax_scale": om.softmax_scale, "query_coords": om.query_coords,
    "quantize_groups": oi.quantize_groups, "pack_nibbles": oi.pack_nibbles,
    "unpack_nibbles": oi.unpack_nibbles, "pack_crumbs": oi.pack_crumbs, "unpack_crumbs": oi.unpack_crumbs,
    "rope_shift": om.rope_shift, "fold_query_weights": om.fold_query_weights, "query_up": om.query_up,
    "rms_normalise": om.rms_normalise, "attend_qk_norm": om.attend_qk_norm,
    "admissible_groups": oi.admissible_groups, "bf16_bracket": om.bf16_bracket,
}


def _rms_per_head(v, g, eps):
    v = np.asarray(v, np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):   # 0 / 0 where a pin passes eps = 0 with zero rows
        return np.asarray(g, np.float64) * v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def _rms_eps_outside(v, g, eps):
    v = np.asarray(v, np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.asarray(g, np.float64) * v / (np.sqrt(np.mean(v * v, axis=(-2, -1), keepdims=True)) + eps)


def _qkn_key_weight_dropped(cfg, st, q_nope, q_rope_rot, w_uk, w_uv, g_q, g_k, eps, q_first, tokens=None):
    return _orig["attend_qk_norm"](cfg, st, q_nope, q_rope_rot, w_uk, w_uv, g_q, np.ones_like(g_k), eps,
                                   q_first, tokens)


def _fold_heads_interleaved(cfg, w_uq, w_uk):
    wq = np.asarray(w_uq, np.float64).reshape(cfg.d_nope, cfg.n_heads, -1).transpose(1, 0, 2)
    return np.matmul(np.asarray(w_uk, np.float64), wq)


def _fold_uk_transposed_inner(cfg, w_uq, w_uk):
    wk = np.asarray(w_uk, np.float64)
    wq = np.asarray(w_uq, np.float64).reshape(cfg.n_heads, cfg.d_nope, -1)
    return np.matmul(wk[..., ::-1], wq)


def _query_up_heads_interleaved(cfg, c_q, w_uq):
    q = np.asarray(c_q, np.float64) @ np.asarray(w_uq, np.float64).T
    return q.reshape(q.shape[:-1] + (cfg.d_nope, cfg.n_heads)).swapaxes(-1, -2)


def _shift_backwards(st, cfg, delta, slot_begin, n_slots):
    _orig["rope_shift"](st, cfg, -np.asarray(delta), slot_begin, n_slots)


def _shift_axes_reversed(st, cfg, delta, slot_begin, n_slots):
    _orig["rope_shift"](st, cfg, np.asarray(delta).reshape(-1, 3)[:, ::-1], slot_begin, n_slots)


def _shift_one_slot_late(st, cfg, delta, slot_begin, n_slots):
    _orig["rope_shift"](st, cfg, delta, slot_begin + 1, n_slots)


def _shift_codes_kept(st, cfg, delta, slot_begin, n_slots):
    keep = {k: st[k].copy() for k in ("codes", "rscale") if k in st}
    _orig["rope_shift"](st, cfg, delta, slot_begin, n_slots)
    st.update(keep)


def _rope_sign(u, coords, cfg):
    return _orig["rope_rotate"](u, -np.asarray(coords, np.float64), cfg)


def _rope_freq(band, theta):
    i = np.arange(band // 2, dtype=np.float64)
    return theta ** (-i / band)


def _coords_hw_swap(cfg, frame, tok):
    c = _orig["token_coords"](cfg, frame, tok)
    if cfg.rope_dims == 3:
        c = c[..., [0, 2, 1]]
    return c


def _visible_le(cfg, f_q, f_k):
    f_q, f_k = np.asarray(f_q), np.asarray(f_k)
    fpb = cfg.frames_per_block
    return (f_k >= 0) & (f_k // fpb <= f_q // fpb) & (f_q - f_k <= cfg.window)


def _visible_not_causal(cfg, f_q, f_k):
    f_q, f_k = np.asarray(f_q), np.asarray(f_k)
    return (f_k >= 0) & (np.abs(f_q - f_k) < cfg.window)


def _slot_frames_off(cfg, newest):
    return _orig["slot_frames"](cfg, newest + 1)


def _query_frames_token(cfg, q_first):
    return q_first + np.arange(cfg.n_q) // max(1, cfg.tokens_per_frame // 2)


def _no_lse_max(q, K, V, mask, scale):
    o, P, lse = _orig["attention_core"](q, K, V, mask, scale)
    s = np.where(mask, (q @ K.T) * scale, -np.inf)
    m = np.where(np.isfinite(s.max(axis=1)), s.max(axis=1), 0.0)
    return o, P, np.where(np.isfinite(lse), lse - m, lse)


def _no_mask(q, K, V, mask, scale):
    return _orig["attention_core"](q, K, V, np.ones_like(mask), scale)


def _wrong_value_head(cfg, cache_b, w_uk, w_uv, h):
    K, _ = _orig["materialize_head"](cfg, cache_b, w_uk, w_uv, h)
    _, V = _orig["materialize_head"](cfg, cache_b, w_uk, w_uv, (h + 1) % cfg.n_heads)
    return K, V


def _wrong_key_head(cfg, cache_b, w_uk, w_uv, h):
    _, V = _orig["materialize_head"](cfg, cache_b, w_uk, w_uv, h)
    K, _ = _orig["materialize_head"](cfg, cache_b, w_uk, w_uv, (h + 1) % cfg.n_heads)
    return K, V


def _wo_untransposed(o_heads, w_o):
    o = np.asarray(o_heads, np.float64)
    w = np.asarray(w_o, np.float64)
    if w.shape[0] == w.shape[1]:
        return o.reshape(o.shape[:-2] + (-1,)) @ w
    return _orig["output_projection"](o_heads, w_o)


def _absorb_wrong_head(cfg, q_nope, q_rope, w_uk, q_first):
    return _orig["absorb_query"](cfg, q_nope, q_rope, np.roll(np.asarray(w_uk), 1, axis=0), q_first)


def _bf16_truncate(a):
    a = np.asarray(a, np.float64)
    _, e = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.trunc(a / step) * step


def _scale_nope_only(cfg):
    return 1.0 / np.sqrt(cfg.d_nope)


def _query_coords_shift(cfg, q_first):
    return _orig["query_coords"](cfg, q_first + 1)


def _half_away(x, group, bits=4):
    qmax, qmin = 2 ** (bits - 1) - 1, -2 ** (bits - 1)
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (n // group, group))
    s16 = (np.max(np.abs(g), axis=-1) / np.float32(qmax)).astype(np.float16)
    s = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.sign(g / s) * np.floor(np.abs(g / s) + np.float32(0.5))
    q = np.where(s == 0, 0, q)
    return np.clip(q, qmin, qmax).astype(np.int8).reshape(x.shape), s16


def _scale_one_more(x, group, bits=4):
    # scale amax / (qmax + 1): 8 for INT4, 2 for INT2
    qmax, qmin = 2 ** (bits - 1) - 1, -2 ** (bits - 1)
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (n // group, group))
    s16 = (np.max(np.abs(g), axis=-1) / np.float32(qmax + 1)).astype(np.float16)
    s = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(g / s)
    q = np.where(s == 0, 0, q)
    return np.clip(q, qmin, qmax).astype(np.int8).reshape(x.shape), s16


def _only_int2(fn):
    # a mistake in the INT2 path only (INT4 calls pass through)
    def wrapped(x, group, bits=4):
        return fn(x, group, bits) if bits == 2 else _orig["quantize_groups"](x, group)
    return wrapped


def _crumbs_reversed_pack(codes):
    c = np.asarray(codes).astype(np.int16)
    out = np.zeros(c.shape[:-1] + (c.shape[-1] // 4,), dtype=np.int16)
    for k in range(4):
        out |= (c[..., k::4] & 0x3) << (2 * (3 - k))
    return out.astype(np.uint8)


def _crumbs_reversed_unpack(packed):
    out = _orig["unpack_crumbs"](packed)
    return out.reshape(out.shape[:-1] + (-1, 4))[..., ::-1].reshape(out.shape)


def _pack_swapped(codes):
    c = np.asarray(codes).astype(np.int16)
    return ((c[..., 1::2] & 0xF) | ((c[..., 0::2] & 0xF) << 4)).astype(np.uint8)


def _unpack_swapped(packed):
    out = _orig["unpack_nibbles"](packed)
    return out.reshape(out.shape[:-1] + (-1, 2))[..., ::-1].reshape(out.shape)


def _admissible_no_zero_groups(lo, hi, group, bits=4):
    # forgets that a group which may be all zero may take a tiny scale
    lo32, hi32 = np.asarray(lo, np.float32), np.asarray(hi, np.float32)
    shp = lo32.shape[:-1] + (lo32.shape[-1] // group, group)
    glo, ghi = lo32.reshape(shp), hi32.reshape(shp)
    small = np.where((glo <= 0) & (ghi >= 0), np.float32(0), np.minimum(np.abs(glo), np.abs(ghi)))
    big = np.maximum(np.abs(glo), np.abs(ghi))
    s_min = oi.group_scale(np.max(small, axis=-1), bits)
    s_max = oi.group_scale(np.max(big, axis=-1), bits)
    cands = [oi.codes_for(x, s[..., None], bits) for x in (glo, ghi) for s in (s_min, s_max)]
    return (np.minimum.reduce(cands).reshape(lo32.shape), np.maximum.reduce(cands).reshape(lo32.shape),
            s_min, s_max)


def _admissible_scale_fixed(lo, hi, group, bits=4):
    # takes the scale of the lower interval ends as the only one
    cmin, cmax, s_min, _ = _orig["admissible_groups"](lo, hi, group, bits)
    q, s = oi.quantize_groups(lo, group, bits)
    return np.minimum(cmin, q), np.maximum(cmin, q), s_min, s


def _bracket_nearest_only(a):
    r = om.round_bf16(a)
    return r, r


MUTANTS = {
    "rope_rotates_backwards": [(om, "rope_rotate", _rope_sign)],
    "rope_frequency_exponent": [(om, "rope_frequencies", _rope_freq)],
    "rope_axes_swapped": [(om, "token_coords", _coords_hw_swap)],
    "window_off_by_one": [(om, "visible", _visible_le)],
    "mask_not_causal": [(om, "visible", _visible_not_causal)],
    "ring_frames_off_by_one": [(om, "slot_frames", _slot_frames_off)],
    "query_frame_index": [(om, "query_frames", _query_frames_token)],
    "lse_without_max": [(om, "attention_core", _no_lse_max)],
    "mask_ignored": [(om, "attention_core", _no_mask)],
    "value_from_other_head": [(om, "materialize_head", _wrong_value_head)],
    "key_from_other_head": [(om, "materialize_head", _wrong_key_head)],
    "output_weight_untransposed": [(om, "output_projection", _wo_untransposed)],
    "absorb_other_head": [(om, "absorb_query", _absorb_wrong_head)],
    "bf16_truncates": [(om, "round_bf16", _bf16_truncate)],
    "softmax_scale_nope_only": [(om, "softmax_scale", _scale_nope_only)],
    "query_rotated_at_next_frame": [(om, "query_coords", _query_coords_shift)],
    "int4_ties_away_from_zero": [(oi, "quantize_groups", _half_away)],
    "int4_scale_amax_over_8": [(oi, "quantize_groups", _scale_one_more)],
    "int2_ties_away_from_zero": [(oi, "quantize_groups", _only_int2(_half_away))],
    "int2_scale_amax_over_2": [(oi, "quantize_groups", _only_int2(_scale_one_more))],
    "int2_crumbs_reversed": [(oi, "pack_crumbs", _crumbs_reversed_pack),
                             (oi, "unpack_crumbs", _crumbs_reversed_unpack)],
    "int4_nibbles_swapped": [(oi, "pack_nibbles", _pack_swapped), (oi, "unpack_nibbles", _unpack_swapped)],
    "rope_shift_backwards": [(om, "rope_shift", _shift_backwards)],
    "rope_shift_axes_reversed": [(om, "rope_shift", _shift_axes_reversed)],
    "rope_shift_slot_range_off_by_one": [(om, "rope_shift", _shift_one_slot_late)],
    "rope_shift_low_bit_codes_kept": [(om, "rope_shift", _shift_codes_kept)],
    "fold_heads_interleaved": [(om, "fold_query_weights", _fold_heads_interleaved)],
    "fold_inner_index_reversed": [(om, "fold_query_weights", _fold_uk_transposed_inner)],
    "query_up_heads_interleaved": [(om, "query_up", _query_up_heads_interleaved)],
    "qk_norm_per_head_rms": [(om, "rms_normalise", _rms_per_head)],
    "qk_norm_eps_outside_root": [(om, "rms_normalise", _rms_eps_outside)],
    "qk_norm_key_weight_dropped": [(om, "attend_qk_norm", _qkn_key_weight_dropped)],
    "admissible_codes_no_zero_groups": [(oi, "admissible_groups", _admissible_no_zero_groups)],
    "admissible_scale_of_low_ends": [(oi, "admissible_groups", _admissible_scale_fixed)],
    "bf16_bracket_nearest_only": [(om, "bf16_bracket", _bracket_nearest_only)],
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    for mod, attr, fn in MUTANTS[name]:
        monkeypatch.setattr(mod, attr, fn)
    res = pins.run_checks(stop_at_first_failure=True)
    failed = [n for n, (err, tol, _) in res.items() if not err <= tol]
    assert failed, f"planted mistake {name} passed every pin"
