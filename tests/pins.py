"""Pins of the CPU oracle against things other than itself.

Each ``check_*`` returns an error figure that must stay below its tolerance
(``CHECKS`` maps name -> (function, tolerance)).  ``test_oracle_pins.py``
asserts that all of them pass; ``test_oracle_mutants.py`` plants plausible
mistakes into the oracle and asserts that every mistake trips at least one.

Kinds of pin used here:
  * brute force: pure-Python scalar loops (complex-number rotation, a deque as
    the sliding window, explicit sums) on tiny workloads;
  * identities: absorption of W^UK into the query and of W^UV into the
    output ("Multi-Head Latent Attention" concept page, Low-rank joint
    compression); content + rotary score decomposition (same page, The RoPE
    problem, and the decoupled fix);
  * rotary invariants: norm preservation, R(0) = I, R(a)R(b) = R(a+b),
    dependence of scores on the offset only, 3D reducing to 1D;
  * closed forms: zero query -> mean of visible values and lse = ln(n);
    a single visible key; fully masked rows;
  * library routines: torch scaled_dot_product_attention, scipy softmax,
    torch's float32 -> bfloat16 and float32 -> float16 conversions.
"""
from __future__ import annotations

import cmath
import math
from collections import deque

import numpy as np

import oracle.int4 as oi
import oracle.mla as om
from mla_inputs import MLAConfig, make_workload

# ---------------------------------------------------------------------------
# tiny workloads for brute force
# ---------------------------------------------------------------------------
TINIER = MLAConfig(
    name="tinier", batch=2, n_heads=2, d_model=8, d_nope=4, d_v=4, d_c=6, d_r=6,
    rope_dims=3, bands=(2, 2, 2), theta=10000.0, grid_h=2, grid_w=2, window=2,
    frames_per_block=1, n_frames=3, q_first=1, q_frames=2, dtype="bf16")
TINIER_BLOCK = TINIER.replace(name="tinier_block", window=3, frames_per_block=2,
                              n_frames=4, q_first=2, q_frames=2, dtype="f32")
TINY_DECODE = MLAConfig(
    name="tiny_decode", batch=2, n_heads=2, d_model=8, d_nope=4, d_v=4, d_c=6, d_r=4,
    rope_dims=1, bands=(4,), theta=10000.0, grid_h=1, grid_w=1, window=8,
    frames_per_block=1, n_frames=6, q_first=5, q_frames=1, dtype="bf16", cache_given=True)
TINY_INT4 = MLAConfig(
    name="tiny_int4", batch=1, n_heads=2, d_model=16, d_nope=4, d_v=4, d_c=64, d_r=8,
    rope_dims=3, bands=(2, 2, 4), theta=10000.0, grid_h=2, grid_w=2, window=2,
    frames_per_block=1, n_frames=3, q_first=2, q_frames=1, dtype="bf16", cache_fmt="int4")


def _tiny_video():
    from mla_inputs import CONFIGS
    return CONFIGS[1]


TINY_INT2 = TINY_INT4.replace(name="tiny_int2", cache_fmt="int2")

BRUTE_CASES = [_tiny_video, lambda: TINIER, lambda: TINIER_BLOCK, lambda: TINY_DECODE,
               lambda: TINY_INT4, lambda: TINY_INT2]


# ---------------------------------------------------------------------------
# brute force (scalar Python)
# ---------------------------------------------------------------------------
def _round_scalar(v: float, dtype: str) -> float:
    if dtype == "f32":
        return float(np.float32(v))
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)              # v = m 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256.0), e - 8)   # round(): ties to even


def _bf_rotate(vec, coords, bands, theta):
    out = list(vec)
    off = 0
    for axis, band in enumerate(bands):
        for i in range(band // 2):
            freq = theta ** (-(2.0 * i) / band)
            z = complex(vec[off + 2 * i], vec[off + 2 * i + 1]) * cmath.exp(1j * coords[axis] * freq)
            out[off + 2 * i], out[off + 2 * i + 1] = z.real, z.imag
        off += band
    return out


def _bf_coords(cfg, frame, tok):
    if cfg.rope_dims == 3:
        return (frame, tok // cfg.grid_w, tok % cfg.grid_w)
    return (frame * cfg.tokens_per_frame + tok,)


def _bf_lowbit(vals, bits=4):
    qmax, qmin = 2 ** (bits - 1) - 1, -2 ** (bits - 1)
    amax = max(abs(v) for v in vals)
    s = float(np.float16(np.float32(amax) / np.float32(qmax)))
    if s == 0.0:
        return [0.0] * len(vals)
    out = []
    for v in vals:
        q = float(np.float32(v) / np.float32(s))
        r = round(q)                      # ties to even
        r = max(qmin, min(qmax, r))
        out.append(r * s)
    return out


def brute_force(cfg, inp):
    """Returns per query token (b, t): y [d_model], o_heads [H][d_v],
    o_lat [H][d_c], lse [H]; and the stored row of every (b, frame, tok)."""
    g = {k: om.as_f64(v).tolist() for k, v in inp.items()}
    B, H, P, W = cfg.batch, cfg.n_heads, cfg.tokens_per_frame, cfg.window
    dc, dr = cfg.d_c, cfg.d_r
    scale = 1.0 / math.sqrt(cfg.d_nope + cfg.d_r)
    rows_out = {}
    results = {}
    for b in range(B):
        ring = deque(maxlen=W)            # (frame, [row per token])
        for f in range(cfg.n_frames):
            rows = []
            for tok in range(P):
                if cfg.cache_given and f < cfg.n_frames - 1:
                    row = g["cache_c"][b][f * P + tok] + g["cache_r"][b][f * P + tok]
                else:
                    xv = g["x_new"][b][0][tok] if cfg.cache_given else g["x"][b][f][tok]
                    yv = [sum(g["w_dkr"][n][k] * xv[k] for k in range(cfg.d_model))
                          for n in range(dc + dr)]
                    row = yv[:dc] + _bf_rotate(yv[dc:], _bf_coords(cfg, f, tok), cfg.bands, cfg.theta)
                row = [_round_scalar(v, cfg.dtype) for v in row]
                if cfg.cache_fmt in ("int4", "int2"):
                    c = []
                    for gi in range(0, dc, 32):
                        c += _bf_lowbit(row[gi:gi + 32], 4 if cfg.cache_fmt == "int4" else 2)
                    row = c + _bf_lowbit(row[dc:], 4)
                rows.append(row)
                rows_out[(b, f, tok)] = row
            ring.append((f, rows))
        # materialise per-head content keys and values of every ring token once
        kv = {}
        for h in range(H):
            for fk, rows in ring:
                for tok, row in enumerate(rows):
                    c = row[:dc]
                    kn = [sum(g["w_uk"][h][j][a] * c[j] for j in range(dc)) for a in range(cfg.d_nope)]
                    vv = [sum(g["w_uv"][h][v][j] * c[j] for j in range(dc)) for v in range(cfg.d_v)]
                    kv[(h, fk, tok)] = (kn, vv)
        for i in range(cfg.n_q):
            fq, tq = cfg.q_first + i // P, i % P
            o_heads, o_lat, lse = [], [], []
            for h in range(H):
                qn = g["q_nope"][b][i][h]
                qr = _bf_rotate(g["q_rope"][b][i][h], _bf_coords(cfg, fq, tq), cfg.bands, cfg.theta)
                keys = []
                for fk, rows in ring:
                    if fk // cfg.frames_per_block <= fq // cfg.frames_per_block and fq - fk < W:
                        keys.extend((row, kv[(h, fk, tok)]) for tok, row in enumerate(rows))
                scores = []
                for row, (kn, _) in keys:
                    kr = row[dc:]
                    s = sum(qn[a] * kn[a] for a in range(cfg.d_nope)) + sum(qr[a] * kr[a] for a in range(dr))
                    scores.append(s * scale)
                if not scores:
                    o_heads.append([0.0] * cfg.d_v)
                    o_lat.append([0.0] * dc)
                    lse.append(-math.inf)
                    continue
                mx = max(scores)
                e = [math.exp(s - mx) for s in scores]
                tot = sum(e)
                p = [v / tot for v in e]
                lse.append(mx + math.log(tot))
                ov = [0.0] * cfg.d_v
                ol = [0.0] * dc
                for pk, (row, (_, vv)) in zip(p, keys):
                    for v in range(cfg.d_v):
                        ov[v] += pk * vv[v]
                    for j in range(dc):
                        ol[j] += pk * row[j]
                o_heads.append(ov)
                o_lat.append(ol)
            yv = [sum(o_heads[h][v] * g["w_o"][n][h * cfg.d_v + v]
                      for h in range(H) for v in range(cfg.d_v)) for n in range(cfg.d_model)]
            results[(b, i)] = {"y": yv, "o_heads": o_heads, "o_lat": o_lat, "lse": lse}
    return results, rows_out


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    fin = np.isfinite(b)
    if not np.array_equal(np.isfinite(a), fin) or not np.array_equal(a[~fin], b[~fin]):
        return np.inf
    return float(np.max(np.abs(a[fin] - b[fin]) / (1.0 + np.abs(b[fin])), initial=0.0))


def check_bruteforce(case=None):
    errs = []
    cases = BRUTE_CASES if case is None else [case]
    for mk in cases:
        cfg = mk()
        inp = make_workload(cfg, seed=3)
        ref, rows = brute_force(cfg, inp)
        out = om.run(cfg, inp)
        st = out["cache"]
        for (b, f, tok), row in rows.items():
            if cfg.cache_given or f > cfg.newest - cfg.window:
                slot = int(om.slot_index(cfg, f, tok))
                errs.append(_rel(st["values"][b, slot], row))
        for n, ((b, i), r) in enumerate(sorted(ref.items())):
            for key in ("y", "o_heads", "o_lat", "lse"):
                errs.append(_rel(out[key][n], r[key]))
    return max(errs)


# ---------------------------------------------------------------------------
# identities
# ---------------------------------------------------------------------------
def check_absorption():
    """Materialised-key scores equal absorbed scores q_abs . [c | k_rope]."""
    errs = []
    for cfg in (TINIER, TINY_DECODE, _tiny_video()):
        inp = make_workload(cfg, seed=5)
        st = om.build_cache(cfg, inp)
        w_uk, w_uv = om.as_f64(inp["w_uk"]), om.as_f64(inp["w_uv"])
        q_nope, q_rope = om.as_f64(inp["q_nope"]), om.as_f64(inp["q_rope"])
        q_abs = om.absorb_query(cfg, q_nope, q_rope, w_uk, cfg.q_first)
        for b in range(cfg.batch):
            for h in range(cfg.n_heads):
                K, _ = om.materialize_head(cfg, st["values"][b], w_uk, w_uv, h)
                Q = np.concatenate([q_nope[b, :, h], q_abs[b, :, h, cfg.d_c:]], axis=-1)
                s_mat = Q @ K.T
                s_abs = q_abs[b, :, h] @ st["values"][b].T
                errs.append(np.max(np.abs(s_mat - s_abs)) / (1 + np.max(np.abs(s_abs))))
    return max(errs)


def check_value_fold():
    """sum_s p_s (W^UV_h c_s) == W^UV_h (sum_s p_s c_s), and y from either."""
    errs = []
    for cfg in (TINIER, TINY_DECODE, _tiny_video()):
        inp = make_workload(cfg, seed=6)
        out = om.run(cfg, inp)
        o_heads, y = om.unabsorb(out["o_lat"], om.as_f64(inp["w_uv"]), om.as_f64(inp["w_o"]))
        errs.append(_rel(o_heads, out["o_heads"]))
        errs.append(_rel(y, out["y"]))
    return max(errs)


# ---------------------------------------------------------------------------
# rotary invariants
# ---------------------------------------------------------------------------
_R3 = MLAConfig(name="r3", batch=1, n_heads=1, d_model=8, d_nope=4, d_v=4, d_c=8, d_r=16,
                rope_dims=3, bands=(4, 6, 6), theta=10000.0, grid_h=4, grid_w=4, window=3,
                frames_per_block=1, n_frames=3, q_first=0, q_frames=1, dtype="f32")
_R1 = _R3.replace(name="r1", rope_dims=1, bands=(16,), grid_h=1, grid_w=1)


def _rot(cfg, u, coords):
    return om.rope_rotate(u, np.asarray(coords, np.float64), cfg)


def check_rope_invariants():
    rng = np.random.default_rng(11)
    errs = []
    for cfg in (_R3, _R1):
        nd = cfg.rope_dims
        u = rng.standard_normal((50, cfg.d_r))
        v = rng.standard_normal((50, cfg.d_r))
        a = rng.uniform(-300, 300, (50, nd))
        bb = rng.uniform(-300, 300, (50, nd))
        d = rng.uniform(-300, 300, (50, nd))
        ru = _rot(cfg, u, a)
        errs.append(np.max(np.abs(np.linalg.norm(ru, axis=1) - np.linalg.norm(u, axis=1))))
        errs.append(np.max(np.abs(_rot(cfg, u, np.zeros((50, nd))) - u)))
        errs.append(np.max(np.abs(_rot(cfg, _rot(cfg, u, a), bb) - _rot(cfg, u, a + bb))) / 10)
        s0 = np.sum(_rot(cfg, u, a) * _rot(cfg, v, bb), axis=1)
        s1 = np.sum(_rot(cfg, u, a + d) * _rot(cfg, v, bb + d), axis=1)
        errs.append(np.max(np.abs(s0 - s1)) / 10)
    # 3D with h = w = 0 acts as 1D rotary on the t band and identity elsewhere
    t_only = _R3.replace(name="t", rope_dims=1, bands=(4,), d_r=4)
    u = rng.standard_normal((20, 16))
    t = rng.uniform(0, 100, (20, 1))
    r3 = _rot(_R3, u, np.concatenate([t, np.zeros((20, 2))], axis=1))
    errs.append(np.max(np.abs(r3[:, :4] - _rot(t_only, u[:, :4], t))))
    errs.append(np.max(np.abs(r3[:, 4:] - u[:, 4:])))
    return float(max(errs))


def check_rope_worked_values():
    """Closed forms: band width 2 rotates by the position in radians; a band of
    width 4 with theta = 1e4 has frequencies 1 and 1e-2."""
    errs = []
    c2 = _R1.replace(name="w2", bands=(2,), d_r=2)
    out = _rot(c2, np.array([[1.0, 0.0]]), [[0.7]])
    errs.append(np.max(np.abs(out - [[math.cos(0.7), math.sin(0.7)]])))
    c4 = _R1.replace(name="w4", bands=(4,), d_r=4)
    out = _rot(c4, np.array([[0.0, 1.0, 1.0, 0.0]]), [[100.0]])
    want = [-math.sin(100.0), math.cos(100.0), math.cos(1.0), math.sin(1.0)]
    errs.append(np.max(np.abs(out - [want])))
    # 3D band order t | h | w: coordinate (0, 0, w) touches only the last band
    out = _rot(_R3, np.ones((1, 16)), [[0.0, 0.0, 1.0]])
    errs.append(np.max(np.abs(out[0, :10] - 1.0)))
    errs.append(abs(out[0, 10] - (math.cos(1.0) - math.sin(1.0))))
    return float(max(errs))


# ---------------------------------------------------------------------------
# softmax / mask special cases
# ---------------------------------------------------------------------------
def check_mask_enumeration():
    errs = 0
    for cfg in (TINIER, TINIER_BLOCK, TINY_DECODE, _tiny_video(),
                TINIER.replace(name="nowrap", n_frames=2, q_first=0, q_frames=2),
                TINIER.replace(name="w5", window=5, n_frames=3, q_first=0, q_frames=3)):
        sf = om.slot_frames(cfg, cfg.newest)
        present = set(range(max(0, cfg.n_frames - cfg.window), cfg.n_frames))
        # every present frame owns exactly P slots and every slot holds a present frame or -1
        for f in present:
            errs += int(np.sum(sf == f) != cfg.tokens_per_frame)
        errs += int(np.any([(v != -1 and v not in present) for v in sf]))
        # round trip: the slot of (f, tok) holds f
        for f in present:
            for tok in range(cfg.tokens_per_frame):
                errs += int(sf[int(om.slot_index(cfg, f, tok))] != f)
        # queries at the configured frames, and queries one frame ahead of the
        # newest appended frame (there the window bound removes the oldest frame)
        for q_first in (cfg.q_first, cfg.newest + 1):
            m = om.mask_matrix(cfg, q_first, cfg.newest)
            for i in range(cfg.n_q):
                fq = q_first + i // cfg.tokens_per_frame
                for s in range(cfg.capacity):
                    fk = sf[s]
                    want = (fk in present and fk // cfg.frames_per_block <= fq // cfg.frames_per_block
                            and fq - fk < cfg.window)
                    errs += int(bool(m[i, s]) != want)
    return float(errs)


def check_softmax_closed_forms():
    rng = np.random.default_rng(7)
    errs = []
    S, dk, dv = 37, 12, 5
    K = rng.standard_normal((S, dk))
    V = rng.standard_normal((S, dv))
    mask = rng.random((6, S)) < 0.5
    mask[0] = False
    mask[1] = False
    mask[1, 9] = True
    q = rng.standard_normal((6, dk))
    q[2:] = 0.0
    o, P, lse = om.attention_core(q, K, V, mask, 0.3)
    errs.append(float(np.max(np.abs(o[0]))) + (0.0 if lse[0] == -np.inf else 1.0))
    errs.append(float(np.max(np.abs(o[1] - V[9]))) + abs(lse[1] - 0.3 * q[1] @ K[9]))
    for r in range(2, 6):
        n = mask[r].sum()
        errs.append(float(np.max(np.abs(o[r] - V[mask[r]].mean(axis=0)))))
        errs.append(abs(lse[r] - math.log(n)))
    errs.append(float(np.max(np.abs(P[1:].sum(axis=1) - 1.0))))
    errs.append(float(np.max(P[~mask])))
    return max(errs)


def check_library_attention():
    import scipy.special
    import torch
    rng = np.random.default_rng(8)
    q = rng.standard_normal((9, 20))
    K = rng.standard_normal((31, 20))
    V = rng.standard_normal((31, 7))
    mask = rng.random((9, 31)) < 0.6
    mask[:, 0] = True
    o, P, lse = om.attention_core(q, K, V, mask, 0.25)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=torch.from_numpy(mask)[None], scale=0.25)[0].numpy()
    s = np.where(mask, 0.25 * q @ K.T, -np.inf)
    errs = [np.max(np.abs(o - ref)), np.max(np.abs(P - scipy.special.softmax(s, axis=1))),
            np.max(np.abs(lse - scipy.special.logsumexp(s, axis=1)))]
    return float(max(errs))


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------
def check_bf16_rounding():
    import torch
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    # exact ties: odd multiples of half a bf16 step
    base = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    _, e = np.frexp(base)
    ties = (base + np.ldexp(1.0, e - 9)).astype(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-40, -3e-39, 3.3e38])])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = om.round_bf16(x.astype(np.float64))
    bad = np.sum(got != want)
    # float64 inputs between two bf16 neighbours, away from the tie
    lo = base[:1000]
    step = np.ldexp(1.0, e[:1000] - 8)
    frac = rng.uniform(0.01, 0.49, 1000)
    bad += np.sum(om.round_bf16(lo + frac * step * np.sign(lo)) != lo)
    bad += np.sum(om.round_bf16(lo + (1 - frac) * step * np.sign(lo)) != lo + step * np.sign(lo))
    return float(bad)


# ---------------------------------------------------------------------------
# INT4 quantiser
# ---------------------------------------------------------------------------
def check_int4():
    import torch
    bad = 0
    allb = np.arange(256, dtype=np.uint8)
    bad += int(np.any(oi.pack_nibbles(oi.unpack_nibbles(allb[None]))[0] != allb))
    codes = oi.unpack_nibbles(allb[None])[0]
    bad += int(np.any((codes[0::2] != ((allb & 15).astype(np.int16) ^ 8) - 8)))
    rng = np.random.default_rng(10)
    x = om.round_bf16(rng.standard_normal((400, 64)) * np.exp(rng.uniform(-8, 8, (400, 1))))
    q, s = oi.quantize_groups(x, 32)
    xh = oi.dequantize_groups(q, s, 32)
    s64 = np.repeat(s.astype(np.float64), 32, axis=1)
    bad += int(np.any(np.abs(x - xh) > s64 / 2 * (1 + 1e-12)))
    amax_pos = np.abs(x.reshape(400, 2, 32)).argmax(axis=2)
    qa = np.take_along_axis(q.reshape(400, 2, 32), amax_pos[..., None], 2)[..., 0]
    bad += int(np.any(np.abs(qa) != 7))
    want_s = torch.from_numpy((np.abs(x.reshape(400, 2, 32)).max(axis=2) / 7.0).astype(np.float32)).half().numpy()
    bad += int(np.any(want_s.view(np.uint16) != s.view(np.uint16)))
    # exact multiples of the scale round-trip
    g = np.array([[7.0, -7.0, 3.0, -5.0, 0.0, 1.0] + [0.0] * 26])
    q2, s2 = oi.quantize_groups(g, 32)
    bad += int(float(s2[0, 0]) != 1.0 or np.any(oi.dequantize_groups(q2, s2, 32) != g))
    # ties go to even: scale 1, values k + 0.5
    t = np.array([[7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5] + [0.0] * 24])
    q3, _ = oi.quantize_groups(t, 32)
    bad += int(list(q3[0, :8]) != [7, 0, 2, 2, 0, -2, -2, 4])
    # zero group -> zero scale, zero codes
    q4, s4 = oi.quantize_groups(np.zeros((1, 32)), 32)
    bad += int(np.any(q4 != 0) or float(s4[0, 0]) != 0.0)
    # row storage round trip
    rows = om.round_bf16(rng.standard_normal((5, 3, 72)))
    st = oi.quantize_cache_rows(rows, 64)
    bad += int(np.any(oi.dequantize_cache_rows(st["codes"], st["cscale"], st["rscale"], 64) != st["values"]))
    bad += int(st["codes"].shape[-1] * 1 + st["cscale"].shape[-1] * 2 + 2 != 36 + 4 + 2)
    return float(bad)


# ---------------------------------------------------------------------------
# INT2 content quantiser (the rotary key stays INT4)
# ---------------------------------------------------------------------------
def check_int2():
    import torch
    bad = 0
    allb = np.arange(256, dtype=np.uint8)
    bad += int(np.any(oi.pack_crumbs(oi.unpack_crumbs(allb[None]))[0] != allb))
    codes = oi.unpack_crumbs(allb[None])[0]
    for k in range(4):   # element 4j + k is bits 2k .. 2k + 1, two's complement
        want = (((allb >> (2 * k)) & 3).astype(np.int16) ^ 2) - 2
        bad += int(np.any(codes[k::4] != want))
    rng = np.random.default_rng(11)
    x = om.round_bf16(rng.standard_normal((400, 64)) * np.exp(rng.uniform(-8, 8, (400, 1))))
    q, s = oi.quantize_groups(x, 32, 2)
    xh = oi.dequantize_groups(q, s, 32)
    s64 = np.repeat(s.astype(np.float64), 32, axis=1)
    bad += int(np.any(np.abs(x - xh) > s64 / 2 * (1 + 1e-12)))   # |x / s| <= 1: never clamped
    bad += int(np.any((q < -1) | (q > 1)))
    amax_pos = np.abs(x.reshape(400, 2, 32)).argmax(axis=2)
    qa = np.take_along_axis(q.reshape(400, 2, 32), amax_pos[..., None], 2)[..., 0]
    bad += int(np.any(np.abs(qa) != 1))
    want_s = torch.from_numpy((np.abs(x.reshape(400, 2, 32)).max(axis=2) / 1.0).astype(np.float32)).half().numpy()
    bad += int(np.any(want_s.view(np.uint16) != s.view(np.uint16)))
    # ties go to even: scale 2 (amax 2), values +-1 and +-3 over 2 -> 0, +-2 over 2 -> +-1
    t = np.array([[2.0, 1.0, -1.0, 0.5, -2.0, 1.5] + [0.0] * 26])
    q3, s3 = oi.quantize_groups(t, 32, 2)
    bad += int(float(s3[0, 0]) != 2.0 or list(q3[0, :6]) != [1, 0, 0, 0, -1, 1])
    # zero group -> zero scale, zero codes
    q4, s4 = oi.quantize_groups(np.zeros((1, 32)), 32, 2)
    bad += int(np.any(q4 != 0) or float(s4[0, 0]) != 0.0)
    # row storage round trip; bytes per token: d_c / 4 + d_r / 2 codes, fp16 scales
    rows = om.round_bf16(rng.standard_normal((5, 3, 72)))
    st = oi.quantize_cache_rows(rows, 64, 32, 2)
    bad += int(np.any(oi.dequantize_cache_rows(st["codes"], st["cscale"], st["rscale"], 64, 32, 2) != st["values"]))
    bad += int(st["codes"].shape[-1] != 64 // 4 + 8 // 2 or st["cscale"].shape[-1] != 2)
    # the rotary part is the INT4 quantiser's
    st4 = oi.quantize_cache_rows(rows, 64)
    bad += int(np.any(st["codes"][..., 16:] != st4["codes"][..., 32:]) or np.any(st["rscale"] != st4["rscale"]))
    return float(bad)


def check_rope_shift():
    """Re-rotation of cached rotary keys, against properties fixed by the
    composition of rotations: rows appended at p and shifted by d equal rows
    appended at p + d (up to the storage rounding); attention is unchanged when
    every key and the query move by the same d; a zero shift, the content
    latent and the slots outside the range are untouched bit for bit; d then
    -d returns the keys; low-bit rows re-quantise within half a step."""
    errs = []
    rng = np.random.default_rng(17)
    for cfg in (_tiny_video(), TINIER_BLOCK, TINY_DECODE.replace(name="tiny_dec_f32", dtype="f32")):
        inp = make_workload(cfg, seed=4)
        st = om.build_cache(cfg, inp)
        ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in st.items()}
        delta = rng.integers(-9, 10, (cfg.batch, 3))
        delta[0, 1:] = 0
        if cfg.batch > 1:
            delta[1] = 0                     # a sequence with a zero shift
        om.rope_shift(st, cfg, delta, 0, cfg.capacity)
        # unchanged: content, zero-shift sequences
        errs.append(float(np.any(st["values"][..., :cfg.d_c] != ref["values"][..., :cfg.d_c])))
        if cfg.batch > 1:
            errs.append(float(np.any(st["values"][1] != ref["values"][1])))
        # appended at p, shifted by d == appended at p + d: the stored key
        # rotated by d against the unrotated projection rotated at p + d
        frames = om.slot_frames(cfg, ref["newest"])
        P = cfg.tokens_per_frame
        y = None
        if not cfg.cache_given:
            x = om.as_f64(inp["x"])
            w = om.as_f64(inp["w_dkr"])
            for s_ in range(cfg.capacity):
                f = frames[s_]
                if f < 0:
                    continue
                yr = x[:, f, s_ % P] @ w[cfg.d_c:].T
                coords = om.token_coords(cfg, f, s_ % P) + delta[:, :cfg.rope_dims]
                want = om.rope_rotate(yr, coords, cfg)
                got = st["values"][:, s_, cfg.d_c:]
                errs.append(np.max(np.abs(got - want)) / max(1.0, np.max(np.abs(want))) / 1e-5)
        # shift back: the original keys up to the storage rounding
        st2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in st.items()}
        om.rope_shift(st2, cfg, -delta, 0, cfg.capacity)
        errs.append(np.max(np.abs(st2["values"] - ref["values"])) / 1e-5)
        # attention with every key and the query moved by the same shift
        if cfg.batch > 1:
            continue
        w_uk, w_uv = om.as_f64(inp["w_uk"]), om.as_f64(inp["w_uv"])
        q_nope, q_rope = om.as_f64(inp["q_nope"]), om.as_f64(inp["q_rope"])
        i = np.arange(cfg.n_q)
        c0 = om.token_coords(cfg, cfg.q_first + i // P, i % P)[None, :, None, :]
        q0 = om.rope_rotate(q_rope, c0, cfg)
        q1 = om.rope_rotate(q_rope, c0 + delta[0, :cfg.rope_dims], cfg)
        _, o0, l0 = om.attend(cfg, ref, q_nope, q0, w_uk, w_uv, cfg.q_first)
        _, o1, l1 = om.attend(cfg, st, q_nope, q1, w_uk, w_uv, cfg.q_first)
        errs.append(np.max(np.abs(o1 - o0)) / 1e-5)
        errs.append(np.max(np.abs(l1 - l0)) / 1e-5)
    # slot range: only [3, 3 + 5) moves
    cfg = _tiny_video()
    st = om.build_cache(cfg, make_workload(cfg, seed=5))
    ref = st["values"].copy()
    om.rope_shift(st, cfg, np.array([[2, 1, -1]]), 3, 5)
    out = np.ones(cfg.capacity, bool)
    out[3:8] = False
    errs.append(float(np.any(st["values"][:, out] != ref[:, out])))
    errs.append(float(not np.any(st["values"][:, 3:8, cfg.d_c:] != ref[:, 3:8, cfg.d_c:])))
    # low-bit: content codes and scales untouched; the re-quantised rotary key
    # is within half a step (plus the bf16 rounding) of the rotated key; amax -> +-7
    for lcfg in (TINY_INT4, TINY_INT2):
        st = om.build_cache(lcfg, make_workload(lcfg, seed=6))
        ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in st.items()}
        d = np.array([[3, -1, 2]])
        om.rope_shift(st, lcfg, d, 0, lcfg.capacity)
        nb = lcfg.d_c * om.content_bits(lcfg) // 8
        errs.append(float(np.any(st["codes"][..., :nb] != ref["codes"][..., :nb])))
        errs.append(float(np.any(st["cscale"] != ref["cscale"])))
        want = om.rope_rotate(ref["values"][..., lcfg.d_c:], d[0].astype(np.float64), lcfg)
        s_new = st["rscale"].astype(np.float64)[..., None]
        bound = s_new / 2 + np.abs(want) * 2.0 ** -8 + 1e-12
        errs.append(float(np.any(np.abs(st["values"][..., lcfg.d_c:] - want) > bound)))
        stored = oi.dequantize_cache_rows(st["codes"], st["cscale"], st["rscale"], lcfg.d_c, 32,
                                          om.content_bits(lcfg))
        errs.append(float(np.any(stored != st["values"])))
        codes = oi.unpack_nibbles(st["codes"][..., nb:])
        errs.append(float(np.any(np.max(np.abs(codes), axis=-1)[st["rscale"] > 0] != 7)))
        # a zero shift leaves every byte
        st3 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref.items()}
        om.rope_shift(st3, lcfg, np.zeros((1, 3), int), 0, lcfg.capacity)
        errs.append(float(any(np.any(st3[k] != ref[k]) for k in ("codes", "cscale", "rscale", "values"))))
    return float(max(errs))


def check_query_fold():
    """Load-time fold of the query and key up-projections: scalar loops on a
    tiny shape for the fold and the query up-projection, then the
    associativity (W^UK_h)^T (W^UQ_h c) = ((W^UK_h)^T W^UQ_h) c on workloads:
    the folded absorbed query equals the absorbed up-projected query."""
    errs = []
    rng = np.random.default_rng(19)
    cfg = TINIER.replace(name="fold", d_cq=5)
    H, dn, dc, dq = cfg.n_heads, cfg.d_nope, cfg.d_c, cfg.d_cq
    w_uq = rng.standard_normal((H * dn, dq))
    w_uk = rng.standard_normal((H, dc, dn))
    c_q = rng.standard_normal((2, 3, dq))
    fold = om.fold_query_weights(cfg, w_uq, w_uk)
    for h in range(H):
        for a in range(dc):
            for j in range(dq):
                v = 0.0
                for i in range(dn):
                    v += float(w_uk[h, a, i]) * float(w_uq[h * dn + i, j])
                errs.append(abs(fold[h, a, j] - v))
    up = om.query_up(cfg, c_q, w_uq)
    for b in range(2):
        for t in range(3):
            for h in range(H):
                for i in range(dn):
                    v = sum(float(c_q[b, t, j]) * float(w_uq[h * dn + i, j]) for j in range(dq))
                    errs.append(abs(up[b, t, h, i] - v))
    for key in (1, 2, 3):
        from mla_inputs import SMALL_CONFIGS
        c = SMALL_CONFIGS[key]
        inp = make_workload(c, seed=3, parts=("c_q", "w_uq", "w_uk", "q_rope"))
        cq, wq, wk = om.as_f64(inp["c_q"]), om.as_f64(inp["w_uq"]), om.as_f64(inp["w_uk"])
        qr = om.as_f64(inp["q_rope"])
        a = om.absorb_query_folded(c, cq, qr, om.fold_query_weights(c, wq, wk), c.q_first)
        b_ = om.absorb_query(c, om.query_up(c, cq, wq), qr, wk, c.q_first)
        errs.append(np.max(np.abs(a - b_)) / np.max(np.abs(b_)))
    return float(max(errs))


def _qkn_inputs(cfg, seed):
    rng = np.random.default_rng(seed)
    inp = make_workload(cfg, seed=seed)
    st = om.build_cache(cfg, inp)
    g_q = rng.uniform(0.5, 1.5, (cfg.n_heads, cfg.d_nope))
    g_k = rng.uniform(0.5, 1.5, (cfg.n_heads, cfg.d_nope))
    return inp, st, g_q, g_k


def check_qk_norm():
    """Explicit post-projection QK RMSNorm: scalar loops on a tiny workload;
    the absorbed form (static weights folded into the key up-projection,
    one inverse RMS per key token and per query token, applied to the content
    score) equals it; with unit-RMS keys and queries and unit weights it is
    plain attention; a common scale of every latent or of the query leaves the
    probabilities."""
    errs = []
    eps = 1e-6
    cfg = TINIER_BLOCK
    inp, st, g_q, g_k = _qkn_inputs(cfg, 7)
    w_uk, w_uv = om.as_f64(inp["w_uk"]), om.as_f64(inp["w_uv"])
    q_nope, q_rope = om.as_f64(inp["q_nope"]), om.as_f64(inp["q_rope"])
    q_rot = om.absorb_query(cfg, q_nope, q_rope, w_uk, cfg.q_first)[..., cfg.d_c:]
    _, o_lat, lse = om.attend_qk_norm(cfg, st, q_nope, q_rot, w_uk, w_uv, g_q, g_k, eps, cfg.q_first)
    H, dn, dc = cfg.n_heads, cfg.d_nope, cfg.d_c
    mask = om.mask_matrix(cfg, cfg.q_first, st["newest"])
    scale = 1.0 / math.sqrt(dn + cfg.d_r)
    # (1) scalar loops
    n = 0
    for b in range(cfg.batch):
        vals = st["values"][b]
        keys = []
        for s_ in range(cfg.capacity):
            k = [[sum(vals[s_, a] * w_uk[h, a, i] for a in range(dc)) for i in range(dn)] for h in range(H)]
            ms = sum(k[h][i] ** 2 for h in range(H) for i in range(dn)) / (H * dn)
            keys.append([[g_k[h][i] * k[h][i] / math.sqrt(ms + eps) for i in range(dn)] for h in range(H)])
        for t in range(cfg.n_q):
            q = q_nope[b, t]
            ms = sum(q[h][i] ** 2 for h in range(H) for i in range(dn)) / (H * dn)
            for h in range(H):
                qh = [g_q[h][i] * q[h][i] / math.sqrt(ms + eps) for i in range(dn)]
                sc = []
                for s_ in range(cfg.capacity):
                    if not mask[t, s_]:
                        continue
                    v = sum(qh[i] * keys[s_][h][i] for i in range(dn))
                    v += sum(q_rot[b, t, h, j] * vals[s_, dc + j] for j in range(cfg.d_r))
                    sc.append((v * scale, s_))
                m = max(v for v, _ in sc)
                tot = sum(math.exp(v - m) for v, _ in sc)
                o = [sum(math.exp(v - m) / tot * vals[s_, a] for v, s_ in sc) for a in range(dc)]
                errs.append(abs(lse[n + t, h] - (m + math.log(tot))))
                errs.append(max(abs(o_lat[n + t, h, a] - o[a]) for a in range(dc)))
        n += cfg.n_q
    # (2) absorbed form: score_h = inv_q inv_k (w_uk[h] (g_q g_k q_h)) . c + q_r . k_r
    gram = np.einsum("hai,hbi->ab", w_uk, w_uk)
    for b in range(cfg.batch):
        C = st["values"][b, :, :dc]
        inv_k = 1.0 / np.sqrt(np.einsum("sa,ab,sb->s", C, gram, C) / (H * dn) + eps)
        qn = q_nope[b]
        inv_q = 1.0 / np.sqrt(np.mean(qn * qn, axis=(1, 2)) + eps)
        q_lat = np.einsum("hai,thi->tha", w_uk, qn * (g_q * g_k)) * inv_q[:, None, None]
        s_abs = (np.einsum("tha,sa->ths", q_lat, C) * inv_k[None, None, :]
                 + np.einsum("thj,sj->ths", q_rot[b], st["values"][b, :, dc:]))
        k_all = om.rms_normalise(np.einsum("sc,hci->shi", C, w_uk), g_k, eps)
        q_all = om.rms_normalise(qn, g_q, eps)
        s_mat = (np.einsum("thi,shi->ths", q_all, k_all)
                 + np.einsum("thj,sj->ths", q_rot[b], st["values"][b, :, dc:]))
        errs.append(np.max(np.abs(s_abs - s_mat)))
    # (3) unit RMS, unit weights, eps 0: plain attention
    for c2 in (TINIER_BLOCK, TINY_DECODE.replace(name="td32", dtype="f32")):
        inp2, st2, _, _ = _qkn_inputs(c2, 8)
        wk2, wv2 = om.as_f64(inp2["w_uk"]), om.as_f64(inp2["w_uv"])
        for b in range(c2.batch):
            C = st2["values"][b, :, :c2.d_c]
            k = np.einsum("sc,hci->shi", C, wk2)
            r = np.sqrt(np.mean(k * k, axis=(1, 2)))
            st2["values"][b, :, :c2.d_c] = C / np.where(r > 0, r, 1.0)[:, None]
        qn2 = om.as_f64(inp2["q_nope"])
        qn2 = qn2 / np.sqrt(np.mean(qn2 * qn2, axis=(-2, -1), keepdims=True))
        qr2 = om.absorb_query(c2, qn2, om.as_f64(inp2["q_rope"]), wk2, c2.q_first)[..., c2.d_c:]
        ones = np.ones((c2.n_heads, c2.d_nope))
        a = om.attend_qk_norm(c2, st2, qn2, qr2, wk2, wv2, ones, ones, 0.0, c2.q_first)
        p = om.attend(c2, st2, qn2, qr2, wk2, wv2, c2.q_first)
        errs.append(max(np.max(np.abs(x - y)) for x, y in zip(a, p)))
    # (4) scale invariance of the probabilities
    st3 = {"values": st["values"].copy(), "newest": st["newest"]}
    st3["values"][..., :dc] *= 3.0
    _, o3, l3 = om.attend_qk_norm(cfg, st3, 0.25 * q_nope, q_rot, w_uk, w_uv, g_q, g_k, 0.0, cfg.q_first)
    _, o0, l0 = om.attend_qk_norm(cfg, st, q_nope, q_rot, w_uk, w_uv, g_q, g_k, 0.0, cfg.q_first)
    errs.append(np.max(np.abs(l3 - l0)))
    errs.append(np.max(np.abs(o3 - 3.0 * o0)))
    return float(max(errs))


# ---------------------------------------------------------------------------
# admissible low-bit codes: the bounds the GPU tests hold stored codes to
# ---------------------------------------------------------------------------
def check_admissible_codes():
    bad = 0
    rng = np.random.default_rng(31)
    v = rng.standard_normal((300, 64)) * np.exp(rng.uniform(-6, 6, (300, 1)))
    lo, hi = om.bf16_bracket(v)
    # the bracket: bf16 values around v, one step apart, round_bf16 picks one
    bad += int(np.any(om.round_bf16(lo) != lo) or np.any(om.round_bf16(hi) != hi))
    bad += int(np.any(lo > v) or np.any(hi < v))
    r = om.round_bf16(v)
    bad += int(np.any((r != lo) & (r != hi)))
    _, e = np.frexp(v)
    bad += int(np.any((hi - lo != 0) & (hi - lo != np.ldexp(1.0, e - 8))))
    ex = om.round_bf16(v)
    elo, ehi = om.bf16_bracket(ex)
    bad += int(np.any(elo != ex) or np.any(ehi != ex))
    for bits, group in ((4, 32), (2, 32), (4, 64)):
        # exact inputs: the bounds collapse to the quantiser's own result
        q, s = oi.quantize_groups(ex, group, bits)
        cmin, cmax, smin, smax = oi.admissible_groups(ex, ex, group, bits)
        bad += int(np.any(cmin != q) or np.any(cmax != q))
        bad += int(np.any(smin.view(np.uint16) != s.view(np.uint16)) or np.any(smax.view(np.uint16) != s.view(np.uint16)))
        # brute force: every choice of bracket ends gives codes and scales
        # inside the bounds, and the bounds are reached
        cmin, cmax, smin, smax = oi.admissible_groups(lo, hi, group, bits)
        seen_lo = np.zeros(cmin.shape, bool)
        seen_hi = np.zeros(cmin.shape, bool)
        for _ in range(64):
            pick = rng.random(v.shape) < 0.5
            x = np.where(pick, lo, hi)
            qx, sx = oi.quantize_groups(x, group, bits)
            bad += int(np.any(qx < cmin) or np.any(qx > cmax))
            bad += int(np.any(sx.astype(np.float64) < smin.astype(np.float64))
                       or np.any(sx.astype(np.float64) > smax.astype(np.float64)))
            seen_lo |= qx == cmin
            seen_hi |= qx == cmax
        # intervals are at most one bf16 step wide: no code range wider than 2
        bad += int(np.any(cmax.astype(int) - cmin.astype(int) > 2))
        bad += int(np.mean(seen_lo & seen_hi) < 0.999)
    # groups whose intervals may all hold zero: the scale may be zero or any
    # tiny value, under which a small element can take the largest code
    # (brute force over interval ends and zero)
    for bits in (4, 2):
        h = np.ldexp(1.0, rng.integers(-30, -8, (200, 1))) * rng.uniform(0.05, 1.0, (200, 32))
        zlo = -h * (rng.random((200, 32)) < 0.7)
        zhi = h * (rng.random((200, 32)) < 0.7)
        cmin, cmax, smin, smax = oi.admissible_groups(zlo, zhi, 32, bits)
        bad += int(np.any(smin != 0))
        for _ in range(64):
            pick = rng.integers(0, 3, (200, 32))
            x = np.where(pick == 0, zlo, np.where(pick == 1, zhi, 0.0))
            # most elements zero, so that a small one can be the group maximum
            x = np.where(rng.random((200, 32)) < 0.9, 0.0, x)
            qx, sx = oi.quantize_groups(x, 32, bits)
            bad += int(np.any(qx < cmin) or np.any(qx > cmax))
            bad += int(np.any(sx.astype(np.float64) > smax.astype(np.float64)))
    # a code two away from the quantiser's is outside the bounds
    q, _ = oi.quantize_groups(ex, 32)
    cmin, cmax, _, _ = oi.admissible_groups(lo, hi, 32)
    moved = np.clip(q.astype(int) + 2, -8, 7)
    inside = (moved >= cmin) & (moved <= cmax) & (moved != q)
    bad += int(np.any(inside & (np.abs(moved - q) == 2)))
    return float(bad)


CHECKS = {
    "bruteforce": (check_bruteforce, 1e-12),
    "absorption": (check_absorption, 1e-12),
    "value_fold": (check_value_fold, 1e-12),
    "rope_invariants": (check_rope_invariants, 1e-9),
    "rope_worked_values": (check_rope_worked_values, 1e-12),
    "mask_enumeration": (check_mask_enumeration, 0.0),
    "softmax_closed_forms": (check_softmax_closed_forms, 1e-12),
    "library_attention": (check_library_attention, 1e-12),
    "bf16_rounding": (check_bf16_rounding, 0.0),
    "int4": (check_int4, 0.0),
    "int2": (check_int2, 0.0),
    "admissible_codes": (check_admissible_codes, 0.0),
    "rope_shift": (check_rope_shift, 0.5),
    "query_fold": (check_query_fold, 1e-12),
    "qk_norm": (check_qk_norm, 1e-9),
}


def run_checks(names=None, stop_at_first_failure=False):
    out = {}
    for name, (fn, tol) in CHECKS.items():
        if names is not None and name not in names:
            continue
        try:
            err = fn()
        except Exception as exc:  # a planted mistake may also crash a check
            err = float("inf")
            out[name] = (err, tol, repr(exc))
            if stop_at_first_failure:
                break
            continue
        out[name] = (err, tol, None)
        if stop_at_first_failure and not err <= tol:
            break
    return out
