#!/usr/bin/env python
"""Throughput of one MLA step on one MI355X, printed as one JSON line.

A step is one pass of the whole path over one batch of seeded synthetic
input, through the C-ABI: mla_cache_append (the newest frame or token),
mla_absorb_q, mla_attention, mla_unabsorb_out.  Inputs are resident in HBM
before timing starts.  Default workload: LLM decode (batch 32, 128 heads,
4096 cached tokens per sequence, d_c 512, d_r 64, bf16).  ``--config 3``
times the video-chunk workload (1560 query tokens over a 12-frame window).

Steps are timed as replays of HIP graphs that capture one step's library
calls (``--eager``: direct calls).  The per-call breakdown comes from a pass
of direct calls with HIP events between them.  The "roofline" object covers
the attention call (the attention kernel and, with key splits, the merge):
algorithmic bytes (decode) or FLOPs (chunk) per call divided by its mean
duration over back-to-back calls, measured with HIP events on the stream the
library launches on.  "cpu_baseline" is the
float64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA attention query-tokens/s + TFLOP/s (% MFMA peak); decode cache GB/s (% HBM)"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20         # Infinity Cache


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2,
                    help="workload 1..6 (default 2: LLM decode; 5, 6: INT4 and INT2 content cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy kernel (for HBM counter calibration)")
    ap.add_argument("--no-chunk-block", action="store_true",
                    help="with the decode workload, skip the video-chunk attention block of the line")
    ap.add_argument("--eager", action="store_true",
                    help="time the steps as direct library calls instead of replays of a captured HIP graph")
    return ap.parse_args()


def _code_lines(text):
    """The lines of a C++ source with line comments and blank lines removed
    (a "//" inside a string literal is kept), so that a comment edit leaves
    the hash of the compiled code unchanged."""
    for line in text.splitlines():
        in_str, cut = False, len(line)
        for i, ch in enumerate(line):
            if ch == '"' and (i == 0 or line[i - 1] != "\\"):
                in_str = not in_str
            elif not in_str and line.startswith("//", i):
                cut = i
                break
        code = line[:cut].rstrip()
        if code:
            yield code


def source_hash():
    """Hash of the attention kernels' code (comments excluded): ties the
    stored HBM-traffic counters to the kernels they were taken from."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "head_latent_attention_cache_amd", "csrc")
    for n in sorted(os.listdir(d)):
        if n.startswith("attention") or n in ("common.hpp", "launch.hpp"):
            h.update(n.encode() + b"\n")
            for line in _code_lines(open(os.path.join(d, n), encoding="utf-8").read()):
                h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the MLA path here runs on a single MI355X and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import head_latent_attention_cache_amd as mla
    from head_latent_attention_cache_amd import api
    from mla_inputs import get_config, make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mla.load()                      # raises if the HIP library is not built
    torch.cuda.set_device(0)
    dev = "cuda"
    cfg = get_config(args.config)
    B, H, P = cfg.batch, cfg.n_heads, cfg.tokens_per_frame
    dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
    dt = api.torch_dtype(dims)

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    t0 = time.time()
    inp = make_workload(cfg, seed=0)
    print(f"[bench] inputs for {cfg.name} drawn in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    w_dkr, w_uk, w_uv, w_o = (dev_t(inp[k]) for k in ("w_dkr", "w_uk", "w_uv", "w_o"))
    q_nope, q_rope = dev_t(inp["q_nope"]), dev_t(inp["q_rope"])

    # frames appended by the step and the cache state before it
    step_frames = 1 if cfg.cache_given else cfg.n_frames - cfg.q_first
    first_step_frame = cfg.n_frames - step_frames
    cache_bytes, aux_bytes = api.cache_nbytes(dims, geom)
    hbm_bound = cfg.cache_given
    n_sets = max(1, math.ceil(3.5 * MALL_BYTES / (cache_bytes + aux_bytes))) if hbm_bound else 1
    n_sets = min(n_sets, 16)
    ws_app = torch.empty(max(16, api.append_workspace_bytes(dims, geom, step_frames * P),
                             api.append_workspace_bytes(dims, geom, P)), dtype=torch.uint8, device=dev)
    caches = []
    if cfg.cache_given:
        cc, cr = dev_t(inp["cache_c"]), dev_t(inp["cache_r"])
        L = cc.shape[1]
        x_step = dev_t(inp["x_new"]).reshape(B, P, cfg.d_model)
        for _ in range(n_sets):
            c, a = api.new_cache(dims, geom)
            c[:, :L, :cfg.d_c] = cc
            c[:, :L, cfg.d_c:] = cr
            caches.append((c, a))
        del cc, cr
    else:
        x = dev_t(inp["x"])
        x_step = x[:, first_step_frame:].reshape(B, step_frames * P, cfg.d_model).contiguous()
        for _ in range(n_sets):
            c, a = api.new_cache(dims, geom)
            for f in range(first_step_frame):
                api.cache_append(dims, geom, x[:, f].contiguous(),
                                 torch.full((B,), f, dtype=torch.int32, device=dev), w_dkr, c, a,
                                 workspace=ws_app)
            caches.append((c, a))
        del x
    frame_t = torch.full((B,), first_step_frame, dtype=torch.int32, device=dev)
    q_first = torch.full((B,), cfg.q_first, dtype=torch.int32, device=dev)
    newest = torch.full((B,), cfg.newest, dtype=torch.int32, device=dev)
    q_abs = [torch.empty((B, cfg.n_q, H, cfg.d_qk), dtype=dt, device=dev) for _ in range(n_sets)]
    o_lat = [torch.empty((B, cfg.n_q, H, cfg.d_c), dtype=dt, device=dev) for _ in range(n_sets)]
    lse = torch.empty((B, cfg.n_q, H), dtype=torch.float32, device=dev)
    o_heads = torch.empty((B, cfg.n_q, H * cfg.d_v), dtype=dt, device=dev)
    y = torch.empty((B, cfg.n_q, cfg.d_model), dtype=dt, device=dev)
    ws_attn_n = api.attention_workspace_bytes(dims, geom, cfg.n_q)
    ws_attn = torch.empty(max(16, ws_attn_n), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] setup done ({n_sets} cache set(s) of {cache_bytes / 1e6:.1f} MB)", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    ev = {k: [] for k in ("append", "absorb", "attention", "unabsorb")}

    def step(i, record):
        c, a = caches[i % n_sets]
        qa, ol = q_abs[i % n_sets], o_lat[i % n_sets]
        marks = []

        def mark():
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                marks.append(e)
        mark()
        api.cache_append(dims, geom, x_step, frame_t, w_dkr, c, a, workspace=ws_app)
        mark()
        api.absorb_q(dims, geom, q_nope, q_rope, q_first, w_uk, qa)
        mark()
        api.attention(dims, geom, qa, q_first, newest, c, a, ol, lse, workspace=ws_attn)
        mark()
        api.unabsorb_out(dims, geom, ol, w_uv, w_o, o_heads, y)
        mark()
        if record:
            for k, (e0, e1) in zip(ev, zip(marks[:-1], marks[1:])):
                ev[k].append((e0, e1))

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    # direct calls, with events between the calls: the per-call times
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, True)
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms_per_step = start.elapsed_time(end) / args.steps
    call_ms = {k: float(np.mean([e0.elapsed_time(e1) for e0, e1 in v])) for k, v in ev.items()}
    ms_per_step, timing = eager_ms_per_step, "direct calls"
    if not args.eager:
        # the same steps captured once per cache set into HIP graphs and
        # replayed: the launch gaps between the step's kernels go away
        graphs = []
        for k in range(n_sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(k, False)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % n_sets].replay()
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            graphs[(args.warmup + i) % n_sets].replay()
        end.record(stream)
        torch.cuda.synchronize()
        ms_per_step, timing = start.elapsed_time(end) / args.steps, "HIP graph replay"

    # the attention call alone, back to back over the rotated cache sets
    # (at least 100 calls where they fit in ~10 s): its mean duration
    # (attention kernel + split merge) is the roofline's launch time,
    # comparable with the kernel trace
    n_attn = max(args.steps, min(100, int(10000.0 / max(call_ms["attention"], 1e-3))))
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(n_attn):
        k = (args.warmup + i) % n_sets
        api.attention(dims, geom, q_abs[k], q_first, newest, caches[k][0], caches[k][1], o_lat[k], lse,
                      workspace=ws_attn)
    end.record(stream)
    torch.cuda.synchronize()
    attn_call_ms = start.elapsed_time(end) / n_attn
    # a second run with events around every call (they add a gap between
    # calls, so the mean above is taken without them): median, minimum and
    # 90th percentile of the call duration
    n_dist = max(10, min(100, int(5000.0 / max(attn_call_ms, 1e-3))))
    call_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dist)]
    for i in range(n_dist):
        k = (args.warmup + i) % n_sets
        call_ev[i][0].record(stream)
        api.attention(dims, geom, q_abs[k], q_first, newest, caches[k][0], caches[k][1], o_lat[k], lse,
                      workspace=ws_attn)
        call_ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_call = np.array([e0.elapsed_time(e1) for e0, e1 in call_ev])
    attn_stats = {"calls": n_attn, "mean_ms": round(attn_call_ms, 5), "timed_singly": n_dist,
                  "median_ms": round(float(np.median(per_call)), 5), "min_ms": round(float(per_call.min()), 5),
                  "p90_ms": round(float(np.percentile(per_call, 90)), 5)}

    # achievable peaks of this device, measured in the same process: a
    # stream of independent bf16 MFMAs and a streaming HBM read
    print("[bench] measuring achievable MFMA and HBM rates", file=sys.stderr, flush=True)
    peaks = measure_peaks(stream)

    # ---- operations beside the step (not part of `value`) ----
    print(f"[bench] step timed ({ms_per_step:.4f} ms); operations beside the step", file=sys.stderr, flush=True)
    adjacent = {}
    # rotary-key shift of every slot of every sequence (alternating +1 / -1
    # frames so the cache returns to its state); bytes: the rotary part of
    # each row read and written (low-bit: codes and the per-token scale)
    c0, a0 = caches[0]
    deltas = [torch.tensor([s_, 0, 0] * B, dtype=torch.int32, device=dev) for s_ in (1, -1)]
    for i in range(2):
        api.cache_rope_shift(dims, geom, deltas[i], 0, cfg.capacity, c0, a0)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        api.cache_rope_shift(dims, geom, deltas[i % 2], 0, cfg.capacity, c0, a0)
    end.record(stream)
    torch.cuda.synchronize()
    shift_ms = start.elapsed_time(end) / args.steps
    rot_bytes = (cfg.d_r // 2 + 2) if cfg.cache_fmt in ("int4", "int2") else cfg.d_r * (2 if cfg.dtype == "bf16" else 4)
    shift_bytes = 2.0 * B * cfg.capacity * rot_bytes
    adjacent["cache_rope_shift"] = {"ms": round(shift_ms, 5), "slots": B * cfg.capacity,
                                    "bytes": shift_bytes, "gbs": round(shift_bytes / shift_ms / 1e6, 1),
                                    "hbm_frac": round(shift_bytes / shift_ms / 1e6 / PEAK_HBM_GBS, 4)}

    # the absorbed query from a low-rank query latent: the fold of W^UQ and
    # W^UK formed once (load time), then one product per step over d_cq,
    # against the per-head absorb of given q_nope (the step's call; the query
    # up-projection that would produce q_nope is outside this library)
    fin = make_workload(cfg, seed=0, parts=("c_q", "w_uq"))
    c_q_t, w_uq_t = dev_t(fin["c_q"]), dev_t(fin["w_uq"])
    del fin
    w_fold = torch.empty((H, cfg.d_c, cfg.d_cq), dtype=dt, device=dev)
    qa_f = torch.empty_like(q_abs[0])
    api.fold_query_weights(dims, w_uq_t, w_uk, w_fold)
    torch.cuda.synchronize()
    start.record(stream)
    api.fold_query_weights(dims, w_uq_t, w_uk, w_fold)
    end.record(stream)
    torch.cuda.synchronize()
    fold_ms = start.elapsed_time(end)
    timed = {}
    for name, call in (("absorb_q_folded", lambda: api.absorb_q_folded(dims, geom, c_q_t, q_rope, q_first, w_fold, qa_f)),
                       ("absorb_q", lambda: api.absorb_q(dims, geom, q_nope, q_rope, q_first, w_uk, qa_f))):
        call()
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            call()
        end.record(stream)
        torch.cuda.synchronize()
        timed[name] = start.elapsed_time(end) / args.steps
    adjacent["query_fold"] = {"d_cq": cfg.d_cq, "fold_ms": round(fold_ms, 4),
                              "absorb_q_folded_ms": round(timed["absorb_q_folded"], 5),
                              "absorb_q_ms": round(timed["absorb_q"], 5),
                              "w_fold_bytes": w_fold.numel() * w_fold.element_size(),
                              "w_uk_bytes": w_uk.numel() * w_uk.element_size(),
                              "w_uq_bytes": w_uq_t.numel() * w_uq_t.element_size()}
    del w_fold, w_uq_t, c_q_t, qa_f

    print("[bench] rotary-key shift and query fold timed", file=sys.stderr, flush=True)
    # QK normalisation: the same cache and queries with the content score
    # scaled by each key's inverse RMS (unit norm weights), against the plain
    # call on the same cache set; plus the per-append key statistic and the
    # query statistic inside the absorb
    cfg_q = cfg.replace(qk_norm=True)
    dims_q = api.dims_from_config(cfg_q)
    # (the MFMA kernels serve it for d_r = 64 and d_r = 512)
    qkn_measured = cfg.d_r in (64, 512) and cfg.d_c == 512 and cfg.dtype == "bf16"
    if qkn_measured:
        _, na_q = api.cache_nbytes(dims_q, geom)
        c0, a0 = caches[0]
        aux_q = torch.zeros(na_q // 2, dtype=torch.float16, device=dev)
        if a0 is not None:
            aux_q[:a0.numel()].copy_(a0)          # the low-bit scales keep their offsets
        gram = torch.empty((cfg.d_c, cfg.d_c), dtype=torch.float32, device=dev)
        w_uk_q = torch.empty_like(w_uk)
        ones = torch.ones((H, cfg.d_nope), dtype=dt, device=dev)
        api.qk_norm_prepare(dims_q, w_uk, ones, ones, w_uk_q, gram)
        f0 = max(0, cfg.newest + 1 - cfg.window)
        api.cache_key_norm(dims_q, geom, (cfg.newest + 1 - f0) * P, torch.full((B,), f0, dtype=torch.int32, device=dev),
                           gram, c0, aux_q)
        f_new = torch.full((B,), cfg.newest, dtype=torch.int32, device=dev)
        ws_kn = torch.empty(max(16, api.key_norm_workspace_bytes(dims_q, geom, P)), dtype=torch.uint8, device=dev)
        qa_q, ol_q = torch.empty_like(q_abs[0]), torch.empty_like(o_lat[0])
        api.absorb_q(dims_q, geom, q_nope, q_rope, q_first, w_uk_q, qa_q)
        timed_q = {}
        calls = (("attention_plain", lambda: api.attention(dims, geom, q_abs[0], q_first, newest, c0, a0, o_lat[0],
                                                           lse, workspace=ws_attn)),
                 ("attention_qk_norm", lambda: api.attention(dims_q, geom, qa_q, q_first, newest, c0, aux_q, ol_q,
                                                             lse, workspace=ws_attn)),
                 ("key_norm_per_append", lambda: api.cache_key_norm(dims_q, geom, P, f_new, gram, c0, aux_q, ws_kn)),
                 ("absorb_q_qk_norm", lambda: api.absorb_q(dims_q, geom, q_nope, q_rope, q_first, w_uk_q, qa_q)))
        for rnd in range(3):            # alternating rounds; the fastest round of each call
            for name, call in calls:
                call()
                torch.cuda.synchronize()
                start.record(stream)
                for i in range(args.steps):
                    call()
                end.record(stream)
                torch.cuda.synchronize()
                t_ms = start.elapsed_time(end) / args.steps
                timed_q[name] = min(t_ms, timed_q.get(name, t_ms))
        adjacent["qk_norm"] = {k + "_ms": round(v, 5) for k, v in timed_q.items()}
        adjacent["qk_norm"]["attention_overhead"] = round(timed_q["attention_qk_norm"] / timed_q["attention_plain"] - 1, 4)
        del aux_q, gram, w_uk_q, qa_q, ol_q, ws_kn

    print("[bench] QK normalisation timed", file=sys.stderr, flush=True)
    # ---- algorithmic work of the attention call ----
    qf = np.arange(cfg.n_q) // P + cfg.q_first
    mask_keys = 0
    for f in qf:   # visible keys per query token (rows of all heads see the same keys)
        lo = max(cfg.newest - cfg.window + 1, 0)
        vis = 0
        for fk in range(lo, cfg.newest + 1):
            if fk // cfg.frames_per_block <= f // cfg.frames_per_block and f - fk < cfg.window:
                vis += P
        mask_keys += vis
    pairs = B * H * mask_keys
    flops = 2.0 * pairs * (cfg.d_qk + cfg.d_c)
    esz = 2 if cfg.dtype == "bf16" else 4
    # every visible cache row is read once per sequence (all heads share it)
    rows_visible = min(cfg.capacity, (cfg.newest + 1) * P)
    cache_row_bytes = (cache_bytes + aux_bytes) / (B * cfg.capacity)
    cache_read = B * rows_visible * cache_row_bytes
    io_bytes = B * cfg.n_q * H * (cfg.d_qk * esz + cfg.d_c * esz + 4)
    attn_ms = attn_call_ms
    attn_s = attn_ms / 1e3
    tflops = flops / attn_s / 1e12
    cache_gbs = cache_read / attn_s / 1e9
    total_gbs = (cache_read + io_bytes) / attn_s / 1e9
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(total_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(total_gbs / PEAK_HBM_GBS, 4)}
        alg_per_launch = {"bytes": cache_read + io_bytes}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
        alg_per_launch = {"flops": flops}
    ach = peaks["hbm_read_gbs"] if hbm_bound else peaks["mfma_bf16_tflops"]
    roof["achievable_peak"] = ach
    roof["frac_achievable"] = round(roof["achieved"] / ach, 4) if ach else None
    roof["traffic"] = None
    roof["kernel"] = "mla_attention"
    roof["launch_ms"] = round(attn_ms, 5)
    src = source_hash()
    tfile = os.path.join(ROOT, "profiles", f"attention_traffic_{cfg.name}.json")
    if os.path.exists(tfile):
        tr = json.load(open(tfile))
        if tr.get("source_hash") == src:
            roof["traffic"] = tr.get("hbm_bytes_per_launch")
    queries = B * cfg.n_q
    value = queries / (ms_per_step / 1e3)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "heads": H, "query_tokens_per_step": queries,
                   "keys_per_sequence": rows_visible, "d_c": cfg.d_c, "d_r": cfg.d_r,
                   "d_model": cfg.d_model, "window_frames": cfg.window, "tokens_per_frame": P,
                   "cache_sets_rotated": n_sets},
        "attention": {"ms": round(attn_ms, 5), "tflops": round(tflops, 2),
                      "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                      "cache_gbs": round(cache_gbs, 1), "cache_hbm_frac": round(cache_gbs / PEAK_HBM_GBS, 4),
                      "query_tokens_per_s": round(queries / attn_s, 1),
                      "algorithmic_per_launch": alg_per_launch, "source_hash": src, "per_call": attn_stats},
        "peaks_measured": peaks,
        "breakdown_ms": {k: round(v, 5) for k, v in call_ms.items()},
        "timing": {"step": timing, "direct_calls_ms_per_step": round(eager_ms_per_step, 5)},
        "roofline": roof,
        "adjacent_ops": adjacent,
    }

    if args.copy_calibration:
        # a plain copy kernel of known size for scaling HBM byte counters:
        # [131072, 1024] bf16 into the first 1024 columns of a [131072, 1152]
        # array (an elementwise copy kernel; 256 MiB read, 256 MiB written)
        rows = 131072
        src_t = torch.ones((rows, 1024), dtype=torch.bfloat16, device=dev)
        big = torch.empty((rows, 1152), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            big[:, :1024] = src_t
        torch.cuda.synchronize()
        out["copy_calibration"] = {"kernel": "elementwise copy, bf16 [131072, 1024] into a [131072, 1152] view",
                                   "read_bytes": rows * 1024 * 2, "write_bytes": rows * 1024 * 2}
        del src_t, big

    # ---- the MFMA-bound half of the metric: video-chunk attention, and the
    # long-horizon video (d_r 512, the wide-row kernel) ----
    if args.config == 2 and not args.no_chunk_block:
        print("[bench] video-chunk attention block", file=sys.stderr, flush=True)
        out["video_chunk"] = chunk_block(stream, peaks)
        print("[bench] long-video attention block", file=sys.stderr, flush=True)
        out["long_video"] = chunk_block(stream, peaks, key=4, n_calls=8, warmup=2)

    # ---- CPU oracle on a bounded sample ----
    if not args.no_cpu_baseline:
        cb = cpu_baseline(cfg, inp, args.cpu_seconds)
        cb.update(host_info())
        cb["gpu_over_oracle"] = round(value / cb["value"], 1) if cb["value"] else None
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


def attention_flops(cfg):
    """Algorithmic FLOPs of one attention call: 2 (d_c + d_r + d_c) per
    (row, visible key), rows = batch x query tokens x heads."""
    import numpy as np
    P = cfg.tokens_per_frame
    qf = np.arange(cfg.n_q) // P + cfg.q_first
    keys = 0
    for f in qf:
        lo = max(cfg.newest - cfg.window + 1, 0)
        keys += sum(P for fk in range(lo, cfg.newest + 1)
                    if fk // cfg.frames_per_block <= f // cfg.frames_per_block and f - fk < cfg.window)
    return 2.0 * cfg.batch * cfg.n_heads * keys * (cfg.d_qk + cfg.d_c)


def chunk_block(stream, peaks, key=3, n_calls=120, warmup=10):
    """Attention over a video window, inputs resident in HBM: the cache built
    by appending every frame of the workload, the absorbed queries of its
    query frames, then back-to-back mla_attention calls timed with HIP events
    on the library's stream; FLOP-based roofline.  key 3: the video chunk
    (1560 query tokens x 32 heads over an 18,720-key window); key 4: the
    long-horizon video (batch 2, 4680 query tokens x 32 heads over 74,880
    keys of 1024-wide rows)."""
    import numpy as np
    import torch
    from head_latent_attention_cache_amd import api
    from mla_inputs import get_config, make_workload

    cfg = get_config(key)
    dev = "cuda"
    dims, geom = api.dims_from_config(cfg), api.geom_from_config(cfg)
    B, H, P = cfg.batch, cfg.n_heads, cfg.tokens_per_frame
    inp = make_workload(cfg, seed=0, parts=["x", "w_dkr", "w_uk", "q_nope", "q_rope"])

    def dev_t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    x = dev_t(inp["x"])
    w_dkr, w_uk = dev_t(inp["w_dkr"]), dev_t(inp["w_uk"])
    cache, aux = api.new_cache(dims, geom)
    ws_app = torch.empty(max(16, api.append_workspace_bytes(dims, geom, P)), dtype=torch.uint8, device=dev)
    for f in range(cfg.n_frames):
        api.cache_append(dims, geom, x[:, f].contiguous(), torch.full((B,), f, dtype=torch.int32, device=dev),
                         w_dkr, cache, aux, workspace=ws_app)
    del x
    q_first = torch.full((B,), cfg.q_first, dtype=torch.int32, device=dev)
    newest = torch.full((B,), cfg.newest, dtype=torch.int32, device=dev)
    q_abs = torch.empty((B, cfg.n_q, H, cfg.d_qk), dtype=torch.bfloat16, device=dev)
    api.absorb_q(dims, geom, dev_t(inp["q_nope"]), dev_t(inp["q_rope"]), q_first, w_uk, q_abs)
    del inp
    o_lat = torch.empty((B, cfg.n_q, H, cfg.d_c), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, cfg.n_q, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, api.attention_workspace_bytes(dims, geom, cfg.n_q)), dtype=torch.uint8, device=dev)

    def call():
        api.attention(dims, geom, q_abs, q_first, newest, cache, aux, o_lat, lse, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_calls):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_calls
    single = []
    for _ in range(min(20, n_calls)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        single.append((a, b))
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in single])
    flops = attention_flops(cfg)
    tflops = flops / (ms / 1e3) / 1e12
    roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "achievable_peak": peaks["mfma_bf16_tflops"],
            "frac_achievable": round(tflops / peaks["mfma_bf16_tflops"], 4) if peaks["mfma_bf16_tflops"] else None,
            "traffic": None, "kernel": "mla_attention", "launch_ms": round(ms, 5)}
    src = source_hash()
    tfile = os.path.join(ROOT, "profiles", f"attention_traffic_{cfg.name}.json")
    if os.path.exists(tfile):
        tr = json.load(open(tfile))
        if tr.get("source_hash") == src:
            roof["traffic"] = tr.get("hbm_bytes_per_launch")
    return {"workload": cfg.name, "calls": n_calls, "warmup": warmup, "ms": round(ms, 5),
            "median_ms": round(float(np.median(per)), 5), "min_ms": round(float(per.min()), 5),
            "p90_ms": round(float(np.percentile(per, 90)), 5), "tflops": round(tflops, 2),
            "query_tokens_per_s": round(B * cfg.n_q / (ms / 1e3), 1), "algorithmic_flops": flops,
            "config": {"batch": B, "heads": H, "query_tokens": cfg.n_q, "keys": cfg.capacity, "d_c": cfg.d_c,
                       "d_r": cfg.d_r, "grid": [cfg.grid_h, cfg.grid_w], "window_frames": cfg.window},
            "source_hash": src, "roofline": roof}


def measure_peaks(stream):
    """Best of five launches of each probe (after one warm-up launch)."""
    import torch
    from head_latent_attention_cache_amd import api
    dev = "cuda"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_rate(launch, work):
        launch()
        torch.cuda.synchronize()
        best = 0.0
        for _ in range(5):
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            best = max(best, work / (e0.elapsed_time(e1) / 1e3))
        return best

    # 1024 work-groups (4 waves per SIMD on 256 CUs), 64,000 MFMAs per wave
    n_wg, iters = 1024, 4000
    out_f = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    flops = api.probe_mfma(n_wg, iters, out_f, False)
    mfma_const = best_rate(lambda: api.probe_mfma(n_wg, iters, out_f, False), flops) / 1e12
    mfma = best_rate(lambda: api.probe_mfma(n_wg, iters, out_f, True), flops) / 1e12
    # 4 GiB read once per launch (16x the 256 MB last-level cache)
    n_wg_r = 4096
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    out_u = torch.empty(n_wg_r * 256, dtype=torch.int32, device=dev)
    nbytes = buf.numel()
    hbm = best_rate(lambda: api.probe_hbm_read(buf, n_wg_r, out_u), nbytes) / 1e9
    del buf, out_u, out_f
    return {"mfma_bf16_tflops": round(mfma, 1), "mfma_bf16_tflops_fixed_operands": round(mfma_const, 1),
            "hbm_read_gbs": round(hbm, 1),
            "mfma_probe": f"{n_wg} work-groups x 4 waves x {iters * 16} independent 32x32x16 bf16 MFMAs; "
                          "two pseudo-random operand pairs in turn (fixed operands: one small-integer pair)",
            "hbm_probe": f"streaming read of {nbytes >> 30} GiB, {n_wg_r} work-groups, 16-byte loads",
            "method": "best of 5 launches, HIP events on the library's stream"}


def host_info():
    """CPU model (from /proc/cpuinfo) and the BLAS library NumPy calls."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        import numpy  # noqa: F401  (loads its BLAS)
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or None
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas}


_WORKER = {}


def _oracle_worker_init(cfg_name, chunk):
    """Pool initializer: the seeded inputs (and, for chunk workloads, the
    oracle's cache, which a resident-input measurement excludes) built once
    per worker, outside the timed region."""
    import oracle.mla as om
    from mla_inputs import get_config, make_workload
    cfg = get_config(cfg_name)
    inp = make_workload(cfg, seed=0)
    _WORKER.update(cfg=cfg, inp=inp, st=om.build_cache(cfg, inp) if chunk else None)


def _oracle_task(arg):
    """One timed unit of oracle work: a whole decode sequence (cache rows,
    absorb, attention with materialised heads, output projection) or one
    query token of a chunk workload (all heads, the whole window)."""
    import oracle.mla as om
    cfg, inp, st = _WORKER["cfg"], _WORKER["inp"], _WORKER["st"]
    t0 = time.time()
    if st is None:
        b = arg
        sub = {k: (v[b:b + 1] if k in ("q_nope", "q_rope", "cache_c", "cache_r", "x_new") else v)
               for k, v in inp.items()}
        om.run(cfg.replace(batch=1), sub)
    else:
        om.run(cfg, inp, tokens=[(0, arg)], st=st)
    return time.time() - t0


def cpu_baseline(cfg, inp, budget_s):
    """Time the float64 oracle (untuned) on this host's cores: a process pool
    with one worker per core of this process's affinity (at most 16) and one
    BLAS thread per worker, on a bounded sample of the workload: one decode
    sequence per worker (one query token, all heads, the full cache), or
    query tokens of a chunk workload (all heads, the whole window; the cache
    build excluded)."""
    import multiprocessing as mp
    import numpy as np
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"                       # read by each worker's BLAS at its NumPy import
    chunk = not cfg.cache_given
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers, initializer=_oracle_worker_init, initargs=(cfg.name, chunk)) as pool:
            pool.map(time.sleep, [0.0] * workers, chunksize=1)      # every worker initialised
            if not chunk:
                n = min(cfg.batch, workers)
                tasks = list(range(n))
                what = (f"{n} of {cfg.batch} sequences (1 query token each, all {cfg.n_heads} heads, full "
                        f"{cfg.n_frames}-token cache)")
            else:
                n = workers * max(1, int(budget_s // 8))
                tasks = [int(t) for t in np.linspace(0, cfg.n_q - 1, n).astype(int)]
                what = (f"{n} of {cfg.n_q} query tokens of sample 0 (all {cfg.n_heads} heads, full key window; "
                        f"cache build excluded)")
            t0 = time.time()
            per = pool.map(_oracle_task, tasks, chunksize=1)
            wall = time.time() - t0
        return {"value": round(len(tasks) / wall, 4), "unit": "query-tokens/s", "cores": workers, "kind": "oracle",
                "sample": f"{what} on a pool of {workers} processes with one BLAS thread each: {wall:.1f} s wall, "
                          f"{sum(per):.1f} s of oracle work"}
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


if __name__ == "__main__":
    main()
