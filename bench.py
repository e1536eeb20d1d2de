#!/usr/bin/env python3
"""Benchmark of the VDN hybrid attention forward on one MI355X.

One step = one call of vdn_hybrid_attn_fwd (gate GEMM, window/anchor softmax,
VDA gram / solve / scan / readout, output GEMM) over one batch of seeded
synthetic bf16 input already resident in HBM.  The default workload is the
102-latent-frame layer: batch 1, 24 heads, head_dim 128 (D = 3072),
102 frames x 4032 tokens (411,264 tokens), 5-frame chunks, +-1 chunk, first
and last frame anchors.

Prints one JSON line: tokens/s and ms per layer call (wall clock over the K
timed calls, plus the median and minimum of the per-call HIP-event times), the
dominant kernel's roofline fraction (window softmax, MFMA bf16) from HIP
events recorded in the timed region, per-phase milliseconds, and the fp64 CPU
oracle timed on a bounded sample of the same workload on this host.

After the forward, the same line carries `vda_backward`: the linear-branch
gradient (vda_scan_bwd) timed on the same workload, per phase against HBM;
`scan_workload`: the linear branch alone (vda_scan_fwd) on its own workload,
B1 H8 d64 T42 N1560, with the scan's time per frame step; and `layer_T42`:
the 42-latent-frame layer (B1 H24 d128 N4032).

    python bench.py [--steps K] [--warmup W] [--config 4] [--no-cpu-baseline] [--bwd-steps 3]

With --sweep it instead runs the batch-2 length sweep (B2 H24 d128 N4032,
T = 42, 62, 82, 102 latent frames): the hybrid layer and the dense
full-softmax baseline (every key allowed, one output projection, no gates) on
identical inputs, one JSON line per length with both layer times, the
softmax-kernel times, the speedup and the softmax density.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "hybrid attn fwd tokens/s + ms/layer @102 latent frames; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

# HBM bytes each phase moves per call (FETCH_SIZE + WRITE_SIZE of its kernels, FETCH_SIZE scaled by a plain
# 1 GiB copy measured in the same process), by workload, from the rocprofv3 counter passes summarised in
# profiles/*_counters.md.  A figure is reported only while the sources of the phase's kernels hash to the
# version the counters were taken on; after any change to them it is reported as null.
COUNTER_TRAFFIC = {
    "hybrid layer B1 H24 d128 T102 N4032": {
        "gate_gemm": 27818898264,
        "key_norms": 2528918822,
        "window_attn": 202261787002,
        "anchor_merge": 710121606,
        "vda_gram": 5374755541,
        "vda_solve": 321107363,
        "vda_scan": 947370309,
        "vda_readout": 7901734562,
        "out_gemm": 26780832459
    },
    "hybrid layer B1 H24 d128 T102 N4032 mxfp8": {
        "window_attn": 183153494679,
        "mxfp8_quantize": 7659447006
    },
    "hybrid layer B1 H24 d128 T102 N4032 bwd": {
        "bwd_recompute": 7284527134,
        "bwd_token": 23391046577,
        "bwd_scan": 1274386041,
        "bwd_frame": 5567570132,
        "bwd_kv_gemm": 10453076697
    },
    "VDA scan B1 H8 d64 T42 N1560": {
        "vda_gram": 145294669,
        "vda_solve": 11091768,
        "vda_scan": 22079605,
        "vda_readout": 186676697
    },
    "hybrid layer B1 H24 d128 T42 N4032": {
        "gate_gemm": 11459876583,
        "key_norms": 1041320133,
        "window_attn": 97548988098,
        "anchor_merge": 401536381,
        "vda_gram": 2213162048,
        "vda_solve": 132282439,
        "vda_scan": 379714950,
        "vda_readout": 3253857106,
        "out_gemm": 10500861517
    }
}
PHASE_SOURCES = {      # phase -> source group of its kernels
    "gate_gemm": "gemm", "out_gemm": "gemm", "window_attn": "window", "anchor_merge": "window", "key_norms": "window",
    "vda_gram": "vda", "vda_solve": "vda", "vda_scan": "vda", "vda_readout": "vda", "mxfp8_quantize": "mxfp8",
    "bwd_recompute": "vda+bwd", "bwd_token": "bwd",
    "bwd_scan": "bwd", "bwd_frame": "bwd", "bwd_kv_gemm": "bwd",
}
SOURCE_GROUPS = {
    "window": ("window_attn.hip",), "gemm": ("gemm.hip",), "vda": ("vda.hip",), "mxfp8": ("mxfp8.hip",),
    "bwd": ("vda_bwd.hip", "vda_bwd.h"), "vda+bwd": ("vda.hip", "vda_bwd.hip", "vda_bwd.h"),
}
SOURCE_SHA = {
    "window": "387d4af33907e61b", "gemm": "ca60a1396242bbce", "vda": "71ddd2f45e486dc2", "mxfp8": "8cdcfa773199d9a4",
    "bwd": "cdf096da5a826c0d", "vda+bwd": "633b208094b4abf4", "common": "9c829e344fbc21af"
}


def _sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "video_diffusion_hybrid_vda_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, phase):
    """Counter-measured HBM bytes per call of `phase` on `workload`, or None if there is no such figure or
    the phase's kernel sources (or the shared headers) changed since it was taken."""
    t = COUNTER_TRAFFIC.get(workload, {}).get(phase)
    if t is None and workload.endswith(" mxfp8"):
        # MXFP8 mode changes only the softmax branch's kernels; the others run as in bf16 mode
        t = COUNTER_TRAFFIC.get(workload[:-len(" mxfp8")], {}).get(phase)
    grp = PHASE_SOURCES.get(phase)
    if t is None or grp is None or _sha(("vdn_common.h", "vdn_internal.h")) != SOURCE_SHA["common"]:
        return None
    for g in grp.split("+"):
        if _sha(SOURCE_GROUPS[g]) != SOURCE_SHA[g]:
            return None
    return t


def frame_key_counts(T, C, W, a0, a1):
    """Allowed key frames of each query frame under the chunk-window/anchor rule."""
    counts = []
    for t in range(T):
        if (a0 and t == 0) or (a1 and t == T - 1):
            counts.append(T)
            continue
        c = t // C
        lo, hi = max(0, (c - W) * C), min(T, (c + W + 1) * C)
        n = hi - lo
        if a0 and lo > 0:
            n += 1
        if a1 and hi < T:
            n += 1
        counts.append(n)
    return counts


def window_flops(cfg):
    """Algorithmic flops of one softmax-branch launch: 2 * d flops for q.k and
    2 * d for p*v per allowed (query, key) pair; masked pairs are not counted."""
    pairs_per_head = cfg.tokens_per_frame ** 2 * sum(
        frame_key_counts(cfg.frames, cfg.chunk_frames, cfg.window_chunks,
                         cfg.anchor_first, cfg.anchor_last))
    return 4 * cfg.head_dim * cfg.batch * cfg.heads * pairs_per_head, pairs_per_head


def phase_rooflines(cfg, phases, gated=True, mode=""):
    """Achieved rate of each hot-path kernel against its own roofline, from the library's per-phase
    HIP-event times: algorithmic bytes (HBM-bound kernels) or flops (MFMA-bound kernels) per call, with the
    bytes the counters measured per call beside them (`traffic`, null when not measured on these sources)."""
    B, H, T, N, d = cfg.batch, cfg.heads, cfg.frames, cfg.tokens_per_frame, cfg.head_dim
    L, D = T * N, cfg.model_dim
    es = 2 if cfg.dtype == "bf16" else 4
    frames = B * H * T
    tok = B * L * D * es                       # one [B, L, D] activation tensor
    dd4 = frames * d * d * 4                   # one fp32 d x d matrix per frame-head
    out = {}

    def ms(name):
        n, tot = phases.get(name, (0, 0.0))
        return tot / n if n else None

    def hbm(name, nbytes):
        t = ms(name)
        if t:
            gbs = nbytes / (t * 1e-3) / 1e9
            out[name] = {"bound": "hbm", "algorithmic_gb": round(nbytes / 1e9, 3), "ms": round(t, 3),
                         "achieved_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(cfg.name + mode, name)}

    def mfma(name, flops):
        t = ms(name)
        if t:
            tf = flops / (t * 1e-3) / 1e12
            out[name] = {"bound": "mfma", "algorithmic_tflop": round(flops / 1e12, 3), "ms": round(t, 3),
                         "achieved_tflops": round(tf, 1), "peak_tflops": PEAK_BF16_TFLOPS,
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(cfg.name + mode, name)}

    # K and V read once; A_t and B_t written (fp32)
    hbm("vda_gram", 2 * tok + 2 * dd4)
    # the softmax kernel's fixed-maximum bound: K read once
    hbm("key_norms", tok)
    # MXFP8 mode: q and k read (bf16), their codes (1 byte per element) and scales (1 per 32) written
    hbm("mxfp8_quantize", 2 * tok + 2 * (tok // es) * (1 + 1 / 32))
    # Q, gate (when given) and output once; both directions' states once per frame
    hbm("vda_readout", (3 if gated else 2) * tok + 2 * dd4)
    mfma("gate_gemm", 2.0 * B * L * D * 2 * D)
    mfma("out_gemm", 2.0 * B * L * 2 * D * D)
    t = ms("vda_scan")
    if t:
        # per frame-head and direction: M_t and B_t read (fp32); S_t written as hi/lo bf16 pairs
        # (bf16 I/O) and as fp32 where the readout reads it (fp32 I/O, or head_dim 32)
        keeps_fp32 = not (es == 2 and d in (64, 128))
        scan_bytes = 2 * frames * (2 * d * d * 4 + (d * d * 4 if keeps_fp32 else 0)
                                   + (2 * d * d * 2 if es == 2 else 0))
        out["vda_scan"] = {"bound": "latency", "ms": round(t, 3), "frame_steps": T,
                           "us_per_step": round(t * 1e3 / T, 2),
                           "algorithmic_gb": round(scan_bytes / 1e9, 3),
                           "achieved_gbs": round(scan_bytes / (t * 1e-3) / 1e9, 1),
                           "frac_of_hbm_peak": round(scan_bytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                           "traffic": measured_traffic(cfg.name + mode, "vda_scan")}
    t = ms("vda_solve")
    if t:
        out["vda_solve"] = {"bound": "latency", "ms": round(t, 3), "systems": frames,
                            "us_per_system_per_cu": round(t * 1e3 * 256 / frames, 2),
                            "traffic": measured_traffic(cfg.name + mode, "vda_solve")}
    return out


def host_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count()}


def timed_calls(fn, steps, warmup):
    """Run fn warmup times, then `steps` times with a torch (HIP) event pair
    around each call on the current stream; returns (wall ms per call,
    per-call event ms list)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


PAGES_SWEEP = {42: {"density_pct": 42.08, "speedup": 1.8}, 102: {"density_pct": 19.98, "speedup": 3.2}}


def length_sweep(args):
    """Hybrid layer vs dense full-softmax layer on identical inputs, B2 H24 d128 N4032."""
    import torch
    from video_diffusion_hybrid_vda_amd import synth, vdn
    torch.cuda.set_device(0)
    base = synth.CONFIGS[5]
    for T in args.sweep_frames:
        cfg = base.replace(frames=T)
        inp = synth.make_inputs(cfg, device="cuda", with_layer=True)
        shape = vdn.shape_from_config(cfg)
        B, L, D = cfg.batch, cfg.seq_len, cfg.model_dim
        out = torch.empty(B, L, D, dtype=torch.bfloat16, device="cuda")
        ws_h = vdn.workspace(shape, vdn.VDN_OP_HYBRID)

        def hybrid():
            vdn.vdn_hybrid_attn_fwd(shape, inp["x"], inp["q"], inp["k"], inp["v"], inp["gamma"],
                                    inp["beta"], inp["w_gs"], inp["w_gl"], inp["rms_w"], inp["w_os"],
                                    inp["w_ol"], out, ws_h)

        vdn.vdn_timing_start()
        _, h_ms = timed_calls(hybrid, args.sweep_steps, 1)
        ph_h = vdn.vdn_timing_stop()
        del ws_h
        ws_d = vdn.workspace(shape, vdn.VDN_OP_DENSE_ATTN)

        def dense():
            vdn.vdn_dense_attn_fwd(shape, inp["q"], inp["k"], inp["v"], inp["w_os"], out, ws_d)

        vdn.vdn_timing_start()
        _, d_ms = timed_calls(dense, args.sweep_steps, 1)
        ph_d = vdn.vdn_timing_stop()
        del ws_d
        _, pairs = window_flops(cfg)
        win_ms = ph_h["window_attn"][1] / ph_h["window_attn"][0]
        den_ms = ph_d["window_attn"][1] / ph_d["window_attn"][0]
        dense_flops = 4 * cfg.head_dim * B * cfg.heads * float(L) ** 2
        line = {
            "sweep": "hybrid vs dense layer", "workload": cfg.name.replace("{42,62,82,102}", str(T)),
            "frames": T, "tokens": B * L, "softmax_density": round(pairs / float(L) ** 2, 5),
            "hybrid_ms_median": round(median(h_ms), 2), "hybrid_ms_min": round(min(h_ms), 2),
            "dense_ms_median": round(median(d_ms), 2), "dense_ms_min": round(min(d_ms), 2),
            "layer_speedup": round(median(d_ms) / median(h_ms), 3),
            "softmax_kernel_ms": {"window": round(win_ms, 2), "dense": round(den_ms, 2)},
            "softmax_kernel_speedup": round(den_ms / win_ms, 3),
            "dense_softmax_tflops": round(dense_flops / (den_ms * 1e-3) / 1e12, 1),
            "calls": args.sweep_steps, "warmup": 1, "dtype": "bf16", "data": "synthetic",
            "pages_h200": PAGES_SWEEP.get(T),
        }
        print(json.dumps(line), flush=True)
        del inp, out
        torch.cuda.empty_cache()


def blas_threads():
    """Host threads given to the oracle's BLAS: the CPUs this process may run
    on, capped by OMP_NUM_THREADS when that is set."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(n, 1)


def cpu_full_runs():
    """The oracle on the two workloads small enough to run whole: the tiny fp32
    layer (B1 H1 d32 T10 N16) and the linear branch at the scan workload (B1 H8
    d64 T42 N1560, both scans and the RMSNorm readout of every token)."""
    import numpy as np
    from oracle import vdn_oracle as O
    from video_diffusion_hybrid_vda_amd import synth
    f64 = lambda t: t.double().numpy()  # noqa: E731
    out = {}
    cfg = synth.CONFIGS[1]
    inp = {k: f64(v) for k, v in synth.make_inputs(cfg, device="cpu").items()}
    t0 = time.perf_counter()
    O.hybrid_layer(*(inp[k] for k in ("x", "q", "k", "v", "gamma", "beta", "w_gs", "w_gl", "rms_w", "w_os",
                                      "w_ol")), eps=cfg.rms_eps)
    dt = time.perf_counter() - t0
    out["tiny_layer"] = {"workload": cfg.name, "s": round(dt, 4), "tokens_per_s": round(cfg.seq_len / dt, 1)}
    cfg = synth.CONFIGS[2]
    inp = {k: f64(v) for k, v in synth.make_inputs(cfg, device="cpu", with_layer=False).items()}
    t0 = time.perf_counter()
    O.vda_branch(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], np.ones(cfg.model_dim), cfg.rms_eps)
    dt = time.perf_counter() - t0
    out["scan_workload"] = {"workload": cfg.name, "s": round(dt, 3), "tokens_per_s": round(cfg.seq_len / dt, 1)}
    return out


def cpu_baseline(cfg, inp):
    """The fp64 oracle, unmodified, timed on this host with its BLAS thread
    count set explicitly.  The benchmark's layer is timed on a bounded sample
    (one head's full forward+backward scans, a sample of readout tokens, softmax
    rows of an interior and an anchor frame, gate/projection rows) and scaled to
    the whole layer: the softmax rows of each query frame by that frame's
    allowed key frames, the rest by exact token and head counts.  The two small
    workloads are also run whole."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import vdn_oracle as O
    threads = blas_threads()
    with threadpool_limits(limits=threads, user_api="blas"):
        B, H, T, N, d = cfg.batch, cfg.heads, cfg.frames, cfg.tokens_per_frame, cfg.head_dim
        L = T * N
        f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
        q, k, v = f64(inp["q"][0, 0]), f64(inp["k"][0, 0]), f64(inp["v"][0, 0])
        gamma, beta = f64(inp["gamma"][0, 0]), f64(inp["beta"][0, 0])
        w = np.ones(d)

        t0 = time.perf_counter()
        sf, sb = O.vda_states(k, v, gamma, beta)
        t_states = time.perf_counter() - t0

        tmid = min(7, T - 1)
        R = min(256, N)
        t0 = time.perf_counter()
        O.vda_readout(q[tmid, :R], sf[tmid], sb[tmid], w, cfg.rms_eps)
        t_readout_tok = (time.perf_counter() - t0) / R

        allowed = O.allowed_frames(T, cfg.chunk_frames, cfg.window_chunks, cfg.anchor_first, cfg.anchor_last)
        Rs = min(64, N)
        t0 = time.perf_counter()
        O.window_attention(q, k, v, allowed, 1 / np.sqrt(d), np.arange(tmid * N, tmid * N + Rs))
        t_win_tok = (time.perf_counter() - t0) / Rs
        t0 = time.perf_counter()
        O.window_attention(q, k, v, allowed, 1 / np.sqrt(d), np.arange(0, Rs))
        t_anchor_tok = (time.perf_counter() - t0) / Rs

        xr = f64(inp["x"][0, :Rs])
        wgs, wgl, wos, wol = (f64(inp[n]) for n in ("w_gs", "w_gl", "w_os", "w_ol"))
        t0 = time.perf_counter()
        g_s, g_l = O.gates(xr, wgs, wgl)
        _ = (g_s * xr) @ wos + (g_l * xr) @ wol
        t_gemm_tok = (time.perf_counter() - t0) / Rs

        counts = frame_key_counts(T, cfg.chunk_frames, cfg.window_chunks, cfg.anchor_first, cfg.anchor_last)
        anchors = {0} if cfg.anchor_first else set()
        if cfg.anchor_last:
            anchors.add(T - 1)
        per_key_frame = t_win_tok / counts[tmid]
        t_softmax = sum(N * (t_anchor_tok if t in anchors else per_key_frame * counts[t]) for t in range(T))
        total = B * (H * (t_states + L * t_readout_tok + t_softmax) + L * t_gemm_tok)
        full = cpu_full_runs()
    sample = (f"head 0 of {H}: VDA forward+backward scans over all {T} frames; readout of {R} tokens; "
              f"softmax of {Rs} tokens of frame {tmid} ({counts[tmid]} key frames) and {Rs} of anchor frame 0; "
              f"gates and projections of {Rs} tokens; scaled to the B{B} H{H} T{T} N{N} layer by exact head and "
              f"token counts, the softmax of each query frame by its allowed key frames (extrapolated layer "
              f"time {total:.0f} s)")
    return {"value": B * L / total, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "full_runs": full, "host": host_info()}


def time_scan_workload(vdn, torch, steps):
    """The linear branch alone (vda_scan_fwd: Gram, solve, both scans, RMSNorm
    readout, no gate) on its own workload, B1 H8 d64 T42 N1560 bf16."""
    from video_diffusion_hybrid_vda_amd import synth
    cfg = synth.CONFIGS[2]
    inp = synth.make_inputs(cfg, device="cuda", with_layer=False)
    shape = vdn.shape_from_config(cfg)
    ws = vdn.workspace(shape, vdn.VDN_OP_VDA_SCAN)
    B, L, D = cfg.batch, cfg.seq_len, cfg.model_dim
    out = torch.empty(B, L, D, dtype=torch.bfloat16, device="cuda")

    def call():
        vdn.vda_scan_fwd(shape, inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], None, None, out, None, ws)

    call()
    torch.cuda.synchronize()
    # the call alone, then its phases with the library's event timer on (at this
    # size the timer's eight event records per call are a visible share of it)
    ms, calls = timed_calls(call, steps, 0)
    vdn.vdn_timing_start()
    timed_calls(call, steps, 0)
    ph = vdn.vdn_timing_stop()
    tok_bytes = B * L * D * 2
    # q, k, v read and out written once (bf16); every d x d statistic, transition and state moved once
    call_bytes = 4 * tok_bytes
    return {"workload": cfg.name, "entry_point": "vda_scan_fwd (no gate, unit RMSNorm weight)",
            "value": B * L / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": round(ms, 4),
            "call_ms_median": round(median(calls), 4), "steps": steps,
            "token_bytes_gb": round(call_bytes / 1e9, 4),
            "token_bytes_frac_of_hbm_peak": round(call_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "phases_ms": {k: round(v[1] / max(v[0], 1), 4) for k, v in ph.items() if v[0] > 0},
            "kernel_rooflines": phase_rooflines(cfg, ph, gated=False)}


def time_layer(vdn, torch, cfg_id, steps):
    """The whole hybrid layer on another workload (by default the 42-frame layer)."""
    from video_diffusion_hybrid_vda_amd import synth
    cfg = synth.CONFIGS[cfg_id]
    inp = synth.make_inputs(cfg, device="cuda", with_layer=True)
    shape = vdn.shape_from_config(cfg)
    ws = vdn.workspace(shape, vdn.VDN_OP_HYBRID)
    B, L, D = cfg.batch, cfg.seq_len, cfg.model_dim
    out = torch.empty(B, L, D, dtype=torch.bfloat16, device="cuda")

    def call():
        vdn.vdn_hybrid_attn_fwd(shape, inp["x"], inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"],
                                inp["w_gs"], inp["w_gl"], inp["rms_w"], inp["w_os"], inp["w_ol"], out, ws)

    call()
    torch.cuda.synchronize()
    vdn.vdn_timing_start()
    ms, calls = timed_calls(call, steps, 0)
    ph = vdn.vdn_timing_stop()
    flops, pairs = window_flops(cfg)
    n, tot = ph["window_attn"]
    wms = tot / max(n, 1)
    ach = flops / (wms * 1e-3) / 1e12
    return {"workload": cfg.name, "value": B * L / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": round(ms, 3),
            "call_ms_median": round(median(calls), 3), "call_ms_min": round(min(calls), 3), "steps": steps,
            "softmax_density": round(pairs / float(L) ** 2, 5),
            "roofline": {"bound": "mfma", "kernel": "window_attn", "achieved": round(ach, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                         "algorithmic_tflop_per_launch": round(flops / 1e12, 3), "avg_ms": round(wms, 3),
                         "traffic": measured_traffic(cfg.name, "window_attn")},
            "phases_ms": {k: round(v[1] / max(v[0], 1), 3) for k, v in ph.items() if v[0] > 0},
            "kernel_rooflines": phase_rooflines(cfg, ph)}


# kernels of the gradient's token-side phases at head_dim 128, bf16 I/O
BWD_KERNELS = {"bwd_token": "tok_grad_bf16_d128_kernel", "bwd_kv_gemm": "kv_grad_bf16_d128_kernel"}


def time_backward(cfg, inp, vdn, torch, steps):
    """Time the linear-branch gradient (vda_scan_bwd) on the workload: gradient of
    <d_out, ungated linear-branch output> with respect to q, k, v, gamma, beta and
    the RMSNorm weight, d_out seeded N(0, 1) in bf16.  Each token-side phase is
    reported against HBM with its algorithmic bytes (every tensor it must read or
    write once); the longer of the two is the roofline entry."""
    B, H, d, T, N = cfg.batch, cfg.heads, cfg.head_dim, cfg.frames, cfg.tokens_per_frame
    L, D = cfg.seq_len, cfg.model_dim
    shape = vdn.shape_from_config(cfg)
    ws = vdn.workspace(shape, vdn.VDN_OP_VDA_BWD)
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 4242)
    d_out = torch.randn(B, L, D, device="cuda", generator=g).to(torch.bfloat16)
    grads = {n: torch.empty_like(inp[n]) for n in ("q", "k", "v")}
    dgamma = torch.empty(B, H, T, dtype=torch.float32, device="cuda")
    dbeta = torch.empty_like(dgamma)
    drms = torch.empty(D, dtype=torch.float32, device="cuda")

    def call():
        vdn.vda_scan_bwd(shape, inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], inp["rms_w"], d_out,
                         grads["q"], grads["k"], grads["v"], dgamma, dbeta, drms, ws)

    call()
    torch.cuda.synchronize()
    vdn.vdn_timing_start()
    ms, calls = timed_calls(call, steps, 0)
    ph = vdn.vdn_timing_stop()
    ph_ms = {k: round(v[1] / max(v[0], 1), 3) for k, v in ph.items() if v[0] > 0}
    tok = B * H * L * d          # elements of one [B, H, L, d] token tensor
    nbytes = {                   # algorithmic HBM bytes per call of each token-side phase (bf16 tokens)
        "bwd_token": 3 * tok * 2,                            # read q and d_out, write dq
        "bwd_kv_gemm": 4 * tok * 2,                          # read k, v; write dk, dv
    }
    kern = {}
    for k, b in nbytes.items():
        if k in ph_ms:
            gbs = b / (ph_ms[k] * 1e-3) / 1e9
            kern[k] = {"bound": "hbm", "achieved_GBps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                       "algorithmic_GB": round(b / 1e9, 3), "avg_ms": ph_ms[k],
                       "traffic": measured_traffic(cfg.name + " bwd", k)}
    dom = max(nbytes, key=lambda k: ph_ms.get(k, 0.0))
    del ws
    return {"mode": "gradient of the ungated linear-branch output w.r.t. q, k, v, gamma, beta and the "
                    "RMSNorm weight (vda_scan_bwd; forward quantities recomputed inside)",
            "value": B * L / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "steps": steps,
            "call_ms_median": round(median(calls), 3), "phases_ms": ph_ms,
            "roofline": dict(kern[dom], kernel=dom + " (" + BWD_KERNELS.get(dom, "?") + ")", peak=PEAK_HBM_GBS,
                             unit="GB/s",
                             achieved=kern[dom]["achieved_GBps"]),
            "kernel_rooflines": kern}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, help="workload index (3 or 4 are full layers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="run the batch-2 hybrid-vs-dense length sweep instead of the single workload")
    ap.add_argument("--sweep-frames", type=int, nargs="+", default=[42, 62, 82, 102])
    ap.add_argument("--sweep-steps", type=int, default=3)
    ap.add_argument("--softmax-mxfp8", action="store_true",
                    help="time the layer with MXFP8 softmax-branch scores instead of bf16 ones")
    ap.add_argument("--mxfp8-steps", type=int, default=3,
                    help="after the bf16 measurement, also time this many calls in MXFP8 mode (0: skip)")
    ap.add_argument("--bwd-steps", type=int, default=3,
                    help="after the forward measurement, also time this many calls of the linear-branch "
                         "gradient (vda_scan_bwd) on the same workload (0: skip)")
    ap.add_argument("--scan-steps", type=int, default=20,
                    help="also time this many calls of vda_scan_fwd on the scan workload B1 H8 d64 T42 N1560 "
                         "(0: skip)")
    ap.add_argument("--t42-steps", type=int, default=5,
                    help="also time this many calls of the 42-frame layer B1 H24 d128 T42 N4032 (0: skip)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="before the timed region, run one plain device-to-device copy of this many MiB "
                         "(a known-traffic kernel for scaling HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        length_sweep(args)
        return

    import torch
    from video_diffusion_hybrid_vda_amd import synth, vdn

    cfg = synth.CONFIGS[args.config]
    torch.cuda.set_device(0)
    inp = synth.make_inputs(cfg, device="cuda", with_layer=True)
    shape = vdn.shape_from_config(cfg, softmax_mxfp8=args.softmax_mxfp8)
    ws = vdn.workspace(shape, vdn.VDN_OP_HYBRID)
    B, L, D = cfg.batch, cfg.seq_len, cfg.model_dim
    out = torch.empty(B, L, D, dtype=torch.bfloat16, device="cuda")

    def layer(sh, w):
        vdn.vdn_hybrid_attn_fwd(sh, inp["x"], inp["q"], inp["k"], inp["v"], inp["gamma"],
                                inp["beta"], inp["w_gs"], inp["w_gl"], inp["rms_w"], inp["w_os"],
                                inp["w_ol"], out, w)

    def step():
        layer(shape, ws)

    if args.calibrate_copy_mb > 0:
        src = torch.ones(args.calibrate_copy_mb << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    vdn.vdn_timing_start()
    ms_per_step, call_ms = timed_calls(step, args.steps, 0)
    phases = vdn.vdn_timing_stop()

    flops, pairs = window_flops(cfg)
    n_attn, attn_ms = phases["window_attn"]
    attn_avg_ms = attn_ms / max(n_attn, 1)
    achieved = flops / (attn_avg_ms * 1e-3) / 1e12
    density = pairs / float(L) ** 2
    phase_ms = {k: round(v[1] / max(v[0], 1), 3) for k, v in phases.items() if v[0] > 0}
    # MXFP8 scores: the q.k half of the window kernel's flops at the fp8 peak, the P V half at bf16
    mx_peak = flops / (0.5 * flops / PEAK_FP8_TFLOPS + 0.5 * flops / PEAK_BF16_TFLOPS)

    def mx_roofline(ms):
        a = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": "window_attn_mxfp8", "achieved": round(a, 2),
                "peak": round(mx_peak, 1), "unit": "TFLOP/s", "frac": round(a / mx_peak, 4),
                "peak_note": "q.k half at the 5.0 PFLOP/s fp8 peak, P V half at the 2.5 PFLOP/s bf16 peak",
                "algorithmic_tflop_per_launch": round(flops / 1e12, 3), "avg_ms": round(ms, 3),
                "traffic": measured_traffic(cfg.name + " mxfp8", "window_attn")}

    mxfp8 = None
    if not args.softmax_mxfp8 and args.mxfp8_steps > 0:
        # the same layer with MXFP8 softmax-branch scores, timed after the bf16 region
        shape8 = vdn.shape_from_config(cfg, softmax_mxfp8=True)
        ws = None
        ws8 = vdn.workspace(shape8, vdn.VDN_OP_HYBRID)
        layer(shape8, ws8)
        torch.cuda.synchronize()
        vdn.vdn_timing_start()
        ms8, call8 = timed_calls(lambda: layer(shape8, ws8), args.mxfp8_steps, 0)
        ph8 = vdn.vdn_timing_stop()
        ph8_ms = {k: round(v[1] / max(v[0], 1), 3) for k, v in ph8.items() if v[0] > 0}
        mxfp8 = {"mode": "softmax-branch scores from MXFP8 q and k (OCP E4M3, E8M0 per 32 elements); "
                         "P V, gates, linear branch and projections bf16",
                 "value": B * L / (ms8 * 1e-3), "unit": "tokens/s", "ms_per_step": ms8,
                 "steps": args.mxfp8_steps, "call_ms_median": round(median(call8), 3),
                 "roofline": mx_roofline(ph8_ms["window_attn"]), "phases_ms": ph8_ms,
                 "kernel_rooflines": phase_rooflines(cfg, ph8, mode=" mxfp8")}
        del ws8

    backward = None
    if args.bwd_steps > 0:
        backward = time_backward(cfg, inp, vdn, torch, args.bwd_steps)
    cpu = None if args.no_cpu_baseline else cpu_baseline(cfg, inp)
    inp = ws = out = None      # free the benchmark layer's buffers before the other workloads
    torch.cuda.empty_cache()
    scan = time_scan_workload(vdn, torch, args.scan_steps) if args.scan_steps > 0 else None
    layer42 = time_layer(vdn, torch, 3, args.t42_steps) if args.t42_steps > 0 and args.config != 3 else None

    result = {
        "metric": METRIC,
        "value": B * L / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+mxfp8 scores" if args.softmax_mxfp8 else "bf16",
        "data": "synthetic (seeded; Q,V,x ~ N(0,1), K rows unit-norm, beta ~ U(0.1,1), gamma ~ U(0.9,1), W ~ N(0,0.02^2))",
        "config": {"workload": cfg.name, "batch": B, "heads": cfg.heads, "head_dim": cfg.head_dim,
                   "frames": cfg.frames, "tokens_per_frame": cfg.tokens_per_frame, "tokens": B * L,
                   "chunk_frames": cfg.chunk_frames, "window_chunks": cfg.window_chunks,
                   "anchors": "first+last", "softmax_density": round(density, 5)},
        "roofline": mx_roofline(attn_avg_ms) if args.softmax_mxfp8 else
                    {"bound": "mfma", "kernel": "window_attn", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "algorithmic_tflop_per_launch": round(flops / 1e12, 3), "avg_ms": round(attn_avg_ms, 3),
                     "traffic": measured_traffic(cfg.name, "window_attn")},
        "kernel_rooflines": phase_rooflines(cfg, phases),
        "call_ms_median": round(median(call_ms), 3),
        "call_ms_min": round(min(call_ms), 3),
        "phases_ms": phase_ms,
    }
    if mxfp8 is not None:
        result["mxfp8_softmax"] = mxfp8
    if backward is not None:
        result["vda_backward"] = backward
    if scan is not None:
        result["scan_workload"] = scan
    if layer42 is not None:
        result["layer_T42"] = layer42
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
