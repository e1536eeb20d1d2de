"""GPU parity of the linear-branch gradient (vda_scan_bwd) against the fp64
oracle (oracle.vda_backward, pinned by finite differences of the forward
oracle in test_vda_backward_oracle.py).

Error measure (tests/measure.py), per output: max |gpu - oracle| / RMS(oracle),
bounded by 2e-2 for bf16 I/O and 1e-4 for fp32 I/O.  For bf16 I/O the
token-side products run on bf16 MFMA with fp32 operands split into hi and lo
bf16 halves and fp32 accumulation; the rest is fp32.  dq, dk and dv are
gradients, heavy-tailed (max/RMS near 10 at the headline shape), so for those
bf16 outputs the bar may apply to the error beyond each element's own bf16
rounding, with all three figures logged; dgamma and the RMSNorm weight's
gradient are held to the plain bar, and dbeta to the plain bar plus the fp32
evaluation error of its cancelling sum (measure.check_sum, with the term
mass from the oracle).  Small
shapes are compared element by element for all six outputs; they span
several 64-row product tiles with ragged tails (N = 70, 130, 100), head_dim
32/64/128, batch > 1, frames with beta = 0, and context tokens (whose rows
of dq, dk, dv must be zero).  The 102-frame headline shape is compared on
whole heads: every gradient of one head depends on that head's inputs only.
"""
import sys
import time

import numpy as np
import pytest
import torch

from oracle.vda_backward import vda_branch_backward
from video_diffusion_hybrid_vda_amd import synth
from video_diffusion_hybrid_vda_amd.synth import VdnConfig

from measure import check, check_sum

pytestmark = pytest.mark.gpu



def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def vdn():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch: the HIP path cannot run")
    from video_diffusion_hybrid_vda_amd import vdn as binding
    return binding


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def grad_inputs(cfg, device):
    """Seeded inputs of the linear branch plus an RMSNorm weight and an upstream
    gradient d_out [B, Lt, D] of the output's dtype."""
    inp = synth.make_inputs(cfg, device="cpu", with_layer=False)
    B, H, d = cfg.batch, cfg.heads, cfg.head_dim
    Lt = cfg.frames * cfg.tokens_per_frame + cfg.context_tokens
    g = torch.Generator().manual_seed(cfg.seed + 77)
    inp["rms_w"] = 0.5 + torch.rand(H * d, generator=g)
    d_out = torch.randn(B, Lt, H * d, generator=g).to(synth.DTYPES[cfg.dtype])
    return {k: v.to(device) for k, v in inp.items()}, d_out.to(device)


def video(t, cfg):
    """[B, H, Lt, d] -> the video rows as [B, H, T, N, d] (fp64)."""
    B, H, T, N, d = cfg.batch, cfg.heads, cfg.frames, cfg.tokens_per_frame, cfg.head_dim
    return np64(t[:, :, :T * N]).reshape(B, H, T, N, d)


def d_out_heads(d_out, cfg):
    """[B, Lt, D] -> the video rows as [B, H, T, N, d] (fp64)."""
    B, H, T, N, d = cfg.batch, cfg.heads, cfg.frames, cfg.tokens_per_frame, cfg.head_dim
    return np64(d_out[:, :T * N]).reshape(B, T, N, H, d).transpose(0, 3, 1, 2, 4)


CASES = [
    ("B2H2_T6_N6_d32_f32", VdnConfig(2, 2, 32, 6, 6, dtype="f32", seed=81)),
    ("H2_T7_N70_d64_bf16", VdnConfig(1, 2, 64, 7, 70, dtype="bf16", seed=82)),
    ("T5_N130_d128_bf16", VdnConfig(1, 1, 128, 5, 130, dtype="bf16", seed=83)),
    ("T4_N100_d128_f32_beta0", VdnConfig(1, 1, 128, 4, 100, dtype="f32", beta_lo=0.0, seed=84)),
    ("T1_N9_d64_f32", VdnConfig(1, 1, 64, 1, 9, dtype="f32", seed=85)),
    ("H2_T6_N20_d32_ctx9_bf16", VdnConfig(1, 2, 32, 6, 20, dtype="bf16", context_tokens=9, seed=86)),
    ("B2H2_T7_N300_d128_ctx5_bf16", VdnConfig(2, 2, 128, 7, 300, dtype="bf16", context_tokens=5, seed=88)),
    # one partial 16-token tile per frame: seven of the eight waves of the
    # bf16 token-side and dK/dV kernels have no tile
    ("T3_N5_d128_bf16", VdnConfig(1, 1, 128, 3, 5, dtype="bf16", seed=89)),
]


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_vda_backward_small(vdn, name, cfg):
    log(f"[vda bwd] {name}")
    inp, d_out = grad_inputs(cfg, "cuda")
    if "beta0" in name:
        inp["beta"][0, 0, 1] = 0.0
    shape = vdn.shape_from_config(cfg)
    got = vdn.vda_scan_grad(shape, inp, d_out)
    torch.cuda.synchronize()
    ref = vda_branch_backward(video(inp["q"], cfg), video(inp["k"], cfg), video(inp["v"], cfg),
                              np64(inp["gamma"]), np64(inp["beta"]), np64(inp["rms_w"]), cfg.rms_eps,
                              d_out_heads(d_out, cfg))
    for n in ("q", "k", "v"):
        check(log, "d" + n, video(got[n], cfg), ref["d" + n], cfg.dtype, stress=True)
        if cfg.context_tokens:
            L = cfg.frames * cfg.tokens_per_frame
            assert torch.count_nonzero(got[n][:, :, L:]).item() == 0, n
    check(log, "dgamma", np64(got["gamma"]), ref["dgamma"], cfg.dtype)
    check_sum(log, "dbeta", np64(got["beta"]), ref["dbeta"], ref["dbeta_mass"], cfg.dtype)
    check(log, "drms_w", np64(got["rms_w"]), ref["drms_w"], cfg.dtype)
    if "beta0" in name:
        assert torch.count_nonzero(got["k"][0, 0, 100:200]).item() == 0
        assert torch.count_nonzero(got["v"][0, 0, 100:200]).item() == 0


def test_vda_backward_headline_two_heads(vdn):
    """B1 H24 d128 T102 N4032 bf16, the launch the benchmark times: every
    gradient of heads 0 and 23 against the oracle."""
    cfg = synth.CONFIGS[4]
    log(f"[vda bwd] {cfg.name}")
    t0 = time.time()
    inp, d_out = grad_inputs(cfg, "cuda")
    shape = vdn.shape_from_config(cfg)
    got = vdn.vda_scan_grad(shape, inp, d_out)
    torch.cuda.synchronize()
    log(f"  gpu done {time.time() - t0:.1f}s")
    T, N, d = cfg.frames, cfg.tokens_per_frame, cfg.head_dim
    dh = d_out_heads(d_out, cfg)
    for h in (0, 23):
        sl = lambda t: np64(t[0:1, h:h + 1]).reshape(1, 1, T, N, d)
        ref = vda_branch_backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), np64(inp["gamma"][0:1, h:h + 1]),
                                  np64(inp["beta"][0:1, h:h + 1]), np64(inp["rms_w"][h * d:(h + 1) * d]),
                                  cfg.rms_eps, dh[0:1, h:h + 1])
        log(f"  head {h} ({time.time() - t0:.1f}s)")
        for n in ("q", "k", "v"):
            check(log, "d" + n, sl(got[n]), ref["d" + n], "bf16", stress=True)
        check(log, "dgamma", np64(got["gamma"][0, h]), ref["dgamma"][0, 0], "bf16")
        check_sum(log, "dbeta", np64(got["beta"][0, h]), ref["dbeta"][0, 0], ref["dbeta_mass"][0, 0], "bf16")
        check(log, "drms_w", np64(got["rms_w"][h * d:(h + 1) * d]), ref["drms_w"], "bf16")


def test_vda_backward_scan_workload_two_heads(vdn):
    """B1 H8 d64 T42 N1560 bf16 (the linear-branch scan workload): every gradient
    of heads 0 and 7, whole, against the oracle."""
    cfg = synth.CONFIGS[2]
    log(f"[vda bwd] {cfg.name}")
    inp, d_out = grad_inputs(cfg, "cuda")
    got = vdn.vda_scan_grad(vdn.shape_from_config(cfg), inp, d_out)
    torch.cuda.synchronize()
    T, N, d = cfg.frames, cfg.tokens_per_frame, cfg.head_dim
    dh = d_out_heads(d_out, cfg)
    for h in (0, 7):
        sl = lambda t: np64(t[0:1, h:h + 1]).reshape(1, 1, T, N, d)
        ref = vda_branch_backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), np64(inp["gamma"][0:1, h:h + 1]),
                                  np64(inp["beta"][0:1, h:h + 1]), np64(inp["rms_w"][h * d:(h + 1) * d]),
                                  cfg.rms_eps, dh[0:1, h:h + 1])
        log(f"  head {h}")
        for n in ("q", "k", "v"):
            check(log, "d" + n, sl(got[n]), ref["d" + n], "bf16", stress=True)
        check(log, "dgamma", np64(got["gamma"][0, h]), ref["dgamma"][0, 0], "bf16")
        check_sum(log, "dbeta", np64(got["beta"][0, h]), ref["dbeta"][0, 0], ref["dbeta_mass"][0, 0], "bf16")
        check(log, "drms_w", np64(got["rms_w"][h * d:(h + 1) * d]), ref["drms_w"], "bf16")


@pytest.mark.parametrize("d", [64, 128])
def test_vda_backward_repeatable_and_range_checked(vdn, d):
    """Two calls on one workspace give bit-identical gradients (no atomics:
    every reduction has a fixed order); with the opt-in range check on,
    beta < 0 or gamma > 1 is rejected with VDN_ERR_PARAM_RANGE (-6) and the
    outputs are left untouched, and valid parameters pass unchanged."""
    cfg = VdnConfig(1, 2, d, 6, 50, dtype="bf16", seed=87)
    inp, d_out = grad_inputs(cfg, "cuda")
    shape = vdn.shape_from_config(cfg)
    ws = vdn.workspace(shape, vdn.VDN_OP_VDA_BWD)
    g1 = vdn.vda_scan_grad(shape, inp, d_out, ws=ws)
    g2 = vdn.vda_scan_grad(shape, inp, d_out, ws=ws)
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n
    prev = vdn.vdn_set_param_check(True)
    try:
        g3 = vdn.vda_scan_grad(shape, inp, d_out, ws=ws)
        torch.cuda.synchronize()
        for n in g1:
            assert torch.equal(g1[n], g3[n]), n
        for key, val in (("beta", -0.5), ("gamma", 1.5)):
            bad = dict(inp)
            bad[key] = inp[key].clone()
            bad[key][0, 1, 3] = val
            sentinel = torch.full_like(g1["q"], 7.0)
            with pytest.raises(vdn.VdnError) as ei:
                vdn.vda_scan_bwd(shape, bad["q"], bad["k"], bad["v"], bad["gamma"], bad["beta"], bad["rms_w"],
                                 d_out, sentinel, torch.empty_like(sentinel), torch.empty_like(sentinel),
                                 torch.empty_like(g1["gamma"]), torch.empty_like(g1["beta"]), None, ws)
            assert ei.value.status == -6, key
            torch.cuda.synchronize()
            assert torch.all(sentinel == 7.0).item(), key
    finally:
        vdn.vdn_set_param_check(prev)
