"""The allocation-free linear-branch entry point (vda_scan_fwd_noalloc)
against vda_scan_fwd on the same inputs, through the C ABI.

Both run the same kernels in the same order, the first on the library's
static scratch and the second on a caller workspace, so their outputs and
states must agree bit for bit (within the parity bar a fortiori).  Two calls
in a row, the second on a smaller shape, show that a call does not depend on
what an earlier call left in the shared scratch."""
import sys

import pytest
import torch

from video_diffusion_hybrid_vda_amd import synth
from video_diffusion_hybrid_vda_amd.synth import VdnConfig

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


def _both(vdn, cfg, with_gate, with_states):
    inp = synth.make_inputs(cfg, device="cuda", with_layer=False)
    B, H, d, Lt = cfg.batch, cfg.heads, cfg.head_dim, cfg.seq_len
    shape = vdn.shape_from_config(cfg)
    dt = synth.DTYPES[cfg.dtype]
    gate = None
    if with_gate:
        g = torch.Generator(device="cuda").manual_seed(cfg.seed + 3)
        gate = torch.rand(B, Lt, H * d, generator=g, device="cuda").to(dt)
    rms_w = (0.5 + torch.rand(H * d, generator=torch.Generator(device="cuda").manual_seed(cfg.seed + 4),
                              device="cuda"))
    out_ref, st_ref = vdn.vda_scan(shape, dict(inp, rms_w=rms_w), gate_l=gate, with_states=True)
    out = torch.full_like(out_ref, 3.0)
    states = torch.full_like(st_ref, 5.0) if with_states else None
    vdn.vda_scan_fwd_noalloc(shape, inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], rms_w, gate, out,
                             states)
    torch.cuda.synchronize()
    return out, out_ref, states, st_ref


@pytest.mark.parametrize("first,second", [
    (synth.CONFIGS[2], VdnConfig(1, 2, 128, 9, 200, dtype="bf16", seed=91)),
    (VdnConfig(2, 3, 64, 11, 70, dtype="f32", seed=92), VdnConfig(1, 1, 32, 5, 30, dtype="f32", seed=93)),
], ids=["scan_workload_then_d128", "f32_B2_then_tiny"])
def test_noalloc_matches_workspace_entry_point(vdn, first, second):
    for i, (cfg, gate, st) in enumerate(((first, False, True), (second, True, False))):
        log(f"[noalloc] call {i + 1}: B{cfg.batch} H{cfg.heads} d{cfg.head_dim} T{cfg.frames} "
            f"N{cfg.tokens_per_frame} {cfg.dtype} gate={gate} states={st}")
        out, out_ref, states, st_ref = _both(vdn, cfg, gate, st)
        assert torch.equal(out, out_ref)
        if st:
            assert torch.equal(states, st_ref)


def test_noalloc_rejects_oversized_shapes_and_checks_ranges(vdn):
    big = synth.CONFIGS[4]
    shape = vdn.shape_from_config(big)
    t = torch.empty(16, device="cuda")
    with pytest.raises(vdn.VdnError) as ei:
        vdn.vda_scan_fwd_noalloc(shape, t, t, t, t, t, None, None, t, None)
    assert ei.value.status == -4 and "scratch" in str(ei.value)
    cfg = VdnConfig(1, 2, 64, 9, 40, dtype="bf16", seed=94)
    inp = synth.make_inputs(cfg, device="cuda", with_layer=False)
    shape = vdn.shape_from_config(cfg)
    out = torch.empty(1, 9 * 40, 128, dtype=torch.bfloat16, device="cuda")
    bad = inp["beta"].clone()
    bad[0, 1, 2] = -0.5
    prev = vdn.vdn_set_param_check(True)
    try:
        with pytest.raises(vdn.VdnError) as ei:
            vdn.vda_scan_fwd_noalloc(shape, inp["q"], inp["k"], inp["v"], inp["gamma"], bad, None, None, out, None)
        assert ei.value.status == -6
        vdn.vda_scan_fwd_noalloc(shape, inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], None, None, out,
                                 None)
        torch.cuda.synchronize()
    finally:
        vdn.vdn_set_param_check(prev)
    assert torch.equal(out, vdn.vda_scan(shape, inp))
