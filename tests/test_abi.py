"""CPU checks of the C ABI: libvdn.so loads, exports every function that
include/vdn.h declares, and rejects bad arguments on the host before any HIP
call (these calls never launch a kernel, so no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vdn.h")
LIB = os.path.join(ROOT, "video_diffusion_hybrid_vda_amd", "libvdn.so")


@pytest.fixture(scope="module")
def vdn():
    if not os.path.exists(LIB):
        from video_diffusion_hybrid_vda_amd import build
        build.build()
    from video_diffusion_hybrid_vda_amd import vdn as binding
    return binding


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_declares_the_entry_points():
    fns = header_functions()
    for name in ("vdn_hybrid_attn_fwd", "vda_scan_fwd", "window_anchor_attn_fwd",
                 "vdn_dense_attn_fwd", "vdn_set_param_check", "vdn_workspace_bytes",
                 "vdn_last_error", "vdn_version", "vdn_timing_start", "vdn_timing_stop"):
        assert name in fns, fns


def test_library_exports_every_declared_function(vdn):
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if " T " in line}
    lib = ctypes.CDLL(LIB)
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(vdn.EXPORTS) == set(header_functions())


def test_library_is_gfx950_only():
    data = open(LIB, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-+(gfx[0-9a-z]+)", data))
    assert targets == {b"gfx950"}, targets


def test_version_and_clean_error_state(vdn):
    assert "gfx950" in vdn.vdn_version()


def test_shape_struct_layout(vdn):
    """14 four-byte fields in the order of include/vdn.h; softmax_mxfp8 last."""
    assert ctypes.sizeof(vdn.vdn_shape) == 14 * 4
    assert vdn.vdn_shape.context_tokens.offset == 12 * 4
    assert vdn.vdn_shape.softmax_mxfp8.offset == 13 * 4
    assert vdn.vdn_shape.dtype.offset == 11 * 4


def _shape(vdn, **kw):
    base = dict(batch=1, heads=2, frames=12, tokens_per_frame=6, head_dim=32, dtype="bf16")
    base.update(kw)
    return vdn.make_shape(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=48), -2), (dict(head_dim=256), -2), (dict(frames=0), -2),
    (dict(tokens_per_frame=0), -2), (dict(batch=0), -2), (dict(heads=-1), -2),
    (dict(chunk_frames=0), -2), (dict(window_chunks=-1), -2), (dict(dtype=7), -3),
    (dict(rms_eps=-1.0), -2), (dict(anchor_first=2), -2), (dict(context_tokens=-1), -2),
    (dict(frames=2 ** 16, tokens_per_frame=2 ** 14, context_tokens=1), -2),
    (dict(softmax_mxfp8=True), -2), (dict(head_dim=128, dtype="f32", softmax_mxfp8=True), -3),
])
def test_bad_shapes_rejected_before_launch(vdn, kw, status):
    s = _shape(vdn, **kw)
    fake = 1 << 20     # never dereferenced: validation fails first
    for call in (
        lambda: vdn._lib.vdn_hybrid_attn_fwd(ctypes.byref(s), *([fake] * 12), fake, 1 << 40, None),
        lambda: vdn._lib.vda_scan_fwd(ctypes.byref(s), *([fake] * 9), fake, 1 << 40, None),
        lambda: vdn._lib.window_anchor_attn_fwd(ctypes.byref(s), *([fake] * 6), fake, 1 << 40, None),
    ):
        assert call() == status
        assert vdn.vdn_last_error() != ""
    assert vdn._lib.vdn_workspace_bytes(ctypes.byref(s), 0) == 0


def test_null_and_misaligned_pointers_rejected(vdn):
    s = _shape(vdn)
    fake = 1 << 20
    args = [fake] * 12
    for i in (0, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11):     # rms_w (index 8) is nullable
        a = list(args)
        a[i] = None
        assert vdn._lib.vdn_hybrid_attn_fwd(ctypes.byref(s), *a, fake, 1 << 40, None) == -1
    a = list(args)
    a[1] = fake + 2
    assert vdn._lib.vdn_hybrid_attn_fwd(ctypes.byref(s), *a, fake, 1 << 40, None) == -1
    assert "aligned" in vdn.vdn_last_error()
    assert vdn._lib.vda_scan_fwd(None, *([fake] * 9), fake, 1 << 40, None) == -1
    with pytest.raises(vdn.VdnError) as ei:
        vdn.window_anchor_attn_fwd(s, None, fake, fake, None, fake, None, None)
    assert ei.value.status == -1


def test_workspace_too_small_rejected(vdn):
    s = _shape(vdn)
    fake = 1 << 20
    vda_args = [fake] * 8 + [None]          # states NULL: kept in the workspace
    for op, call in (
        (0, lambda n, w: vdn._lib.vdn_hybrid_attn_fwd(ctypes.byref(s), *([fake] * 12), w, n, None)),
        (1, lambda n, w: vdn._lib.vda_scan_fwd(ctypes.byref(s), *vda_args, w, n, None)),
    ):
        need = vdn.vdn_workspace_bytes(s, op)
        assert need >= 256
        assert call(need - 1, fake) == -4
        assert "workspace" in vdn.vdn_last_error()
        assert call(need, None) == -4


def test_workspace_sizes_cover_the_layout(vdn):
    """Hybrid workspace at the 102-frame headline shape holds the gates and
    branch outputs (2 x [B*L, 2D] bf16), the VDA matrices and the anchor
    partials; all sizes are 256-byte multiples."""
    s = vdn.make_shape(1, 24, 102, 4032, 128, "bf16")
    L, D = 102 * 4032, 24 * 128
    hyb = vdn.vdn_workspace_bytes(s, 0)
    vda = vdn.vdn_workspace_bytes(s, 1)
    att = vdn.vdn_workspace_bytes(s, 2)
    assert hyb >= 2 * L * 2 * D * 2 + vda + att
    assert vda >= 4 * 24 * 102 * 128 * 128 * 4
    assert att >= 2 * 24 * 2 * 4032 * 128 * 4       # two anchor frames, >= 2 key splits
    assert hyb % 256 == 0 and vda % 256 == 0 and att % 256 == 0
    with pytest.raises(vdn.VdnError):
        vdn.vdn_workspace_bytes(s, 9)


def test_dense_entry_point_rejects_bad_arguments(vdn):
    s = _shape(vdn)
    fake = 1 << 20
    need = vdn.vdn_workspace_bytes(s, vdn.VDN_OP_DENSE_ATTN)
    call = lambda args, w, n: vdn._lib.vdn_dense_attn_fwd(ctypes.byref(s), *args, w, n, None)  # noqa: E731
    for i in range(5):
        a = [fake] * 5
        a[i] = None
        assert call(a, fake, need) == -1
    a = [fake] * 5
    a[3] = fake + 8
    assert call(a, fake, need) == -1
    assert call([fake] * 5, fake, need - 1) == -4
    assert call([fake] * 5, None, need) == -4


def test_dense_workspace_holds_projection_and_output(vdn):
    """The dense baseline's workspace holds W_o^T [D, D] and the softmax
    output [B*L, D]; its window and anchor fields do not change the size."""
    s = vdn.make_shape(2, 24, 42, 4032, 128, "bf16")
    L, D = 42 * 4032, 24 * 128
    n = vdn.vdn_workspace_bytes(s, vdn.VDN_OP_DENSE_ATTN)
    assert n >= D * D * 2 + 2 * L * D * 2 and n % 256 == 0
    s2 = vdn.make_shape(2, 24, 42, 4032, 128, "bf16", window_chunks=3, anchor_first=False)
    assert vdn.vdn_workspace_bytes(s2, vdn.VDN_OP_DENSE_ATTN) == n


def test_huge_window_is_the_whole_sequence(vdn):
    """A window wider than the sequence sizes exactly like one of nC chunks
    (no integer overflow in the frame-range arithmetic)."""
    nC = (102 + 4) // 5
    a = vdn.make_shape(1, 24, 102, 4032, 128, "bf16", window_chunks=nC)
    b = vdn.make_shape(1, 24, 102, 4032, 128, "bf16", window_chunks=2 ** 31 - 1)
    for op in (vdn.VDN_OP_HYBRID, vdn.VDN_OP_WINDOW_ATTN):
        assert vdn.vdn_workspace_bytes(a, op) == vdn.vdn_workspace_bytes(b, op)


def test_param_check_switch(vdn):
    """The range check is off by default; the switch returns the previous
    setting.  (Its device-side verdict is tested on the GPU.)"""
    assert vdn.vdn_set_param_check(True) is False
    assert vdn.vdn_set_param_check(False) is True
    assert vdn.vdn_set_param_check(False) is False


def test_timing_session_without_launches(vdn):
    """Starting and stopping a timing session with no recorded launch touches
    no GPU and reports every phase with zero launches."""
    vdn.vdn_timing_start()
    stats = vdn.vdn_timing_stop()
    assert "window_attn" in stats and "vda_scan" in stats
    assert all(n == 0 for n, _ in stats.values())


def test_context_tokens_grow_the_workspace(vdn):
    """Context rows add gate and branch-output rows to the layer workspace and
    a dense query group (its key-split partials) to the softmax workspace."""
    a = vdn.make_shape(1, 4, 42, 64, 64, "bf16")
    b = vdn.make_shape(1, 4, 42, 64, 64, "bf16", context_tokens=100)
    D = 4 * 64
    for op in (vdn.VDN_OP_HYBRID, vdn.VDN_OP_WINDOW_ATTN, vdn.VDN_OP_DENSE_ATTN):
        assert vdn.vdn_workspace_bytes(b, op) > vdn.vdn_workspace_bytes(a, op)
    grow = vdn.vdn_workspace_bytes(b, vdn.VDN_OP_HYBRID) - vdn.vdn_workspace_bytes(a, vdn.VDN_OP_HYBRID)
    assert grow >= 2 * 100 * 2 * D * 2      # gates and branch outputs, [rows, 2D] bf16 each
    # the linear branch reads video rows only: its workspace does not change
    assert vdn.vdn_workspace_bytes(b, vdn.VDN_OP_VDA_SCAN) == vdn.vdn_workspace_bytes(a, vdn.VDN_OP_VDA_SCAN)


def test_mxfp8_quantize_rejects_bad_arguments(vdn):
    fake = 1 << 20
    assert vdn._lib.vdn_mxfp8_quantize(None, 32, fake, fake, None) == -1
    assert vdn._lib.vdn_mxfp8_quantize(fake, 32, None, fake, None) == -1
    assert vdn._lib.vdn_mxfp8_quantize(fake + 4, 32, fake, fake, None) == -1
    assert "aligned" in vdn.vdn_last_error()
    assert vdn._lib.vdn_mxfp8_quantize(fake, 33, fake, fake, None) == -2
    assert vdn._lib.vdn_mxfp8_quantize(fake, -32, fake, fake, None) == -2


def test_mxfp8_window_entry_rejects_bad_arguments(vdn):
    fake = 1 << 20
    ok = _shape(vdn, head_dim=128)
    call = lambda s, *a: vdn._lib.window_anchor_attn_mxfp8_fwd(ctypes.byref(s), *a)
    args = [fake] * 8 + [fake, 1 << 40, None]
    assert call(_shape(vdn, head_dim=64), *args) == -2           # head_dim 128 only
    assert call(_shape(vdn, head_dim=128, dtype="f32"), *args) == -3
    for i in (0, 1, 2, 3, 4, 6):                                  # codes, scales, v, out
        a = list(args)
        a[i] = None
        assert call(ok, *a) == -1
    a = list(args)
    a[1] = fake + 8                                               # misaligned scales
    assert call(ok, *a) == -1
    a = list(args)
    a[8] = None   # no workspace: the anchor rows of 102 frames are split over keys, their partials need one
    assert call(vdn.make_shape(1, 2, 102, 4032, 128, "bf16"), *a) == -4


def test_mxfp8_mode_grows_the_workspace(vdn):
    """With softmax_mxfp8 the softmax-branch workspace also holds the codes and
    scales of q and k: 2 * B*H*Lt*(d + d/32) bytes (plus alignment)."""
    B, H, T, N, d = 1, 24, 102, 4032, 128
    plain = vdn.make_shape(B, H, T, N, d, "bf16")
    mx = vdn.make_shape(B, H, T, N, d, "bf16", softmax_mxfp8=True)
    extra = 2 * B * H * T * N * (d + d // 32)
    for op in (0, 2, 3):
        grow = vdn.vdn_workspace_bytes(mx, op) - vdn.vdn_workspace_bytes(plain, op)
        assert extra <= grow <= extra + 4 * 256, (op, grow)
    assert vdn.vdn_workspace_bytes(mx, 1) == vdn.vdn_workspace_bytes(plain, 1)


def test_vda_bwd_entry_rejects_bad_arguments(vdn):
    fake = 1 << 20
    ok = _shape(vdn)
    need = vdn.vdn_workspace_bytes(ok, vdn.VDN_OP_VDA_BWD)
    call = lambda s, *a: vdn._lib.vda_scan_bwd(ctypes.byref(s), *a)
    # q k v gamma beta rms_w d_out dq dk dv dgamma dbeta drms_w | ws ws_bytes stream
    args = [fake] * 13 + [fake, need, None]
    for i in (0, 1, 2, 3, 4, 6, 7, 8, 9, 10, 11):                # rms_w and drms_w may be NULL
        a = list(args)
        a[i] = None
        assert call(ok, *a) == -1, i
    for i in (0, 5, 6, 12):
        a = list(args)
        a[i] = fake + 4                                           # misaligned
        assert call(ok, *a) == -1, i
    a = list(args)
    a[14] = need - 1
    assert call(ok, *a) == -4
    a[13], a[14] = None, need
    assert call(ok, *a) == -4
    assert call(_shape(vdn, head_dim=48), *args) == -2
    assert call(_shape(vdn, dtype=7), *args) == -3
    assert call(vdn.make_shape(300, 300, 2, 4, 32, "bf16"), *args) == -2   # batch * heads > 65535


def test_vda_bwd_workspace_holds_the_adjoint_buffers(vdn):
    """The gradient's workspace holds 17 per-frame d x d fp32 matrices (recomputed
    forward, both directions of the adjoint chain) and u / du of every token and
    direction in fp32."""
    B, H, T, N, d = 1, 24, 102, 4032, 128
    s = vdn.make_shape(B, H, T, N, d, "bf16")
    n = vdn.vdn_workspace_bytes(s, vdn.VDN_OP_VDA_BWD)
    nf = B * H * T
    low = 17 * nf * d * d * 4 + nf * 2 * N * d * 4
    assert low <= n <= low + 32 * 256 + nf * (4 + 2 * d * 4) + 256
    assert n % 256 == 0


def test_noalloc_entry_rejects_bad_arguments_before_any_launch(vdn):
    """vda_scan_fwd_noalloc checks its arguments and its scratch bound on the
    host: NULL or misaligned pointers, and a shape whose scratch would exceed
    the library's static 64 MiB (the 102-frame layer's linear branch needs
    about 1 GB), are rejected without touching a device."""
    lib = ctypes.CDLL(LIB)
    lib.vda_scan_fwd_noalloc.argtypes = [ctypes.POINTER(vdn.vdn_shape)] + [ctypes.c_void_p] * 10
    lib.vda_scan_fwd_noalloc.restype = ctypes.c_int
    p = ctypes.c_void_p(1 << 20)
    big = vdn.make_shape(1, 24, 102, 4032, 128, "bf16")
    assert vdn.vdn_workspace_bytes(big, vdn.VDN_OP_VDA_SCAN) > (64 << 20)
    rc = lib.vda_scan_fwd_noalloc(ctypes.byref(big), p, p, p, p, p, None, None, p, None, None)
    assert rc == -4 and "scratch" in vdn.vdn_last_error()
    small = vdn.make_shape(1, 8, 42, 1560, 64, "bf16")
    assert vdn.vdn_workspace_bytes(small, vdn.VDN_OP_VDA_SCAN) <= (64 << 20)
    rc = lib.vda_scan_fwd_noalloc(ctypes.byref(small), None, p, p, p, p, None, None, p, None, None)
    assert rc == -1
    rc = lib.vda_scan_fwd_noalloc(ctypes.byref(small), ctypes.c_void_p((1 << 20) + 4), p, p, p, p, None, None,
                                  p, None, None)
    assert rc == -1
