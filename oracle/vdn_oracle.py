"""Plain fp64 CPU oracle for the Video DeltaNet (VDN) hybrid attention forward.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  It shares no code with the
HIP path (no kernels, headers, helpers or constants) and imports nothing from
the product package; both sides are fed from the seeded generator module.

Sources.  The method is described on web pages about the paper "Video DeltaNet:
A Video-Native Hybrid Attention for Livestream Video Generation" (arXiv
2609.20744).  Citations use these tags:
  [P3]  10100.com article "直播视频生成太慢？UC Berkeley开源Video DeltaNet ..."
        - section 方法概述, part 1 (hybrid allocation: sliding-window softmax
          over VAE chunks plus boundary anchors), part 2 (frame-level delta
          rule, VDA), part 3 (branch calibration: gates, RMSNorm, separate
          output projections); section 实验结果, the figure caption (forward
          plus backward scan).
  [P2]  hotpaper.ai page "Video DeltaNet: A Video-Native Hybrid Attention for
        Livestream Video Generation" - abstract and 기술적 접근법 (technical
        approach: RMS normalisation and learnable gates).
  [P1]  ai-feeds.com page "Video DeltaNet:面向直播视频生成的视频原生混合注意力"
        - section 方法 / 关键模块 (key modules).

What the pages fix and what is read into them (each reading is listed, with
the alternatives, in the repository's design notes):
  * Per frame t and head, the state is the minimiser of
        ||S - Sbar_t||_F^2 + beta_t * sum_i ||S k_i - v_i||^2
    over all N tokens of the frame; setting the derivative to zero gives
        S_t = (Sbar_t + B_t)(I + A_t)^-1,
    A_t = beta_t K_t^T K_t (key correlations), B_t = beta_t V_t^T K_t
    (value-key writes).  [P3 方法概述 part 2]
  * Reading D-1: the decayed old state is Sbar_t = gamma_t * S_prev with one
    scalar gamma per frame and head.  Reading D-2: scans start from S = 0.
  * The linear memory is bidirectional: a forward scan over frames and a
    backward scan.  [P3 实验结果 figure caption; P2 abstract]  Reading D-5/D-6:
    both directions read the state after frame t's own write; the backward
    scan uses the same gamma_t, beta_t as the forward one, visited in
    reverse.
  * Readout u = S_t q; each direction goes through RMSNorm (over head_dim,
    eps, weight w) and the two are summed; an independent sigmoid output gate
    multiplies the result.  [P3 方法概述 part 3; P2 기술적 접근법]  Readings
    D-7/D-8/D-9.
  * Softmax branch: 5-frame chunks; a query chunk sees its own chunk and one
    chunk on each side; every frame also sees all tokens of the first and
    last latent frame, and those two frames see the whole sequence.  One
    softmax over the union of allowed keys.  A content-dependent sigmoid gate
    multiplies the output.  [P3 方法概述 parts 1 and 3]  Readings D-10..D-12.
  * Each branch has its own output projection; the two projections are
    summed.  [P3 方法概述 part 3; P1 关键模块]
  * Context (text / audio) tokens: every interaction that involves one keeps
    the full softmax, and the linear branch covers only video-to-video context.
    [P3 方法概述 part 1, last sentence; P3 内容介绍 item 1; P1 方法 / 输入与整体流程]
    Reading C-1: the sequence is the T*N video tokens followed by n_ctx
    context tokens; a video query's one softmax runs over its allowed video
    keys plus every context key; a context query attends every token; the
    linear branch output of a context row is zero; gates and projections
    treat context rows like video rows.

Everything is computed in float64 from the (already rounded) inputs.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "frame_stats", "transition", "frame_update", "vda_states",
    "rms_norm", "vda_readout", "vda_branch",
    "allowed_frames", "key_frames", "window_attention",
    "sigmoid", "gates", "merge_heads", "hybrid_layer", "hybrid_layer_rows",
    "dense_layer", "window_attention_ctx", "hybrid_layer_ctx",
]


# --------------------------------------------------------------------------
# Linear branch: Video Delta Attention  [P3 方法概述 part 2]
# --------------------------------------------------------------------------


def mxfp8_values(x):
    """Values (float64) of the MXFP8 encoding of x along its last axis
    (oracle.mxfp8: OCP MXFP8, blocks of 32 along head_dim)."""
    from oracle import mxfp8
    return mxfp8.dequantize(*mxfp8.quantize(x))


def frame_stats(k_t: np.ndarray, v_t: np.ndarray, beta_t: float):
    """Frame statistics of one frame and head.

    k_t, v_t: [N, d] key and value rows of the frame's N tokens.
    Returns A_t = beta_t K_t^T K_t ([d_k, d_k], key correlations) and
    B_t = beta_t V_t^T K_t ([d_v, d_k], value-key writes).  [P3 方法概述 part 2]
    """
    k_t = np.asarray(k_t, dtype=np.float64)
    v_t = np.asarray(v_t, dtype=np.float64)
    a_t = beta_t * (k_t.T @ k_t)
    b_t = beta_t * (v_t.T @ k_t)
    return a_t, b_t


def transition(a_t: np.ndarray) -> np.ndarray:
    """M_t = (I + A_t)^-1, the inherited-state transition.  [P3 方法概述 part 2]

    I + A_t is symmetric positive definite for beta_t >= 0; a plain LAPACK
    solve against the identity is used (no structure exploited).
    """
    d = a_t.shape[0]
    eye = np.eye(d)
    return np.linalg.solve(eye + a_t, eye)


def frame_update(s_prev: np.ndarray, gamma_t: float, a_t: np.ndarray, b_t: np.ndarray):
    """One frame-level delta-rule step: S_t = (gamma_t S_prev + B_t)(I + A_t)^-1.

    The decayed old state is gamma_t * S_prev (reading D-1).  [P3 方法概述 part 2]
    """
    return (gamma_t * s_prev + b_t) @ transition(a_t)


def vda_states(k: np.ndarray, v: np.ndarray, gamma: np.ndarray, beta: np.ndarray):
    """Forward and backward frame scans of one (batch, head).

    k, v: [T, N, d]; gamma, beta: [T].
    Returns (s_fwd, s_bwd), each [T, d_v, d_k]: s_fwd[t] is the state after
    frames 0..t were written in that order, s_bwd[t] the state after frames
    T-1..t were written in that order.  Both start from zero (reading D-2).
    [P3 方法概述 part 2; 实验结果 figure caption (forward plus backward scan)]
    """
    T, _, d = k.shape
    stats = [frame_stats(k[t], v[t], float(beta[t])) for t in range(T)]

    s_fwd = np.zeros((T, d, d))
    s = np.zeros((d, d))
    for t in range(T):
        a_t, b_t = stats[t]
        s = frame_update(s, float(gamma[t]), a_t, b_t)
        s_fwd[t] = s

    s_bwd = np.zeros((T, d, d))
    s = np.zeros((d, d))
    for t in range(T - 1, -1, -1):
        a_t, b_t = stats[t]
        s = frame_update(s, float(gamma[t]), a_t, b_t)
        s_bwd[t] = s
    return s_fwd, s_bwd


def rms_norm(u: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: u / sqrt(mean(u^2) + eps) * w.
    [P3 方法概述 part 3; P2 기술적 접근법]  (Reading D-8: per token and head.)"""
    u = np.asarray(u, dtype=np.float64)
    return u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps) * w


def vda_readout(q_t: np.ndarray, s_fwd_t: np.ndarray, s_bwd_t: np.ndarray,
                w: np.ndarray, eps: float) -> np.ndarray:
    """Linear-branch output of the tokens of one frame (before the gate).

    q_t: [n, d]; each token reads u = S q from both directions; the result is
    RMSNorm(u_fwd) + RMSNorm(u_bwd) (reading D-7).  [P3 方法概述 part 3]
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    u_f = q_t @ s_fwd_t.T
    u_b = q_t @ s_bwd_t.T
    return rms_norm(u_f, w, eps) + rms_norm(u_b, w, eps)


def vda_branch(q, k, v, gamma, beta, rms_w, eps):
    """Ungated linear-branch output for every head.

    q, k, v: [B, H, T, N, d]; gamma, beta: [B, H, T]; rms_w: [H*d].
    Returns (o_l [B, H, T, N, d], s_fwd [B, H, T, d, d], s_bwd [B, H, T, d, d]).
    """
    B, H, T, N, d = q.shape
    o = np.zeros((B, H, T, N, d))
    sf = np.zeros((B, H, T, d, d))
    sb = np.zeros((B, H, T, d, d))
    for b in range(B):
        for h in range(H):
            sf[b, h], sb[b, h] = vda_states(k[b, h], v[b, h], gamma[b, h], beta[b, h])
            w_h = rms_w[h * d:(h + 1) * d]
            for t in range(T):
                o[b, h, t] = vda_readout(q[b, h, t], sf[b, h, t], sb[b, h, t], w_h, eps)
    return o, sf, sb


# --------------------------------------------------------------------------
# Softmax branch: chunked sliding window plus boundary anchors
# [P3 方法概述 part 1]
# --------------------------------------------------------------------------

def allowed_frames(T: int, chunk_frames: int = 5, window_chunks: int = 1,
                   anchor_first: bool = True, anchor_last: bool = True) -> np.ndarray:
    """Frame-level mask [T_query, T_key] of the softmax branch.

    Chunk of frame t is t // chunk_frames, counted from frame 0 (reading
    D-11).  A query frame sees key frames whose chunk is within
    window_chunks of its own; every query frame sees the first and last
    frame; the first and last frame see every frame.  [P3 方法概述 part 1]
    """
    ok = np.zeros((T, T), dtype=bool)
    for t in range(T):
        for s in range(T):
            near = abs(t // chunk_frames - s // chunk_frames) <= window_chunks
            anchor_key = (anchor_first and s == 0) or (anchor_last and s == T - 1)
            anchor_query = (anchor_first and t == 0) or (anchor_last and t == T - 1)
            ok[t, s] = near or anchor_key or anchor_query
    return ok


def key_frames(allowed: np.ndarray, t: int) -> np.ndarray:
    """Key frames visible from query frame t, each once, in frame order."""
    return np.nonzero(allowed[t])[0]


def window_attention(q, k, v, allowed, scale, rows=None):
    """Softmax branch of one (batch, head), ungated.

    q, k, v: [T, N, d].  For every query token one softmax runs over all key
    tokens of the allowed frames (each key once, reading D-12), logits
    (q . k) * scale (reading D-10: scale = 1/sqrt(d)).
    rows: optional 1-D array of flat query-token indices (t*N + n); default
    all tokens.  Returns (o [len(rows), d], lse [len(rows)]) with lse the
    natural log of the softmax denominator of the scaled logits.
    """
    T, N, d = q.shape
    if rows is None:
        rows = np.arange(T * N)
    rows = np.asarray(rows)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    frames_of_rows = rows // N
    for t in np.unique(frames_of_rows):
        sel = np.nonzero(frames_of_rows == t)[0]
        kf = key_frames(allowed, int(t))
        keys = np.concatenate([np.asarray(k[s], dtype=np.float64) for s in kf], axis=0)
        vals = np.concatenate([np.asarray(v[s], dtype=np.float64) for s in kf], axis=0)
        qs = np.asarray(q[t], dtype=np.float64)[rows[sel] % N]
        logits = (qs @ keys.T) * scale
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        den = p.sum(axis=1, keepdims=True)
        o[sel] = (p @ vals) / den
        lse[sel] = (m + np.log(den))[:, 0]
    return o, lse


# --------------------------------------------------------------------------
# Gates and output projections  [P3 方法概述 part 3; P1 关键模块]
# --------------------------------------------------------------------------

def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def gates(x, w_gs, w_gl):
    """Content-dependent sigmoid gates (reading D-9: elementwise, no bias):
    g_s = sigmoid(x W_gs) for the softmax branch, g_l = sigmoid(x W_gl) for
    the linear branch.  x: [..., D]; W: [D, D] (y = x W)."""
    x = np.asarray(x, dtype=np.float64)
    return sigmoid(x @ w_gs), sigmoid(x @ w_gl)


def merge_heads(o):
    """[B, H, T, N, d] -> token-major [B, T*N, H*d] (column h*d + j)."""
    B, H, T, N, d = o.shape
    return np.transpose(o, (0, 2, 3, 1, 4)).reshape(B, T * N, H * d)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def hybrid_layer(x, q, k, v, gamma, beta, w_gs, w_gl, rms_w, w_os, w_ol,
                 chunk_frames=5, window_chunks=1, anchor_first=True,
                 anchor_last=True, scale=None, eps=1e-6, return_parts=False):
    """Full VDN hybrid attention forward (video-to-video tokens only).

    out = (g_s * O_s) W_os + (g_l * O_l) W_ol, where O_s is the softmax
    branch and O_l the bidirectional VDA branch, both token-major [B, L, D].
    [P3 方法概述 parts 1-3; P1 关键模块]
    """
    x, q, k, v = _f64(x), _f64(q), _f64(k), _f64(v)
    gamma, beta, rms_w = _f64(gamma), _f64(beta), _f64(rms_w)
    w_gs, w_gl, w_os, w_ol = _f64(w_gs), _f64(w_gl), _f64(w_os), _f64(w_ol)
    B, H, T, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    allowed = allowed_frames(T, chunk_frames, window_chunks, anchor_first, anchor_last)

    o_s = np.zeros((B, H, T, N, d))
    lse = np.zeros((B, H, T * N))
    for b in range(B):
        for h in range(H):
            o, l = window_attention(q[b, h], k[b, h], v[b, h], allowed, scale)
            o_s[b, h] = o.reshape(T, N, d)
            lse[b, h] = l
    o_l, sf, sb = vda_branch(q, k, v, gamma, beta, rms_w, eps)

    g_s, g_l = gates(x, w_gs, w_gl)
    y_s = g_s * merge_heads(o_s)
    y_l = g_l * merge_heads(o_l)
    out = y_s @ w_os + y_l @ w_ol
    if return_parts:
        return out, dict(o_s=o_s, o_l=o_l, lse=lse, s_fwd=sf, s_bwd=sb,
                         g_s=g_s, g_l=g_l, y_s=y_s, y_l=y_l)
    return out


def hybrid_layer_rows(x, q, k, v, gamma, beta, w_gs, w_gl, rms_w, w_os, w_ol,
                      rows, chunk_frames=5, window_chunks=1, anchor_first=True,
                      anchor_last=True, scale=None, eps=1e-6, states=None,
                      softmax_mxfp8=False):
    """hybrid_layer restricted to the output tokens `rows` (flat t*N + n) of
    every batch entry, for workloads too large to evaluate whole.

    The linear branch still needs every frame's state (full scans); the
    softmax branch, gates and projections are evaluated only at `rows`.
    `states` may carry precomputed (s_fwd, s_bwd) of shape [B, H, T, d, d].
    softmax_mxfp8: reading F-1 of [P3] 实验结果 (the denoiser runs in MXFP8):
    the softmax branch's score product takes the MXFP8 values of its two
    operands, q and k as the layer receives them (blocks of 32 along
    head_dim), and the softmax applies its scale to that product as usual,
    logits = scale * (q8 . k8); probabilities, v, the linear branch (which
    reads the unquantised q and k), gates and projections are unchanged.
    Returns out [B, len(rows), D].
    """
    # q, k, v are converted to float64 one (batch, head) slice at a time so that
    # full-size inputs need not be held in float64 whole.
    gamma, beta, rms_w = _f64(gamma), _f64(beta), _f64(rms_w)
    B, H, T, N, d = q.shape
    rows = np.asarray(rows)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    allowed = allowed_frames(T, chunk_frames, window_chunks, anchor_first, anchor_last)
    R = len(rows)
    y_s = np.zeros((B, R, H * d))
    y_l = np.zeros((B, R, H * d))
    xr = _f64(np.asarray(x)[:, rows, :])
    g_s, g_l = gates(xr, _f64(w_gs), _f64(w_gl))
    for b in range(B):
        for h in range(H):
            qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
            if softmax_mxfp8:
                o, _ = window_attention(mxfp8_values(qh), mxfp8_values(kh), vh, allowed, scale, rows)
            else:
                o, _ = window_attention(qh, kh, vh, allowed, scale, rows)
            y_s[b, :, h * d:(h + 1) * d] = o
            if states is None:
                sf, sb = vda_states(kh, vh, gamma[b, h], beta[b, h])
            else:
                sf, sb = states[0][b, h], states[1][b, h]
            w_h = rms_w[h * d:(h + 1) * d]
            for i, r in enumerate(rows):
                t, n = divmod(int(r), N)
                y_l[b, i, h * d:(h + 1) * d] = vda_readout(qh[t, n][None], sf[t], sb[t], w_h, eps)[0]
            del qh, kh, vh
    return (g_s * y_s) @ _f64(w_os) + (g_l * y_l) @ _f64(w_ol)


def dense_layer(q, k, v, w_o, scale=None):
    """Dense full-softmax baseline on the same Q/K/V: every query sees every
    key, then one output projection, no gates.  Used only to compare cost."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    allowed = np.ones((T, T), dtype=bool)
    o = np.zeros((B, H, T, N, d))
    for b in range(B):
        for h in range(H):
            oo, _ = window_attention(q[b, h], k[b, h], v[b, h], allowed, scale)
            o[b, h] = oo.reshape(T, N, d)
    return merge_heads(o) @ _f64(w_o)


# --------------------------------------------------------------------------
# Context (text / audio) tokens  [P3 方法概述 part 1; P1 方法 / 输入与整体流程] - reading C-1
# --------------------------------------------------------------------------

def window_attention_ctx(q, k, v, allowed, N, scale, rows=None):
    """Softmax branch of one (batch, head) with context tokens, ungated.

    q, k, v: [T*N + n_ctx, d] - the video tokens (frame-major) followed by
    n_ctx context tokens; `allowed` is the [T, T] frame mask.  A video query
    of frame t sees the key tokens of its allowed frames plus every context
    token, under one softmax; a context query sees every token.  rows:
    optional flat query indices (default all).  Returns (o [len(rows), d],
    lse [len(rows)]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T = allowed.shape[0]
    L = T * N
    Ltot, d = q.shape
    if rows is None:
        rows = np.arange(Ltot)
    rows = np.asarray(rows)
    ctx_keys = np.arange(L, Ltot)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for i, r in enumerate(rows):
        if r < L:
            t = r // N
            frames = key_frames(allowed, int(t))
            keys = np.concatenate([np.arange(f * N, (f + 1) * N) for f in frames] + [ctx_keys])
        else:
            keys = np.arange(Ltot)
        logits = (k[keys] @ q[r]) * scale
        m = logits.max()
        p = np.exp(logits - m)
        o[i] = (p @ v[keys]) / p.sum()
        lse[i] = m + np.log(p.sum())
    return o, lse


def hybrid_layer_ctx(x, q, k, v, gamma, beta, w_gs, w_gl, rms_w, w_os, w_ol, N,
                     chunk_frames=5, window_chunks=1, anchor_first=True,
                     anchor_last=True, scale=None, eps=1e-6, rows=None):
    """Hybrid attention forward with n_ctx context tokens after the video.

    x: [B, T*N + n_ctx, D]; q, k, v: [B, H, T*N + n_ctx, d]; gamma, beta
    [B, H, T].  The softmax branch follows window_attention_ctx; the linear
    branch runs on the video tokens only and is zero on context rows; gates
    and projections as in hybrid_layer.  rows: optional flat output rows
    (default all); the linear branch's scans always cover every frame.
    Returns out [B, len(rows), D].  [P3 方法概述 parts 1-3; reading C-1]
    """
    gamma, beta, rms_w = _f64(gamma), _f64(beta), _f64(rms_w)
    B, H, Ltot, d = q.shape
    T = gamma.shape[2]
    L = T * N
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if rows is None:
        rows = np.arange(Ltot)
    rows = np.asarray(rows)
    allowed = allowed_frames(T, chunk_frames, window_chunks, anchor_first, anchor_last)
    R = len(rows)
    y_s = np.zeros((B, R, H * d))
    y_l = np.zeros((B, R, H * d))
    g_s, g_l = gates(_f64(np.asarray(x)[:, rows, :]), _f64(w_gs), _f64(w_gl))
    for b in range(B):
        for h in range(H):
            qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
            o, _ = window_attention_ctx(qh, kh, vh, allowed, N, scale, rows)
            y_s[b, :, h * d:(h + 1) * d] = o
            kv = kh[:L].reshape(T, N, d), vh[:L].reshape(T, N, d)
            sf, sb = vda_states(kv[0], kv[1], gamma[b, h], beta[b, h])
            w_h = rms_w[h * d:(h + 1) * d]
            for i, r in enumerate(rows):
                if r < L:
                    t = int(r) // N
                    y_l[b, i, h * d:(h + 1) * d] = vda_readout(qh[r][None], sf[t], sb[t], w_h, eps)[0]
    return (g_s * y_s) @ _f64(w_os) + (g_l * y_l) @ _f64(w_ol)
