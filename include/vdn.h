/*
 * vdn.h - C ABI of libvdn.so: the Video DeltaNet (VDN) hybrid attention
 * forward on one AMD Instinct MI355X (gfx950).
 *
 * The operation is the video-to-video attention of Video DeltaNet as described
 * in the 10100.com article on the paper (section 方法概述, parts 1-3) and the
 * hotpaper.ai abstract page "Video DeltaNet: A Video-Native Hybrid Attention
 * for Livestream Video Generation":
 *   softmax branch  O_s: one softmax per query token over the keys of its own
 *                   5-frame VAE chunk and one chunk on each side, plus every
 *                   token of the first and last latent frame; those two frames
 *                   attend the whole sequence (part 1);
 *   linear branch   O_l: Video Delta Attention, a frame-level delta rule
 *                   S_t = (gamma_t S_{t-1} + B_t)(I + A_t)^-1 with
 *                   A_t = beta_t K_t^T K_t and B_t = beta_t V_t^T K_t, run as a
 *                   forward and a backward scan over frames; each direction's
 *                   readout S_t q goes through RMSNorm and the two are summed
 *                   (part 2, and the forward-plus-backward scan figure);
 *   calibration     out = (g_s * O_s) W_os + (g_l * O_l) W_ol with content-
 *                   dependent sigmoid gates g_s = sigmoid(x W_gs),
 *                   g_l = sigmoid(x W_gl) (part 3).
 *
 * Notation: B batch, H heads, d head_dim, T latent frames, N tokens per frame,
 * L = T*N video tokens, Nc = shape->context_tokens text/audio tokens after
 * them, Lt = L + Nc, D = H*d model width.  Video token l = t*N + n; context
 * token c is row L + c.
 *
 * Context tokens (10100.com article, 方法概述 part 1, last sentence; ai-feeds
 * page, 方法 / 输入与整体流程): every interaction that involves a text or audio
 * token keeps the full softmax and the linear branch covers only video
 * context.  So a video query's softmax also covers every context key, a
 * context query attends every token, and the linear branch is zero on
 * context rows.  With Nc = 0 the layouts below are exactly those of a
 * video-only layer.
 *
 * Layouts (all row-major, contiguous, element type = shape->dtype unless
 * stated otherwise):
 *   q, k, v           [B, H, Lt, d]     = [B, H, T, N, d] followed, per (b, h),
 *                                       by Nc context rows; rows of k must be
 *                                       L2-normalised by the caller (the
 *                                       operator does not do it)
 *   gamma, beta       [B, H, T]         float32, per-frame decay / write strength
 *   x                 [B, Lt, D]        layer input the gates read
 *   w_gs, w_gl,
 *   w_os, w_ol        [D, D]            y = x @ W (input dimension first)
 *   rms_w             [D]               float32 RMSNorm weight (head h uses
 *                                       rms_w[h*d .. h*d+d-1]); NULL = ones
 *   gate_s, gate_l    [B, Lt, D]        gate values already in (0,1); NULL = 1
 *   out               [B, Lt, D]
 *   states            [2, B, H, T, d, d] float32; [0] forward-scan state after
 *                                       frame t, [1] backward-scan state after
 *                                       frame t; S is d_v x d_k (row = value dim)
 *   lse               [B, H, Lt]        float32 natural-log softmax denominator
 *                                       of the scaled logits
 *
 * Ownership: the caller allocates and owns every buffer, including the device
 * workspace `ws` whose size vdn_workspace_bytes() returns.  All data pointers
 * are device pointers (hipMalloc'd or equivalent) except `shape`, which is a
 * host pointer read before the call returns.  The library allocates no device
 * memory and keeps no pointer after it returns.
 *
 * Execution: every compute entry point validates its arguments on the host,
 * then enqueues its kernels on `stream` (a hipStream_t passed as void*; NULL =
 * the null stream) and returns without synchronising.  Outputs are valid once
 * the stream has been synchronised.  Calls on distinct streams with distinct
 * buffers may run concurrently.  Inputs and outputs must not overlap.
 *
 * Errors: functions return VDN_OK (0) or a negative status; on a negative
 * status nothing has been enqueued (except VDN_ERR_HIP, raised when a launch
 * fails), and vdn_last_error() returns a message for the calling thread.
 * Parameter ranges (beta >= 0 so that I + A_t is positive definite,
 * 0 <= gamma <= 1) are preconditions: they live in device memory and are not
 * read back, unless vdn_set_param_check(1) has been called (then the entry
 * points that read gamma and beta check them on the device first and
 * synchronise the stream to read the verdict).  NaN/Inf inputs propagate to
 * the outputs; they are not trapped.
 */
#ifndef VDN_H
#define VDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VDN_OK 0
#define VDN_ERR_INVALID_ARG (-1) /* NULL pointer, bad op code, misaligned pointer */
#define VDN_ERR_BAD_SHAPE (-2)   /* dimension < 1, head_dim not 32/64/128, ... */
#define VDN_ERR_DTYPE (-3)       /* dtype not VDN_F32 / VDN_BF16 */
#define VDN_ERR_WORKSPACE (-4)   /* ws NULL or ws_bytes < vdn_workspace_bytes() */
#define VDN_ERR_HIP (-5)         /* a HIP launch or runtime call failed */
#define VDN_ERR_PARAM_RANGE (-6) /* beta < 0 or gamma outside [0, 1]; reported only while
                                    vdn_set_param_check(1) is in effect */

enum vdn_dtype { VDN_F32 = 0, VDN_BF16 = 1 };

enum vdn_op {
  VDN_OP_HYBRID = 0,      /* vdn_hybrid_attn_fwd    */
  VDN_OP_VDA_SCAN = 1,    /* vda_scan_fwd           */
  VDN_OP_WINDOW_ATTN = 2, /* window_anchor_attn_fwd */
  VDN_OP_DENSE_ATTN = 3,  /* vdn_dense_attn_fwd     */
  VDN_OP_VDA_BWD = 4      /* vda_scan_bwd           */
};

typedef struct vdn_shape {
  int32_t batch;            /* B >= 1 */
  int32_t heads;            /* H >= 1 */
  int32_t frames;           /* T >= 1 latent frames */
  int32_t tokens_per_frame; /* N >= 1 */
  int32_t head_dim;         /* d in {32, 64, 128} */
  int32_t chunk_frames;     /* latent frames per VAE temporal chunk (5), >= 1 */
  int32_t window_chunks;    /* chunks seen on each side of the query chunk (1), >= 0 */
  int32_t anchor_first;     /* 1: frame 0 is a two-way global anchor */
  int32_t anchor_last;      /* 1: frame T-1 is a two-way global anchor */
  float softmax_scale;      /* logit scale; <= 0 selects 1/sqrt(d) */
  float rms_eps;            /* RMSNorm epsilon (1e-6) */
  int32_t dtype;            /* enum vdn_dtype: storage of q,k,v,x,W,gates,out */
  int32_t context_tokens;   /* Nc >= 0 text/audio tokens after the video tokens (0) */
  int32_t softmax_mxfp8;    /* 1: softmax-branch scores from MXFP8 q and k (below);
                               needs dtype VDN_BF16 and head_dim 128 (0) */
} vdn_shape;

/* Bytes of device workspace `op` needs for `shape` (0 on an invalid shape,
 * with vdn_last_error() set).  The workspace holds per-frame statistics,
 * transitions and states of the linear branch, anchor-row partial results,
 * per-head key-norm maxima and per-work-item flags of the softmax branch,
 * transposed weights, gates and branch outputs. */
size_t vdn_workspace_bytes(const vdn_shape* shape, int op); /* >= 256 when valid */

/* Full hybrid attention forward (10100.com article, 方法概述 parts 1-3):
 *   out = (sigmoid(x W_gs) * O_s) W_os + (sigmoid(x W_gl) * O_l) W_ol.
 * Inputs x, q, k, v, gamma, beta, w_gs, w_gl, rms_w (nullable), w_os, w_ol;
 * output out [B, L, D]. */
int vdn_hybrid_attn_fwd(const vdn_shape* shape, const void* x, const void* q,
                        const void* k, const void* v, const float* gamma,
                        const float* beta, const void* w_gs, const void* w_gl,
                        const float* rms_w, const void* w_os, const void* w_ol,
                        void* out, void* ws, size_t ws_bytes, void* stream);

/* Linear branch alone (10100.com article, 方法概述 part 2; forward-plus-
 * backward scan figure):
 *   out[b, t*N+n, h*d+i] = gate_l * (RMSNorm(S_fwd_t q) + RMSNorm(S_bwd_t q))_i
 * and zero on context rows.  gate_l may be NULL (no gate); states may be
 * NULL (kept in the workspace). */
int vda_scan_fwd(const vdn_shape* shape, const void* q, const void* k,
                 const void* v, const float* gamma, const float* beta,
                 const float* rms_w, const void* gate_l, void* out,
                 float* states, void* ws, size_t ws_bytes, void* stream);

/* vda_scan_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and arguments without the workspace.  Its scratch (the
 * per-frame statistics, transitions, states and their hi/lo copies, and the
 * range-check verdict: vdn_workspace_bytes(shape, VDN_OP_VDA_SCAN) bytes when
 * states is NULL, no more when states is given) is a static device array of the
 * library, 64 MiB (67108864 bytes) per device, held by each device that loads
 * the library until the process ends.  The call allocates nothing, device or
 * host.  A shape whose scratch would exceed 64 MiB returns VDN_ERR_WORKSPACE
 * with nothing enqueued (B1 H8 d64 T42 needs 33 MiB).  Every call on one
 * device shares that device's scratch: calls that overlap in time on one
 * device (on different streams or threads) race and give undefined results;
 * calls on one stream are ordered and safe.  Nothing in the scratch needs to
 * start at zero: each call writes every scratch byte it reads. */
int vda_scan_fwd_noalloc(const vdn_shape* shape, const void* q, const void* k,
                         const void* v, const float* gamma, const float* beta,
                         const float* rms_w, const void* gate_l, void* out,
                         float* states, void* stream);

/* Gradient of the linear branch (10100.com article, 方法概述 part 2, the
 * delta rule, and part 3, RMSNorm per direction; the article's staged
 * adaptation trains this branch).  For the ungated output
 *   o[b, t*N+n, h*d+i] = (RMSNorm(S_fwd_t q) + RMSNorm(S_bwd_t q))_i
 * of vda_scan_fwd (gate_l = NULL) and d_out = dLoss/do, the call writes
 *   dq, dk, dv   [B, H, Lt, d]  dtype; zero on context rows
 *   dgamma, dbeta [B, H, T]     float32
 *   drms_w       [D]            float32 (may be NULL: not computed)
 * d_out has the layout of out, [B, Lt, D] (its context rows are not read).
 * The gradient is the derivative of the forward rule taken step by step in
 * reverse (readout, both scans, the solve (I + A_t)^-1, the Gram products);
 * the forward quantities are recomputed from q, k, v, gamma, beta in the
 * workspace (op VDN_OP_VDA_BWD).  Precision: fp32 accumulation throughout;
 * with fp32 I/O every product is fp32, with bf16 I/O the token-side products
 * (S q, the readout adjoint, dq, dS, dK, dV) run on bf16 matrix cores with
 * each fp32 operand split into a bf16 high and low half (the low-by-low term
 * dropped, about 16 significant bits per operand), and the d x d products,
 * scans and solve adjoints stay fp32.  rms_w may be NULL (ones).
 * batch * heads must not exceed 65535. */
int vda_scan_bwd(const vdn_shape* shape, const void* q, const void* k,
                 const void* v, const float* gamma, const float* beta,
                 const float* rms_w, const void* d_out, void* dq, void* dk,
                 void* dv, float* dgamma, float* dbeta, float* drms_w,
                 void* ws, size_t ws_bytes, void* stream);

/* Softmax branch alone (10100.com article, 方法概述 part 1):
 *   out[b, l, h*d+i] = gate_s * (softmax over allowed keys of
 *                      scale * q_l . k) @ v
 * gate_s and lse may be NULL. */
int window_anchor_attn_fwd(const vdn_shape* shape, const void* q,
                           const void* k, const void* v, const void* gate_s,
                           void* out, float* lse, void* ws, size_t ws_bytes,
                           void* stream);

/* MXFP8 mode of the softmax branch.  The 10100.com article (实验结果, the
 * paragraph on scaling with sequence length) runs the denoiser in MXFP8
 * without saying which operations.  Read here: the two operands of the
 * softmax branch's score product, q and k as the layer receives them, are
 * MXFP8, and the softmax scales their product as usual,
 * logit = scale * (q8 . k8); the softmax, P V, v, the gates, the linear
 * branch (which reads the unquantised q and k) and the projections stay as in
 * the bf16 path.
 * Format: OCP Microscaling (MX) v1.0 MXFP8, i.e. blocks of 32 consecutive
 * elements (along head_dim) in OCP FP8 E4M3 (bias 7, largest finite 448)
 * sharing one E8M0 scale 2^(code - 127).  With shape->softmax_mxfp8 = 1,
 * vdn_hybrid_attn_fwd, window_anchor_attn_fwd and vdn_dense_attn_fwd quantise
 * their bf16 q and k into the workspace (vdn_workspace_bytes grows by
 * 2 * B*H*Lt*(d + d/32) bytes) and take the scores from them. */

/* MXFP8 quantisation of n_elems bf16 values x (n_elems a non-negative
 * multiple of 32), block i = x[32 i .. 32 i + 31]: scales[i] = clamp(
 * floor(log2 max|x|) - 8, -127, 127) + 127 (0 for an all-zero block) and
 * codes[32 i + j] = x / 2^(scales[i] - 127) rounded to the nearest E4M3
 * value, ties to the even code, magnitudes >= 448 saturating to 448, sign
 * bit = sign of x.  For a [rows, d] tensor (d a multiple of 32) this gives
 * codes [rows, d] and scales [rows, d / 32].  x and codes 16-byte aligned,
 * scales any alignment; all device pointers, caller-owned.  Non-finite
 * inputs give unspecified codes.  Errors: VDN_ERR_INVALID_ARG (NULL or
 * misaligned pointer), VDN_ERR_BAD_SHAPE (n_elems). */
int vdn_mxfp8_quantize(const void* x, int64_t n_elems, void* codes,
                       void* scales, void* stream);

/* Softmax branch (10100.com article, 方法概述 part 1) with scores from
 * MXFP8 q and k given as codes [B, H, Lt, 128] (uint8 E4M3) and scales
 * [B, H, Lt, 4] (uint8 E8M0), as vdn_mxfp8_quantize writes them; v, gate_s,
 * out and lse as window_anchor_attn_fwd.  shape->dtype must be VDN_BF16 and
 * head_dim 128 (VDN_ERR_DTYPE / VDN_ERR_BAD_SHAPE otherwise); the
 * softmax_mxfp8 field is ignored.  Workspace: vdn_workspace_bytes(shape,
 * VDN_OP_WINDOW_ATTN) of the shape with softmax_mxfp8 = 0 suffices. */
int window_anchor_attn_mxfp8_fwd(const vdn_shape* shape, const void* q_codes,
                                 const void* q_scales, const void* k_codes,
                                 const void* k_scales, const void* v,
                                 const void* gate_s, void* out, float* lse,
                                 void* ws, size_t ws_bytes, void* stream);

/* Dense full-softmax baseline layer, the cost reference of the length sweep
 * (10100.com article, 实验结果 / 效率阶梯: softmax density and backbone
 * speedup against dense attention as the number of latent frames grows):
 *   out = concat_h(softmax over all L keys of scale * q_l . k) @ v) @ w_o
 * No gates and one output projection w_o [D, D].  The window and anchor fields
 * of `shape` are ignored (every key frame is allowed); batch, heads, frames,
 * tokens_per_frame, head_dim, softmax_scale and dtype are read.  The
 * workspace (op VDN_OP_DENSE_ATTN) holds w_o transposed and the attention
 * output [B, L, D]. */
int vdn_dense_attn_fwd(const vdn_shape* shape, const void* q, const void* k,
                       const void* v, const void* w_o, void* out, void* ws,
                       size_t ws_bytes, void* stream);

/* Opt-in range check of gamma and beta (a debugging aid).  While on, every
 * call of vdn_hybrid_attn_fwd and vda_scan_fwd first runs one small kernel
 * over the B*H*T entries of gamma and beta, then waits for the stream and
 * returns VDN_ERR_PARAM_RANGE (nothing else enqueued) if some beta < 0 or
 * some gamma lies outside [0, 1].  The verdict travels through a 256-byte
 * slot of those calls' workspace (always reserved).  Process-wide; off by default.  Returns
 * the previous setting. */
int vdn_set_param_check(int on);

/* Phase timing, a tracing aid for benchmarks.  Between vdn_timing_start()
 * and vdn_timing_stop() every compute entry point records a pair of HIP
 * events on its stream around each of its phases (transposes, gate GEMM,
 * window attention, anchor-row merge, VDA gram / solve / scan / readout,
 * output GEMM).  vdn_timing_stop() waits for those events, then fills up to
 * max_stats entries with the phase name, the number of launches recorded and
 * their summed duration in milliseconds, and returns the number of phases
 * (or a negative status).  Event recording does not synchronise the stream;
 * timing state is process-wide, so time one stream at a time. */
typedef struct vdn_phase_stat {
  const char* name;  /* static string owned by the library */
  int32_t launches;
  float total_ms;
} vdn_phase_stat;

int vdn_timing_start(void);
int vdn_timing_stop(vdn_phase_stat* stats, int max_stats);

/* Message of the last failing call on this thread ("" if none). */
const char* vdn_last_error(void);

/* Library version string. */
const char* vdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VDN_H */
