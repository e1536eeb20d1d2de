// C ABI of libvdn.so (declared in include/vdn.h): argument validation,
// workspace layout and the launch sequence of each entry point.  No device
// memory is allocated here; every buffer comes from the caller, except the
// fixed static scratch array of the allocation-free linear-branch entry point.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "vda_bwd.h"
#include "vdn.h"
#include "vdn_internal.h"

using namespace vdn;

// Scratch of vda_scan_fwd_noalloc (the linear branch's per-frame statistics,
// transitions, states and their hi/lo copies, and the range-check verdict)
// for callers that cannot allocate.  Each device that loads the library
// holds its own copy until the process ends.  In host code the name is only
// a stand-in: the device address comes from hipGetSymbolAddress, once per
// device with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

size_t elem_size(int dtype) { return dtype == VDN_BF16 ? 2 : 4; }

int check_shape(const vdn_shape* s) {
  if (!s) return fail(VDN_ERR_INVALID_ARG, "shape is NULL");
  if (s->dtype != VDN_F32 && s->dtype != VDN_BF16)
    return fail(VDN_ERR_DTYPE, "dtype %d is not VDN_F32 (0) or VDN_BF16 (1)", s->dtype);
  if (s->batch < 1 || s->heads < 1 || s->frames < 1 || s->tokens_per_frame < 1)
    return fail(VDN_ERR_BAD_SHAPE, "batch, heads, frames and tokens_per_frame must be >= 1");
  if (s->head_dim != 32 && s->head_dim != 64 && s->head_dim != 128)
    return fail(VDN_ERR_BAD_SHAPE, "head_dim %d not in {32, 64, 128}", s->head_dim);
  if (s->chunk_frames < 1) return fail(VDN_ERR_BAD_SHAPE, "chunk_frames must be >= 1");
  if (s->context_tokens < 0) return fail(VDN_ERR_BAD_SHAPE, "context_tokens must be >= 0");
  if (s->window_chunks < 0) return fail(VDN_ERR_BAD_SHAPE, "window_chunks must be >= 0");
  if ((s->anchor_first != 0 && s->anchor_first != 1) || (s->anchor_last != 0 && s->anchor_last != 1))
    return fail(VDN_ERR_BAD_SHAPE, "anchor_first / anchor_last must be 0 or 1");
  if (!(s->rms_eps >= 0.f) || !isfinite(s->rms_eps))
    return fail(VDN_ERR_BAD_SHAPE, "rms_eps must be finite and >= 0");
  if (!isfinite(s->softmax_scale)) return fail(VDN_ERR_BAD_SHAPE, "softmax_scale must be finite");
  if (s->softmax_mxfp8 != 0 && s->softmax_mxfp8 != 1)
    return fail(VDN_ERR_BAD_SHAPE, "softmax_mxfp8 must be 0 or 1");
  if (s->softmax_mxfp8 && s->dtype != VDN_BF16)
    return fail(VDN_ERR_DTYPE, "softmax_mxfp8 needs dtype VDN_BF16");
  if (s->softmax_mxfp8 && s->head_dim != 128)
    return fail(VDN_ERR_BAD_SHAPE, "softmax_mxfp8 needs head_dim 128");
  const int64_t L = (int64_t)s->frames * s->tokens_per_frame + s->context_tokens;
  if (L > (1LL << 30))
    return fail(VDN_ERR_BAD_SHAPE, "frames * tokens_per_frame + context_tokens exceeds 2^30");
  const int64_t D = (int64_t)s->heads * s->head_dim;
  if (D > (1 << 20)) return fail(VDN_ERR_BAD_SHAPE, "heads * head_dim exceeds 2^20");
  if ((int64_t)s->batch * L > (1LL << 31) - 1)
    return fail(VDN_ERR_BAD_SHAPE, "batch * (frames * tokens_per_frame + context_tokens) exceeds 2^31 - 1");
  // the kernels address one (batch, head)'s q/k/v rows with 32-bit byte offsets
  if (L * s->head_dim * (s->dtype == VDN_BF16 ? 2 : 4) > (1LL << 31) - 1)
    return fail(VDN_ERR_BAD_SHAPE, "one (batch, head) of q/k/v exceeds 2 GiB");
  return VDN_OK;
}

// ---- softmax-branch work decomposition
AttnParams make_attn_params(const vdn_shape* s) {
  AttnParams p;
  memset(&p, 0, sizeof(p));
  const int T = s->frames, N = s->tokens_per_frame, C = s->chunk_frames;
  // a window of nC chunks on each side already reaches every frame
  const int W = s->window_chunks < (T + C - 1) / C ? s->window_chunks : (T + C - 1) / C;
  const int BM = attn_query_tile(s->dtype, s->head_dim), BN = kAttnBN;
  p.bm = BM;
  p.B = s->batch;
  p.H = s->heads;
  p.T = T;
  p.N = N;
  p.L = T * N;
  p.ctx = s->context_tokens;
  p.Lt = p.L + p.ctx;
  p.C = C;
  p.W = W;
  p.a0 = s->anchor_first;
  p.a1 = s->anchor_last;
  p.nC = (T + C - 1) / C;
  auto tiles = [&](int frames) { return frames > 0 ? (int)(((int64_t)frames * N + BM - 1) / BM) : 0; };
  if (p.nC == 1) {
    p.tiles0 = tiles(T - p.a0 - p.a1);
    p.n_window_tiles = p.tiles0;
  } else {
    p.tiles0 = tiles(C - p.a0);
    p.tilesM = tiles(C);
    p.tilesL = tiles(T - p.a1 - (p.nC - 1) * C);
    p.n_window_tiles = p.tiles0 + (p.nC - 2) * p.tilesM + p.tilesL;
  }
  // dense query groups, in row order: first frame, last frame, context tokens
  p.nG = 0;
  auto add_group = [&](int row0, int rows) {
    p.grp_row0[p.nG] = row0;
    p.grp_rows[p.nG] = rows;
    p.grp_tiles[p.nG] = (rows + BM - 1) / BM;
    p.grp_part[p.nG] = p.dense_rows;
    p.dense_rows += rows;
    ++p.nG;
  };
  if (p.a0) add_group(0, N);
  if (p.a1 && !(p.a0 && T == 1)) add_group((T - 1) * N, N);
  if (p.ctx > 0) add_group(p.L, p.ctx);
  const int64_t Lt = p.Lt;
  const int64_t key_tiles = (Lt + BN - 1) / BN;
  // Split dense rows so each piece sees about as many keys as a window tile.
  const int64_t win_frames = (int64_t)(2 * W + 1) * C + 2;
  const int64_t win_keys = (win_frames < T ? win_frames : T) * N + p.ctx;
  int64_t ns = p.nG ? (Lt + win_keys - 1) / win_keys : 1;
  if (ns < 1) ns = 1;
  if (ns > key_tiles) ns = key_tiles;
  const int64_t tiles_per_split = (key_tiles + ns - 1) / ns;
  p.keys_per_split = (int)(tiles_per_split * BN);
  p.nsplit = (int)((Lt + p.keys_per_split - 1) / p.keys_per_split);
  int dense_tiles = 0;
  for (int g = 0; g < p.nG; ++g) dense_tiles += p.grp_tiles[g];
  p.tiles_per_bh = p.n_window_tiles + p.nsplit * dense_tiles;
  p.total = p.B * p.H * p.tiles_per_bh;
  const float scale = s->softmax_scale > 0.f ? s->softmax_scale : 1.f / sqrtf((float)s->head_dim);
  p.scale_log2 = scale * 1.4426950408889634f;
  return p;
}

// ---- workspace layouts
struct VdaLayout {
  size_t am, bc, states, split, flag, total;
};
// The fp32 states are read back only by the fp32 readout and by a caller that
// asks for them: in bf16 I/O the readout takes the hi/lo pairs, and with
// head_dim 64 or 128 (the MFMA scan) the scan then writes no fp32 copy at all.
bool scan_keeps_fp32_states(const vdn_shape* s) {
  return !(s->dtype == VDN_BF16 && (s->head_dim == 128 || s->head_dim == 64));
}

VdaLayout vda_layout(const vdn_shape* s, bool need_states) {
  need_states = need_states && scan_keeps_fp32_states(s);
  const size_t dd = (size_t)s->head_dim * s->head_dim;
  const size_t frames = (size_t)s->batch * s->heads * s->frames;
  VdaLayout l;
  size_t off = 0;
  l.am = off; off = align_up(off + frames * dd * 4);
  l.bc = off; off = align_up(off + frames * dd * 4);
  l.states = off; off = align_up(off + (need_states ? 2 * frames * dd * 4 : 0));
  // bf16 I/O: states also as hi/lo bf16 pairs for the readout
  l.split = off; off = align_up(off + (s->dtype == VDN_BF16 ? 2 * frames * dd * 2 * 2 : 0));
  l.flag = off; off += kAlign;                                  // parameter-check verdict
  l.total = off;
  return l;
}

// Gradient of the linear branch: recomputed forward quantities, the adjoint
// chain's per-frame matrices ([frame][direction][d][d] where both directions
// are kept) and the token-side buffer U = S q, then du, [frame][direction][N][d].
struct VdaBwdLayout {
  size_t ones, kk, vk, am, bm, states, dsg, dx, xs, dm, p, da, cdb, u, dwp, flag, total;
};
VdaBwdLayout vda_bwd_layout(const vdn_shape* s) {
  const size_t d = s->head_dim, dd = d * d;
  const size_t nf = (size_t)s->batch * s->heads * s->frames;
  const size_t N = s->tokens_per_frame;
  VdaBwdLayout l;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  l.ones = take(nf * 4);             // beta = 1 for the recomputed Gram products
  l.kk = take(nf * dd * 4);          // K^T K
  l.vk = take(nf * dd * 4);          // V^T K
  l.am = take(nf * dd * 4);          // A_t, then M_t^T
  l.bm = take(nf * dd * 4);          // B_t
  l.states = take(2 * nf * dd * 4);  // S_t of both scans, [dir][frame]
  l.dsg = take(2 * nf * dd * 4);     // dS_t, then G_t
  l.dx = take(2 * nf * dd * 4);      // dX_t
  l.xs = take(2 * nf * dd * 4);      // X_t
  l.dm = take(nf * dd * 4);          // dM_t
  l.p = take(nf * dd * 4);           // M_t^T dM_t
  l.da = take(nf * dd * 4);          // dA_t
  l.cdb = take(2 * nf * dd * 4);     // [dA_t + dA_t^T, dB_t]
  l.u = take(nf * 2 * N * d * 4);    // u, then du
  l.dwp = take(nf * 2 * d * 4);      // partial RMSNorm-weight gradients
  l.flag = take(kAlign);
  l.total = off;
  return l;
}

struct AttnLayout {
  size_t part_o, part_ml, qc, qs, kc, ks, kmax, fallback, total;
};
// with softmax_mxfp8, q and k quantised to MXFP8 (codes [B, H, Lt, d], scales [B, H, Lt, d / 32])
AttnLayout attn_layout(const vdn_shape* s, const AttnParams& p) {
  AttnLayout l;
  size_t off = 0;
  const size_t rows = p.nsplit > 1 ? (size_t)p.B * p.H * p.nsplit * p.dense_rows : 0;
  l.part_o = off; off = align_up(off + rows * s->head_dim * 4);
  l.part_ml = off; off = align_up(off + rows * 2 * 4);
  const size_t elems = s->softmax_mxfp8 ? (size_t)p.B * p.H * p.Lt * s->head_dim : 0;
  l.qc = off; off = align_up(off + elems);
  l.qs = off; off = align_up(off + elems / 32);
  l.kc = off; off = align_up(off + elems);
  l.ks = off; off = align_up(off + elems / 32);
  // the bf16 head_dim-128 softmax kernel's fixed maximum: key-norm maxima and
  // the per-work-item fallback marks
  const bool fx = s->dtype == VDN_BF16 && s->head_dim == 128;
  l.kmax = off; off = align_up(off + (fx ? (size_t)p.B * p.H * kKeyNormParts * 4 : 0));
  l.fallback = off; off = align_up(off + (fx ? (size_t)p.total : 0));
  l.total = off;
  return l;
}

struct HybridLayout {
  size_t wg, wo, gates, ybuf, vda, attn, total;
};
HybridLayout hybrid_layout(const vdn_shape* s, const AttnParams& p) {
  const size_t es = elem_size(s->dtype);
  const size_t D = (size_t)s->heads * s->head_dim;
  const size_t rows = (size_t)s->batch * ((size_t)s->frames * s->tokens_per_frame + s->context_tokens);
  HybridLayout l;
  size_t off = 0;
  l.wg = off; off = align_up(off + 2 * D * D * es);       // [W_gs^T ; W_gl^T]   [2D, D]
  l.wo = off; off = align_up(off + 2 * D * D * es);       // [W_os^T | W_ol^T]   [D, 2D]
  l.gates = off; off = align_up(off + rows * 2 * D * es); // [g_s | g_l]         [B*L, 2D]
  l.ybuf = off; off = align_up(off + rows * 2 * D * es);  // [y_s | y_l]         [B*L, 2D]
  l.vda = off; off = align_up(off + vda_layout(s, true).total);
  l.attn = off; off = align_up(off + attn_layout(s, p).total);
  l.total = off;
  return l;
}

// Dense baseline: every key frame allowed, no anchors (they would add nothing).
vdn_shape dense_shape(const vdn_shape* s) {
  vdn_shape d = *s;
  d.window_chunks = (s->frames + s->chunk_frames - 1) / s->chunk_frames;
  d.anchor_first = 0;
  d.anchor_last = 0;
  return d;
}

struct DenseLayout {
  size_t wo, ybuf, attn, total;
};
DenseLayout dense_layout(const vdn_shape* s) {
  const vdn_shape ds = dense_shape(s);
  const size_t es = elem_size(s->dtype);
  const size_t D = (size_t)s->heads * s->head_dim;
  const size_t rows = (size_t)s->batch * ((size_t)s->frames * s->tokens_per_frame + s->context_tokens);
  DenseLayout l;
  size_t off = 0;
  l.wo = off; off = align_up(off + D * D * es);          // W_o^T  [D, D]
  l.ybuf = off; off = align_up(off + rows * D * es);     // softmax output [B*L, D]
  l.attn = off; off = align_up(off + attn_layout(&ds, make_attn_params(&ds)).total);
  l.total = off;
  return l;
}

bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 15u) != 0; }

std::atomic<int> g_param_check{0};

// With the range check on: run it, wait for the stream, report a violation.
int check_params(const vdn_shape* s, const float* gamma, const float* beta, char* flag_slot,
                 hipStream_t st) {
  if (!g_param_check.load(std::memory_order_relaxed)) return VDN_OK;
  const int n = s->batch * s->heads * s->frames;
  int* flag = (int*)flag_slot;
  hipError_t e = launch_param_check(gamma, beta, n, flag, st);
  int host_flag = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess)
    return fail(VDN_ERR_HIP, "parameter check: %s", hipGetErrorString(e));
  if (host_flag)
    return fail(VDN_ERR_PARAM_RANGE, "parameter check: some beta < 0 or gamma outside [0, 1]");
  return VDN_OK;
}

// ---- opt-in phase timing: HIP event pairs recorded around each phase
enum Phase {
  kPhTranspose, kPhGateGemm, kPhWindowAttn, kPhAnchorMerge, kPhGram, kPhSolve, kPhScan,
  kPhReadout, kPhOutGemm, kPhQuantize, kPhBwdRecompute, kPhBwdU, kPhBwdRms, kPhBwdDq, kPhBwdDs,
  kPhBwdScan, kPhBwdFrame, kPhBwdKv, kPhBwdDw, kPhBwdToken, kPhKeyNorms, kNumPhases
};
const char* const kPhaseNames[kNumPhases] = {"transpose_weights", "gate_gemm", "window_attn",
                                             "anchor_merge",      "vda_gram",  "vda_solve",
                                             "vda_scan",          "vda_readout", "out_gemm",
                                             "mxfp8_quantize", "bwd_recompute", "bwd_u_gemm",
                                             "bwd_rms",        "bwd_dq_gemm", "bwd_ds_gemm",
                                             "bwd_scan",       "bwd_frame",   "bwd_kv_gemm",
                                             "bwd_dw",         "bwd_token",   "key_norms"};

struct Timer {
  std::mutex mu;
  bool on = false;
  bool failed = false;
  struct Rec { int phase; hipEvent_t a, b; };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;   // events are reused across timing sessions
  size_t used = 0;
  hipEvent_t take() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) { failed = true; return nullptr; }
      pool.push_back(e);
    }
    return pool[used++];
  }
};
Timer g_timer;

// Returns a record index, or -1 when timing is off.
int phase_begin(int phase, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (!g_timer.on || g_timer.failed) return -1;
  hipEvent_t a = g_timer.take(), b = g_timer.take();
  if (!a || !b) return -1;
  hipEventRecord(a, st);
  g_timer.recs.push_back({phase, a, b});
  return (int)g_timer.recs.size() - 1;
}

void phase_end(int idx, hipStream_t st) {
  if (idx < 0) return;
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (idx < (int)g_timer.recs.size()) hipEventRecord(g_timer.recs[idx].b, st);
}

int hip_fail(hipError_t e, const char* what) {
  return fail(VDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(char** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VDN_ERR_INVALID_ARG, "device %d is beyond the %d devices the scratch table covers", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = (char*)p;
  }
  *ptr = g_scratch_ptr[dev];
  return VDN_OK;
}

// Linear branch on already validated arguments.
int run_vda(const vdn_shape* s, const void* q, const void* k, const void* v,
            const float* gamma, const float* beta, const float* rms_w, const void* gate,
            int64_t ldg, void* out, int64_t ldo, float* states, char* ws, hipStream_t st) {
  const VdaLayout l = vda_layout(s, states == nullptr);
  float* am = (float*)(ws + l.am);
  float* bc = (float*)(ws + l.bc);
  float* st_buf = states ? states : scan_keeps_fp32_states(s) ? (float*)(ws + l.states) : nullptr;
  __bf16* split = s->dtype == VDN_BF16 ? (__bf16*)(ws + l.split) : nullptr;
  const int d = s->head_dim;
  const int nframes = s->batch * s->heads * s->frames;
  const int N = s->tokens_per_frame, L = s->frames * N, Lt = L + s->context_tokens;
  hipError_t e;
  // the linear branch covers video tokens only: its output is zero on context rows
  if (s->context_tokens > 0) {
    e = launch_zero_rows(out, s->batch, Lt, L, s->context_tokens, ldo, (int64_t)s->heads * d,
                         s->dtype == VDN_BF16 ? 2 : 4, st);
    if (e != hipSuccess) return hip_fail(e, "zero fill launch");
  }
  int ph = phase_begin(kPhGram, st);
  e = launch_vda_gram(s->dtype, d, k, v, beta, am, bc, nframes, s->frames, N, Lt, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "vda gram launch");
  ph = phase_begin(kPhSolve, st);
  e = launch_vda_solve(d, am, nframes, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "vda solve launch");
  ph = phase_begin(kPhScan, st);
  e = launch_vda_scan(d, am, bc, gamma, st_buf, split, s->batch * s->heads, s->frames, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "vda scan launch");
  ph = phase_begin(kPhReadout, st);
  e = launch_vda_readout(s->dtype, d, q, st_buf, split, rms_w, gate, ldg, out, ldo, s->batch,
                         s->heads, s->frames, N, Lt, s->rms_eps, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "vda readout launch");
  return VDN_OK;
}

// Gradient of the linear branch on already validated arguments: the forward
// quantities are recomputed (Gram products without beta, then scaled), then
// the adjoint runs readout -> scans -> solve -> Gram.
int run_vda_bwd(const vdn_shape* s, const void* q, const void* k, const void* v, const float* gamma,
                const float* beta, const float* rms_w, const void* d_out, void* dq, void* dk, void* dv,
                float* dgamma, float* dbeta, float* drms_w, char* ws, hipStream_t st) {
  const VdaBwdLayout l = vda_bwd_layout(s);
  float* ones = (float*)(ws + l.ones);
  float* kk = (float*)(ws + l.kk);
  float* vk = (float*)(ws + l.vk);
  float* am = (float*)(ws + l.am);
  float* bm = (float*)(ws + l.bm);
  float* states = (float*)(ws + l.states);
  float* dsg = (float*)(ws + l.dsg);
  float* dx = (float*)(ws + l.dx);
  float* xs = (float*)(ws + l.xs);
  float* dm = (float*)(ws + l.dm);
  float* pm = (float*)(ws + l.p);
  float* da = (float*)(ws + l.da);
  float* cdb = (float*)(ws + l.cdb);
  float* u = (float*)(ws + l.u);
  float* dwp = (float*)(ws + l.dwp);
  const int dt = s->dtype, d = s->head_dim, H = s->heads, T = s->frames, N = s->tokens_per_frame;
  const int L = T * N, Lt = L + s->context_tokens, BH = s->batch * H;
  const int64_t nf = (int64_t)BH * T, dd = (int64_t)d * d, Nd = (int64_t)N * d, Ltd = (int64_t)Lt * d;
  const int es = dt == VDN_BF16 ? 2 : 4;
  // bf16 I/O: token-side products on bf16 MFMA (fp32 operands split hi + lo)
  const bool mfma = dt == VDN_BF16;
  hipError_t e = hipSuccess;
  auto step = [&](int phase, const char* what, auto&& body) -> int {
    const int ph = phase_begin(phase, st);
    e = body();
    phase_end(ph, st);
    return e == hipSuccess ? VDN_OK : hip_fail(e, what);
  };
  int rc;
  if (s->context_tokens > 0) {
    // the linear branch does not read context rows: their gradient is zero
    for (void* g : {dq, dk, dv}) {
      e = launch_zero_rows(g, BH, Lt, L, s->context_tokens, d, d, es, st);
      if (e != hipSuccess) return hip_fail(e, "zero fill launch");
    }
  }
  rc = step(kPhBwdRecompute, "vda_bwd recompute", [&] {
    hipError_t r = launch_fill(ones, 1.f, nf, st);
    if (r == hipSuccess) r = launch_vda_gram(dt, d, k, v, ones, kk, vk, (int)nf, T, N, Lt, st);
    if (r == hipSuccess) r = launch_scale_frames(kk, vk, beta, am, bm, nf, dd, st);
    if (r == hipSuccess) r = launch_vda_solve(d, am, (int)nf, st);
    if (r == hipSuccess) r = launch_vda_scan(d, am, bm, gamma, states, nullptr, BH, T, st);
    return r;
  });
  if (rc != VDN_OK) return rc;

  if (dt == VDN_BF16 && d == 128) {
    // u, du, dq, dS and the RMSNorm-weight partials in one pass per direction; u and du
    // never leave the chip (the u buffer holds dq's fp32 share of the first direction)
    rc = step(kPhBwdToken, "vda_bwd token launch", [&] {
      return launch_tok_grad(q, d_out, (int64_t)H * d, states, rms_w, u, dq, dsg, dwp, nf, H, T, N, Lt,
                             s->rms_eps, st);
    });
    if (rc != VDN_OK) return rc;
  } else {
    // U[f][dir] = Q_t S_dir,t^T
    BGemm g;
    g.a0 = q; g.b0 = states; g.c = u;
    g.M = N; g.N = d; g.K = d;
    g.sam = d; g.sak = 1; g.sbk = 1; g.sbn = d; g.ldc = d;
    g.batch = 2 * nf; g.n0 = 2; g.n1 = T;
    g.sa[0] = 0; g.sa[1] = Nd; g.sa[2] = Ltd;
    g.sb[0] = nf * dd; g.sb[1] = dd; g.sb[2] = T * dd;
    g.sc[0] = Nd; g.sc[1] = 2 * Nd; g.sc[2] = T * 2 * Nd;
    rc = step(kPhBwdU, "vda_bwd u launch", [&] { return launch_bgemm(dt, 0, 0, g, st, mfma); });
    if (rc != VDN_OK) return rc;
    rc = step(kPhBwdRms, "vda_bwd rms launch", [&] {
      return launch_rms_bwd(dt, d, u, d_out, (int64_t)H * d, rms_w, dwp, nf, H, T, N, Lt, s->rms_eps, st);
    });
    if (rc != VDN_OK) return rc;

    // dq = du_f S_f + du_b S_b (K = 2d over the two directions)
    g = BGemm();
    g.a0 = u; g.a1 = u + Nd; g.b0 = states; g.b1 = states + nf * dd; g.c = dq;
    g.M = N; g.N = d; g.K = 2 * d; g.ks = d;
    g.sam = d; g.sak = 1; g.sbk = d; g.sbn = 1; g.ldc = d;
    g.batch = nf; g.n0 = T; g.n1 = 1;
    g.sa[0] = 2 * Nd; g.sa[2] = T * 2 * Nd;
    g.sb[0] = dd; g.sb[2] = T * dd;
    g.sc[0] = Nd; g.sc[2] = Ltd;
    rc = step(kPhBwdDq, "vda_bwd dq launch", [&] { return launch_bgemm(0, 0, dt, g, st, mfma); });
    if (rc != VDN_OK) return rc;

    // dS[f][dir] = du^T Q_t (sum over the frame's tokens)
    g = BGemm();
    g.a0 = u; g.b0 = q; g.c = dsg;
    g.M = d; g.N = d; g.K = N;
    g.sam = 1; g.sak = d; g.sbk = d; g.sbn = 1; g.ldc = d;
    g.batch = 2 * nf; g.n0 = 2; g.n1 = T;
    g.sa[0] = Nd; g.sa[1] = 2 * Nd; g.sa[2] = T * 2 * Nd;
    g.sb[0] = 0; g.sb[1] = Nd; g.sb[2] = Ltd;
    g.sc[0] = dd; g.sc[1] = 2 * dd; g.sc[2] = T * 2 * dd;
    rc = step(kPhBwdDs, "vda_bwd dS launch", [&] { return launch_bgemm(0, dt, 0, g, st, mfma); });
    if (rc != VDN_OK) return rc;
  }

  rc = step(kPhBwdScan, "vda_bwd scan launch", [&] { return launch_scan_bwd(d, am, gamma, dsg, dx, BH, T, st); });
  if (rc != VDN_OK) return rc;

  rc = step(kPhBwdFrame, "vda_bwd frame launch", [&] {
    hipError_t r = launch_frame_bwd(states, bm, gamma, dx, xs, cdb, dgamma, T, nf, d, st);
    // dM = sum_dir X^T G (K = 2d over the stacked directions)
    BGemm m;
    m.a0 = xs; m.b0 = dsg; m.c = dm;
    m.M = d; m.N = d; m.K = 2 * d;
    m.sam = 1; m.sak = d; m.sbk = d; m.sbn = 1; m.ldc = d;
    m.batch = nf; m.n0 = T; m.n1 = 1;
    m.sa[0] = 2 * dd; m.sa[2] = T * 2 * dd;
    m.sb[0] = 2 * dd; m.sb[2] = T * 2 * dd;
    m.sc[0] = dd; m.sc[2] = T * dd;
    if (r == hipSuccess) r = launch_bgemm(0, 0, 0, m, st);
    // P = M^T dM, then dA = -P M^T (am holds M^T)
    m = BGemm();
    m.a0 = am; m.b0 = dm; m.c = pm;
    m.M = d; m.N = d; m.K = d;
    m.sam = d; m.sak = 1; m.sbk = d; m.sbn = 1; m.ldc = d;
    m.batch = nf; m.n0 = T; m.n1 = 1;
    m.sa[0] = dd; m.sa[2] = T * dd;
    m.sb[0] = dd; m.sb[2] = T * dd;
    m.sc[0] = dd; m.sc[2] = T * dd;
    if (r == hipSuccess) r = launch_bgemm(0, 0, 0, m, st);
    m.a0 = pm; m.b0 = am; m.c = da; m.alpha = -1.f;
    if (r == hipSuccess) r = launch_bgemm(0, 0, 0, m, st);
    if (r == hipSuccess) r = launch_sym_dbeta(d, da, kk, vk, cdb, dbeta, nf, st);
    return r;
  });
  if (rc != VDN_OK) return rc;

  rc = step(kPhBwdKv, "vda_bwd dk/dv launch", [&] {
    // bf16 at head_dim 128: both in one pass over K and V
    if (dt == VDN_BF16 && d == 128) return launch_kv_grad(k, v, cdb, beta, dk, dv, nf, T, N, Lt, st);
    // dK = beta (K (dA + dA^T) + V dB)  (K = 2d over [K | V] and [dA + dA^T ; dB])
    BGemm m;
    m.a0 = k; m.a1 = v; m.b0 = cdb; m.b1 = cdb + dd; m.c = dk;
    m.M = N; m.N = d; m.K = 2 * d; m.ks = d;
    m.sam = d; m.sak = 1; m.sbk = d; m.sbn = 1; m.ldc = d;
    m.batch = nf; m.n0 = T; m.n1 = 1;
    m.sa[0] = Nd; m.sa[2] = Ltd;
    m.sb[0] = 2 * dd; m.sb[2] = T * 2 * dd;
    m.sc[0] = Nd; m.sc[2] = Ltd;
    m.alpha_z = beta;
    hipError_t r = launch_bgemm(dt, 0, dt, m, st, mfma);
    // dV = beta K dB^T
    m.a1 = nullptr; m.b0 = cdb + dd; m.b1 = nullptr; m.c = dv;
    m.K = d; m.ks = 0; m.sbk = 1; m.sbn = d;
    if (r == hipSuccess) r = launch_bgemm(dt, 0, dt, m, st, mfma);
    return r;
  });
  if (rc != VDN_OK) return rc;
  if (drms_w) {
    rc = step(kPhBwdDw, "vda_bwd dw launch", [&] { return launch_dw_reduce(dwp, drms_w, s->batch, H, T, d, st); });
    if (rc != VDN_OK) return rc;
  }
  return VDN_OK;
}

// Softmax branch.  With s->softmax_mxfp8, q and k are quantised into the
// workspace first, unless qs / ks already point at MXFP8 scales (then q and k
// are the codes).
int run_attn(const vdn_shape* s, const void* q, const void* k, const void* v, const void* gate,
             int64_t ldg, void* out, int64_t ldo, float* lse, char* ws, hipStream_t st,
             const void* qs = nullptr, const void* ks = nullptr) {
  AttnParams p = make_attn_params(s);
  const AttnLayout l = attn_layout(s, p);
  p.q = q;
  p.k = k;
  p.v = v;
  p.gate = gate;
  p.out = out;
  p.lse = lse;
  p.ldg = ldg;
  p.ldo = ldo;
  p.part_o = (float*)(ws + l.part_o);
  p.part_ml = (float*)(ws + l.part_ml);
  const bool mx = s->softmax_mxfp8 || qs;
  hipError_t e;
  int ph;
  if (mx && !qs) {
    const int64_t n = (int64_t)p.B * p.H * p.Lt * s->head_dim;
    ph = phase_begin(kPhQuantize, st);
    e = launch_mxfp8_quantize(q, n, ws + l.qc, ws + l.qs, st);
    if (e == hipSuccess) e = launch_mxfp8_quantize(k, n, ws + l.kc, ws + l.ks, st);
    phase_end(ph, st);
    if (e != hipSuccess) return hip_fail(e, "mxfp8 quantize launch");
    p.q = ws + l.qc;
    p.qs = ws + l.qs;
    p.k = ws + l.kc;
    p.ks = ws + l.ks;
  } else if (mx) {
    p.qs = qs;
    p.ks = ks;
  }
  if (!mx && s->dtype == VDN_BF16 && s->head_dim == 128 && p.total > 0) {
    p.kmax = (float*)(ws + l.kmax);
    p.kmax_parts = kKeyNormParts;
    p.fallback = (unsigned char*)(ws + l.fallback);
    ph = phase_begin(kPhKeyNorms, st);
    e = launch_key_norm_max(k, (float*)(ws + l.kmax), (int64_t)p.B * p.H, p.Lt, kKeyNormParts, st);
    phase_end(ph, st);
    if (e != hipSuccess) return hip_fail(e, "key norm launch");
  }
  ph = phase_begin(kPhWindowAttn, st);
  e = mx ? launch_window_attn_mxfp8(p, st) : launch_window_attn(s->dtype, s->head_dim, p, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "window attention launch");
  ph = phase_begin(kPhAnchorMerge, st);
  e = launch_attn_merge(s->dtype, s->head_dim, p, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "anchor merge launch");
  return VDN_OK;
}

// Argument checks shared by the two linear-branch forward entry points.
int check_vda_args(const char* fn, const vdn_shape* shape, const void* q, const void* k, const void* v,
                   const float* gamma, const float* beta, const void* gate_l, const void* out,
                   const float* states, const void* ws) {
  int rc = check_shape(shape);
  if (rc != VDN_OK) return rc;
  if (!q || !k || !v || !gamma || !beta || !out)
    return fail(VDN_ERR_INVALID_ARG, "%s: q, k, v, gamma, beta and out must be non-NULL", fn);
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(gate_l) ||
      misaligned(states) || misaligned(ws) || misaligned(gamma) || misaligned(beta))
    return fail(VDN_ERR_INVALID_ARG, "%s: device pointers must be 16-byte aligned", fn);
  return VDN_OK;
}

}  // namespace

extern "C" {

const char* vdn_last_error(void) { return g_err; }

const char* vdn_version(void) { return "vdn-mi355x 0.1 (gfx950)"; }

size_t vdn_workspace_bytes(const vdn_shape* shape, int op) {
  if (check_shape(shape) != VDN_OK) return 0;
  const AttnParams p = make_attn_params(shape);
  size_t n = 0;
  switch (op) {
    case VDN_OP_HYBRID: n = hybrid_layout(shape, p).total; break;
    case VDN_OP_VDA_SCAN: n = vda_layout(shape, true).total; break;
    case VDN_OP_WINDOW_ATTN: n = attn_layout(shape, p).total; break;
    case VDN_OP_DENSE_ATTN: n = dense_layout(shape).total; break;
    case VDN_OP_VDA_BWD: n = vda_bwd_layout(shape).total; break;
    default: fail(VDN_ERR_INVALID_ARG, "unknown op %d", op); return 0;
  }
  // Never 0 for a valid request, so that 0 always signals an error.
  return n > kAlign ? n : kAlign;
}

int vda_scan_fwd(const vdn_shape* shape, const void* q, const void* k, const void* v,
                 const float* gamma, const float* beta, const float* rms_w, const void* gate_l,
                 void* out, float* states, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_vda_args("vda_scan_fwd", shape, q, k, v, gamma, beta, gate_l, out, states, ws);
  if (rc != VDN_OK) return rc;
  const size_t need = vda_layout(shape, states == nullptr).total;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(VDN_ERR_WORKSPACE, "vda_scan_fwd: workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : (size_t)0);
  rc = check_params(shape, gamma, beta, (char*)ws + vda_layout(shape, states == nullptr).flag,
                    (hipStream_t)stream);
  if (rc != VDN_OK) return rc;
  const int64_t D = (int64_t)shape->heads * shape->head_dim;
  return run_vda(shape, q, k, v, gamma, beta, rms_w, gate_l, D, out, D, states, (char*)ws,
                 (hipStream_t)stream);
}

int vda_scan_fwd_noalloc(const vdn_shape* shape, const void* q, const void* k, const void* v,
                         const float* gamma, const float* beta, const float* rms_w, const void* gate_l,
                         void* out, float* states, void* stream) {
  int rc = check_vda_args("vda_scan_fwd_noalloc", shape, q, k, v, gamma, beta, gate_l, out, states, nullptr);
  if (rc != VDN_OK) return rc;
  const VdaLayout l = vda_layout(shape, states == nullptr);
  if (l.total > kScratchBytes)
    return fail(VDN_ERR_WORKSPACE,
                "vda_scan_fwd_noalloc: the shape needs %zu bytes of scratch, the static scratch holds %zu "
                "(call vda_scan_fwd with a workspace)", l.total, kScratchBytes);
  char* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != VDN_OK) return rc;
  rc = check_params(shape, gamma, beta, ws + l.flag, (hipStream_t)stream);
  if (rc != VDN_OK) return rc;
  const int64_t D = (int64_t)shape->heads * shape->head_dim;
  return run_vda(shape, q, k, v, gamma, beta, rms_w, gate_l, D, out, D, states, ws, (hipStream_t)stream);
}

int vda_scan_bwd(const vdn_shape* shape, const void* q, const void* k, const void* v,
                 const float* gamma, const float* beta, const float* rms_w, const void* d_out,
                 void* dq, void* dk, void* dv, float* dgamma, float* dbeta, float* drms_w, void* ws,
                 size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc != VDN_OK) return rc;
  if (!q || !k || !v || !gamma || !beta || !d_out || !dq || !dk || !dv || !dgamma || !dbeta)
    return fail(VDN_ERR_INVALID_ARG,
                "vda_scan_bwd: q, k, v, gamma, beta, d_out, dq, dk, dv, dgamma and dbeta must be non-NULL");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(d_out) || misaligned(dq) ||
      misaligned(dk) || misaligned(dv) || misaligned(ws) || misaligned(gamma) || misaligned(beta) ||
      misaligned(rms_w) || misaligned(dgamma) || misaligned(dbeta) || misaligned(drms_w))
    return fail(VDN_ERR_INVALID_ARG, "vda_scan_bwd: device pointers must be 16-byte aligned");
  if ((int64_t)shape->batch * shape->heads > 65535)
    return fail(VDN_ERR_BAD_SHAPE, "vda_scan_bwd: batch * heads exceeds 65535");
  const size_t need = vda_bwd_layout(shape).total;
  if (!ws || ws_bytes < need)
    return fail(VDN_ERR_WORKSPACE, "vda_scan_bwd: workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : (size_t)0);
  rc = check_params(shape, gamma, beta, (char*)ws + vda_bwd_layout(shape).flag, (hipStream_t)stream);
  if (rc != VDN_OK) return rc;
  return run_vda_bwd(shape, q, k, v, gamma, beta, rms_w, d_out, dq, dk, dv, dgamma, dbeta, drms_w,
                     (char*)ws, (hipStream_t)stream);
}

int window_anchor_attn_fwd(const vdn_shape* shape, const void* q, const void* k, const void* v,
                           const void* gate_s, void* out, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
  int rc = check_shape(shape);
  if (rc != VDN_OK) return rc;
  if (!q || !k || !v || !out)
    return fail(VDN_ERR_INVALID_ARG, "window_anchor_attn_fwd: q, k, v and out must be non-NULL");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(gate_s) ||
      misaligned(ws))
    return fail(VDN_ERR_INVALID_ARG, "window_anchor_attn_fwd: device pointers must be 16-byte aligned");
  const AttnParams p = make_attn_params(shape);
  const size_t need = attn_layout(shape, p).total;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(VDN_ERR_WORKSPACE, "window_anchor_attn_fwd: workspace of %zu bytes needed, %zu given",
                need, ws ? ws_bytes : (size_t)0);
  const int64_t D = (int64_t)shape->heads * shape->head_dim;
  return run_attn(shape, q, k, v, gate_s, D, out, D, lse, (char*)ws, (hipStream_t)stream);
}

int vdn_mxfp8_quantize(const void* x, int64_t n_elems, void* codes, void* scales, void* stream) {
  if (!x || !codes || !scales)
    return fail(VDN_ERR_INVALID_ARG, "vdn_mxfp8_quantize: x, codes and scales must be non-NULL");
  if (misaligned(x) || misaligned(codes))
    return fail(VDN_ERR_INVALID_ARG, "vdn_mxfp8_quantize: x and codes must be 16-byte aligned");
  if (n_elems < 0 || n_elems % 32)
    return fail(VDN_ERR_BAD_SHAPE, "vdn_mxfp8_quantize: n_elems %lld is not a non-negative multiple of 32",
                (long long)n_elems);
  const hipError_t e = launch_mxfp8_quantize(x, n_elems, codes, scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mxfp8 quantize launch");
  return VDN_OK;
}

int window_anchor_attn_mxfp8_fwd(const vdn_shape* shape, const void* q_codes, const void* q_scales,
                                 const void* k_codes, const void* k_scales, const void* v,
                                 const void* gate_s, void* out, float* lse, void* ws, size_t ws_bytes,
                                 void* stream) {
  int rc = check_shape(shape);
  if (rc != VDN_OK) return rc;
  if (shape->dtype != VDN_BF16)
    return fail(VDN_ERR_DTYPE, "window_anchor_attn_mxfp8_fwd: v, gate and out must be bf16");
  if (shape->head_dim != 128)
    return fail(VDN_ERR_BAD_SHAPE, "window_anchor_attn_mxfp8_fwd: head_dim must be 128");
  if (!q_codes || !q_scales || !k_codes || !k_scales || !v || !out)
    return fail(VDN_ERR_INVALID_ARG,
                "window_anchor_attn_mxfp8_fwd: codes, scales, v and out must be non-NULL");
  if (misaligned(q_codes) || misaligned(q_scales) || misaligned(k_codes) || misaligned(k_scales) ||
      misaligned(v) || misaligned(out) || misaligned(gate_s) || misaligned(ws))
    return fail(VDN_ERR_INVALID_ARG, "window_anchor_attn_mxfp8_fwd: device pointers must be 16-byte aligned");
  vdn_shape s = *shape;
  s.softmax_mxfp8 = 0;   // the codes are given: no quantisation buffers
  const AttnParams p = make_attn_params(&s);
  const size_t need = attn_layout(&s, p).total;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(VDN_ERR_WORKSPACE, "window_anchor_attn_mxfp8_fwd: workspace of %zu bytes needed, %zu given",
                need, ws ? ws_bytes : (size_t)0);
  const int64_t D = (int64_t)shape->heads * shape->head_dim;
  return run_attn(&s, q_codes, k_codes, v, gate_s, D, out, D, lse, (char*)ws, (hipStream_t)stream,
                  q_scales, k_scales);
}

int vdn_hybrid_attn_fwd(const vdn_shape* shape, const void* x, const void* q, const void* k,
                        const void* v, const float* gamma, const float* beta, const void* w_gs,
                        const void* w_gl, const float* rms_w, const void* w_os, const void* w_ol,
                        void* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc != VDN_OK) return rc;
  if (!x || !q || !k || !v || !gamma || !beta || !w_gs || !w_gl || !w_os || !w_ol || !out)
    return fail(VDN_ERR_INVALID_ARG,
                "vdn_hybrid_attn_fwd: every input except rms_w, and out, must be non-NULL");
  const void* ptrs[] = {x, q, k, v, gamma, beta, w_gs, w_gl, rms_w, w_os, w_ol, out, ws};
  for (const void* ptr : ptrs)
    if (misaligned(ptr))
      return fail(VDN_ERR_INVALID_ARG, "vdn_hybrid_attn_fwd: device pointers must be 16-byte aligned");
  const AttnParams p = make_attn_params(shape);
  const HybridLayout l = hybrid_layout(shape, p);
  if (!ws || ws_bytes < l.total)
    return fail(VDN_ERR_WORKSPACE, "vdn_hybrid_attn_fwd: workspace of %zu bytes needed, %zu given",
                l.total, ws ? ws_bytes : (size_t)0);

  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  rc = check_params(shape, gamma, beta, w + l.vda + vda_layout(shape, true).flag, st);
  if (rc != VDN_OK) return rc;
  const size_t es = elem_size(shape->dtype);
  const int D = shape->heads * shape->head_dim;
  const int rows = shape->batch * (shape->frames * shape->tokens_per_frame + shape->context_tokens);
  char* wg = w + l.wg;
  char* wo = w + l.wo;
  char* gates = w + l.gates;
  char* ybuf = w + l.ybuf;
  hipError_t e;
  // weights -> k-contiguous: wg[n][k] (n < D: W_gs, n >= D: W_gl); wo[n][k] (k < D: W_os, else W_ol)
  int ph = phase_begin(kPhTranspose, st);
  e = launch_transpose(shape->dtype, w_gs, wg, D, D, D, st);
  if (e == hipSuccess) e = launch_transpose(shape->dtype, w_gl, wg + (size_t)D * D * es, D, D, D, st);
  if (e == hipSuccess) e = launch_transpose(shape->dtype, w_os, wo, D, D, 2 * (int64_t)D, st);
  if (e == hipSuccess) e = launch_transpose(shape->dtype, w_ol, wo + (size_t)D * es, D, D, 2 * (int64_t)D, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "transpose launch");
  // gates [g_s | g_l] = sigmoid(x [W_gs | W_gl])
  ph = phase_begin(kPhGateGemm, st);
  e = launch_gemm_nt(shape->dtype, kEpiSigmoid, x, wg, gates, rows, 2 * D, D, D, D, 2 * (int64_t)D, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "gate gemm launch");
  // y_s = g_s * softmax branch ; y_l = g_l * linear branch
  rc = run_attn(shape, q, k, v, gates, 2 * (int64_t)D, ybuf, 2 * (int64_t)D, nullptr, w + l.attn, st);
  if (rc != VDN_OK) return rc;
  rc = run_vda(shape, q, k, v, gamma, beta, rms_w, gates + (size_t)D * es, 2 * (int64_t)D,
               ybuf + (size_t)D * es, 2 * (int64_t)D, nullptr, w + l.vda, st);
  if (rc != VDN_OK) return rc;
  // out = [y_s | y_l] [W_os ; W_ol]
  ph = phase_begin(kPhOutGemm, st);
  e = launch_gemm_nt(shape->dtype, kEpiStore, ybuf, wo, out, rows, D, 2 * D, 2 * (int64_t)D,
                     2 * (int64_t)D, D, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "output gemm launch");
  return VDN_OK;
}

int vdn_dense_attn_fwd(const vdn_shape* shape, const void* q, const void* k, const void* v,
                       const void* w_o, void* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc != VDN_OK) return rc;
  if (!q || !k || !v || !w_o || !out)
    return fail(VDN_ERR_INVALID_ARG, "vdn_dense_attn_fwd: q, k, v, w_o and out must be non-NULL");
  const void* ptrs[] = {q, k, v, w_o, out, ws};
  for (const void* ptr : ptrs)
    if (misaligned(ptr))
      return fail(VDN_ERR_INVALID_ARG, "vdn_dense_attn_fwd: device pointers must be 16-byte aligned");
  const DenseLayout l = dense_layout(shape);
  if (!ws || ws_bytes < l.total)
    return fail(VDN_ERR_WORKSPACE, "vdn_dense_attn_fwd: workspace of %zu bytes needed, %zu given",
                l.total, ws ? ws_bytes : (size_t)0);
  const vdn_shape ds = dense_shape(shape);
  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  const int D = shape->heads * shape->head_dim;
  const int rows = shape->batch * (shape->frames * shape->tokens_per_frame + shape->context_tokens);
  int ph = phase_begin(kPhTranspose, st);
  hipError_t e = launch_transpose(shape->dtype, w_o, w + l.wo, D, D, D, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "transpose launch");
  rc = run_attn(&ds, q, k, v, nullptr, D, w + l.ybuf, D, nullptr, w + l.attn, st);
  if (rc != VDN_OK) return rc;
  ph = phase_begin(kPhOutGemm, st);
  e = launch_gemm_nt(shape->dtype, kEpiStore, w + l.ybuf, w + l.wo, out, rows, D, D, D, D, D, st);
  phase_end(ph, st);
  if (e != hipSuccess) return hip_fail(e, "output gemm launch");
  return VDN_OK;
}

int vdn_set_param_check(int on) { return g_param_check.exchange(on ? 1 : 0); }

int vdn_timing_start(void) {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  g_timer.on = true;
  g_timer.failed = false;
  g_timer.recs.clear();
  g_timer.used = 0;
  return VDN_OK;
}

int vdn_timing_stop(vdn_phase_stat* stats, int max_stats) {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  g_timer.on = false;
  if (g_timer.failed) return fail(VDN_ERR_HIP, "vdn_timing_stop: could not create HIP events");
  int launches[kNumPhases] = {0};
  double total[kNumPhases] = {0.0};
  for (const Timer::Rec& r : g_timer.recs) {
    hipError_t e = hipEventSynchronize(r.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "vdn_timing_stop");
    launches[r.phase] += 1;
    total[r.phase] += ms;
  }
  g_timer.recs.clear();
  if (stats) {
    for (int i = 0; i < kNumPhases && i < max_stats; ++i) {
      stats[i].name = kPhaseNames[i];
      stats[i].launches = launches[i];
      stats[i].total_ms = (float)total[i];
    }
  }
  return kNumPhases;
}

}  // extern "C"
