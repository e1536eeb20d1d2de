// Internal interface of the VDA-branch gradient kernels (vda_bwd.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdn {

// Batched product C[z] = alpha * alpha_z[z] * A[z] B[z] (+ C[z] if accumulate),
// fp32 accumulation.  Element (m, k) of A[z] is a_s[off_a(z) + m*sam + k'*sak]
// where k' = k and a_s = a0 for k < ks, k' = k - ks and a_s = a1 otherwise
// (a1 NULL: a0); B likewise with (k, n) -> k'*sbk + n*sbn; C[z](m, n) is
// c[off_c(z) + m*ldc + n].  Batch index z splits as z0 = z % n0,
// z1 = (z / n0) % n1, z2 = z / (n0 n1) and off_x(z) = z0 sx[0] + z1 sx[1] + z2 sx[2]
// (in elements).  alpha_z may be NULL.
struct BGemm {
  const void* a0 = nullptr;
  const void* a1 = nullptr;
  const void* b0 = nullptr;
  const void* b1 = nullptr;
  void* c = nullptr;
  int M = 0, N = 0, K = 0, ks = 0;
  int64_t sam = 0, sak = 0, sbk = 0, sbn = 0, ldc = 0;
  int64_t batch = 0;
  int n0 = 1, n1 = 1;
  int64_t sa[3] = {0, 0, 0}, sb[3] = {0, 0, 0}, sc[3] = {0, 0, 0};
  float alpha = 1.f;
  const float* alpha_z = nullptr;
  int accumulate = 0;
  int a_kfast = 0, b_nfast = 0;   // set by launch_bgemm
  int vec = 0;                    // set by launch_bgemm: 16-byte vector loads allowed
};

// ta, tb, tc: 0 = fp32, 1 = bf16 element type of A, B, C.  mfma: run on bf16
// MFMA with fp32 operands split into hi + lo bf16 (one operand must be bf16 or
// C bf16); otherwise fp32 FMA.
hipError_t launch_bgemm(int ta, int tb, int tc, BGemm p, hipStream_t st, bool mfma = false);
hipError_t launch_fill(float* x, float v, int64_t n, hipStream_t st);
// am = beta_f kk, bm = beta_f vk over nf frames of dd elements
hipError_t launch_scale_frames(const float* kk, const float* vk, const float* beta, float* am,
                               float* bm, int64_t nf, int64_t dd, hipStream_t st);
// U [nf][2][N][d]: u in, du out; d_out rows b*Lt + t*N + n, columns h*d + i, stride ldo;
// dw_part [nf][2][d]
hipError_t launch_rms_bwd(int dtype, int d, float* U, const void* d_out, int64_t ldo,
                          const float* rms_w, float* dw_part, int64_t nf, int H, int T, int N, int Lt,
                          float eps, hipStream_t st);
// dsg [nf][2][d][d]: dS in, G out; dx [nf][2][d][d]; Mt [nf][d][d] = M^T
hipError_t launch_scan_bwd(int d, const float* Mt, const float* gamma, float* dsg, float* dx, int BH,
                           int T, hipStream_t st);
// states [2][nf][d][d], bm [nf][d][d]; xs, cdb [nf][2][d][d] (cdb[f][1] = dB); dgamma [nf]
hipError_t launch_frame_bwd(const float* states, const float* bm, const float* gamma, const float* dx,
                            float* xs, float* cdb, float* dgamma, int T, int64_t nf, int d,
                            hipStream_t st);
// cdb[f][0] = dA + dA^T; dbeta[f] = <dA, kk> + <cdb[f][1], vk>
hipError_t launch_sym_dbeta(int d, const float* dA, const float* kk, const float* vk, float* cdb,
                            float* dbeta, int64_t nf, hipStream_t st);
// bf16 tokens, head_dim 128: dK = beta (K cdb[f][0] + V cdb[f][1]), dV = beta K cdb[f][1]^T per frame
hipError_t launch_kv_grad(const void* k, const void* v, const float* cdb, const float* beta, void* dk, void* dv,
                          int64_t nf, int T, int N, int Lt, hipStream_t st);
// bf16 tokens, head_dim 128: the readout adjoint of both directions (u, du, RMSNorm weight partials
// dwp [nf][2][d]), dq (via the fp32 partial dqp [nf][N][d]) and dS into dsg [nf][2][d][d]
hipError_t launch_tok_grad(const void* q, const void* d_out, int64_t ldo, const float* states, const float* rms_w,
                           float* dqp, void* dq, float* dsg, float* dwp, int64_t nf, int H, int T, int N, int Lt,
                           float eps, hipStream_t st);
hipError_t launch_dw_reduce(const float* part, float* drms_w, int B, int H, int T, int d,
                            hipStream_t st);

}  // namespace vdn
