// Linear branch of Video DeltaNet: Video Delta Attention (VDA), the
// frame-level delta rule (10100.com article on Video DeltaNet, 方法概述 part 2)
//   S_t = (gamma_t S_prev + B_t)(I + A_t)^-1,
//   A_t = beta_t K_t^T K_t,  B_t = beta_t V_t^T K_t,
// scanned forward and backward over frames (the article's forward-plus-
// backward scan figure), read out as RMSNorm(S_t q) per direction, summed and
// gated (方法概述 part 3).
//
// Four kernels, one HBM pass each over the large tensors:
//   gram    : per (frame, head) A_t and B_t from K_t, V_t     (MFMA, HBM-bound)
//   solve   : per (frame, head) M_t = (I + A_t)^-1 by a Cholesky factorisation
//             held in LDS, and C_t = B_t M_t                    (LDS, latency)
//   scan    : S_t = gamma_t S_prev M_t + C_t, both directions    (T-step chain)
//   readout : u = S_t q both directions, RMSNorm, sum, gate     (MFMA, HBM-bound)
#include <math.h>

#include "vdn_common.h"
#include "vdn_internal.h"

namespace vdn {

// ---------------------------------------------------------------------------
// gram: A = beta K^T K (symmetric, upper 16x16 tiles computed and mirrored),
// B = beta V^T K.  Token rows are staged transposed in LDS so both MFMA
// operands read contiguous token runs.
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_gram_kernel(const T* __restrict__ k,
                                                       const T* __restrict__ v,
                                                       const float* __restrict__ beta,
                                                       float* __restrict__ A,
                                                       float* __restrict__ Bm, int N) {
  using MM = Mma<T>;
  constexpr int KP = MM::kPack, KS = MM::kStep;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int NC = 32;                // tokens per LDS stage
  constexpr int LDT = NC + EPC;         // transposed row stride (elements)
  constexpr int CPR = D / EPC;          // 16-byte chunks per token row
  constexpr int NT = D / 16;
  constexpr int NA = NT * (NT + 1) / 2, NB = NT * NT, NTOT = NA + NB;
  constexpr int PER = (NTOT + 3) / 4;   // output tiles per wave
  __shared__ __attribute__((aligned(16))) T Sm[2 * D * LDT];   // [K^T | V^T]

  const int64_t f = blockIdx.x;
  const T* kf = k + f * N * D;
  const T* vf = v + f * N * D;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane % 16, lg = lane / 16;

  int aoff[PER], boff[PER], tinfo[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int tile = wave + 4 * u;
    int ti = 0, tj = 0, isA = 0;
    if (tile < NA) {
      int rem = tile;
      while (rem >= NT - ti) { rem -= NT - ti; ++ti; }
      tj = ti + rem;
      isA = 1;
    } else if (tile < NTOT) {
      ti = (tile - NA) / NT;
      tj = (tile - NA) % NT;
    }
    aoff[u] = (isA ? 0 : D * LDT) + (ti * 16 + li) * LDT;
    boff[u] = (tj * 16 + li) * LDT;
    tinfo[u] = (isA << 16) | (ti << 8) | tj;
  }

  f32x4 acc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int n0 = 0; n0 < N; n0 += NC) {
    __syncthreads();
    for (int c = tid; c < NC * CPR; c += 256) {
      const int row = c % NC, cc = c / NC;
      Chunk16 kk = zero_chunk(), vv = zero_chunk();
      if (n0 + row < N) {
        kk = *reinterpret_cast<const Chunk16*>(kf + (int64_t)(n0 + row) * D + cc * EPC);
        vv = *reinterpret_cast<const Chunk16*>(vf + (int64_t)(n0 + row) * D + cc * EPC);
      }
      const T* ke = reinterpret_cast<const T*>(&kk);
      const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
      for (int x = 0; x < EPC; ++x) {
        Sm[(cc * EPC + x) * LDT + row] = ke[x];
        Sm[D * LDT + (cc * EPC + x) * LDT + row] = ve[x];
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < NC / KS; ++ks)
#pragma unroll
      for (int u = 0; u < PER; ++u)
        if (wave + 4 * u < NTOT)
          acc[u] = MM::run(MM::load(Sm + aoff[u] + ks * KS + lg * KP),
                           MM::load(Sm + boff[u] + ks * KS + lg * KP), acc[u]);
  }

  const float bt = beta[f];
  float* Af = A + f * D * D;
  float* Bf = Bm + f * D * D;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if (wave + 4 * u >= NTOT) continue;
    const int isA = tinfo[u] >> 16, ti = (tinfo[u] >> 8) & 255, tj = tinfo[u] & 255;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = ti * 16 + lg * 4 + r, col = tj * 16 + li;
      const float val = bt * acc[u][r];
      if (isA) {
        Af[row * D + col] = val;
        if (ti != tj) Af[col * D + row] = val;
      } else {
        Bf[row * D + col] = val;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// solve: one workgroup per (frame, head).  I + A_t is symmetric positive
// definite (beta >= 0), so it is factored as L L^T in LDS by a right-looking
// Cholesky; W = L^-1 by column-parallel forward substitution; M = W^T W;
// C = B M.  AM holds A_t on entry and M_t on exit; BC holds B_t then C_t.
template <int D>
__global__ __launch_bounds__(256) void vda_solve_kernel(float* __restrict__ AM,
                                                        float* __restrict__ BC) {
  constexpr int LD = D + 1;
  __shared__ float Ls[D * LD];
  __shared__ float Ws[D * LD];
  __shared__ float dg[D];
  const int64_t f = blockIdx.x;
  float* a = AM + f * D * D;
  float* bm = BC + f * D * D;
  const int tid = threadIdx.x;

  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, j = e % D;
    Ls[i * LD + j] = a[e] + (i == j ? 1.f : 0.f);
  }
  __syncthreads();

  // Step k updates the trailing block with the still-unscaled column k
  // (a_ik a_jk / a_kk) and scales column k-1, which step k no longer reads,
  // so one barrier per step suffices.
  for (int kk = 0; kk < D; ++kk) {
    const float akk = Ls[kk * LD + kk];
    const float inv_akk = 1.f / akk;
    if (tid == 0) dg[kk] = akk;
    const int m = D - 1 - kk;
    for (int e = tid; e < m * m; e += 256) {
      const int ii = kk + 1 + e / m, jj = kk + 1 + e % m;
      if (jj <= ii) Ls[ii * LD + jj] -= Ls[ii * LD + kk] * Ls[jj * LD + kk] * inv_akk;
    }
    if (kk > 0) {
      const int c = kk - 1;
      const float sq = sqrtf(dg[c]);
      for (int i = c + tid; i < D; i += 256)
        Ls[i * LD + c] = (i == c) ? sq : Ls[i * LD + c] / sq;
    }
    __syncthreads();
  }
  if (tid == 0) Ls[(D - 1) * LD + (D - 1)] = sqrtf(dg[D - 1]);
  __syncthreads();

  // W = L^-1: thread j solves L w = e_j; W[i][j] = 0 for i < j falls out.
  if (tid < D) {
    const int j = tid;
    for (int i = 0; i < D; ++i) {
      float s = (i == j) ? 1.f : 0.f;
      for (int q = 0; q < i; ++q) s -= Ls[i * LD + q] * Ws[q * LD + j];
      Ws[i * LD + j] = s / Ls[i * LD + i];
    }
  }
  __syncthreads();

  // M = W^T W (symmetric) into Ls.
  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, j = e % D;
    if (j < i) continue;
    float s = 0.f;
    for (int q = i; q < D; ++q) s += Ws[q * LD + i] * Ws[q * LD + j];
    Ls[i * LD + j] = s;
    Ls[j * LD + i] = s;
  }
  __syncthreads();
  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, j = e % D;
    a[e] = Ls[i * LD + j];
    Ws[i * LD + j] = bm[e];
  }
  __syncthreads();
  // C = B M
  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, j = e % D;
    float s = 0.f;
    for (int q = 0; q < D; ++q) s += Ws[i * LD + q] * Ls[q * LD + j];
    bm[e] = s;
  }
}

// ---------------------------------------------------------------------------
// scan: S_t = gamma_t S_prev M_t + C_t.  Rows of S are independent given M_t,
// so each workgroup owns kScanRows rows of one (batch, head, direction) and
// walks the T frames, staging M_t in LDS.  Writes every S_t (fp32).
template <int D, int R>
__global__ __launch_bounds__(256) void vda_scan_kernel(const float* __restrict__ M,
                                                       const float* __restrict__ Cm,
                                                       const float* __restrict__ gamma,
                                                       float* __restrict__ states, int T,
                                                       int64_t bhtdd) {
  constexpr int TPR = 256 / R;     // threads per state row
  constexpr int CPT = D / TPR;     // columns per thread
  constexpr int LDM = D + 4;
  __shared__ __attribute__((aligned(16))) float Ms[D * LDM];
  __shared__ float Ss[R * LDM];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * R;
  const int64_t bh = blockIdx.y;
  const int dir = blockIdx.z;
  const int row = tid / TPR, col0 = (tid % TPR) * CPT;
  for (int i = tid; i < R * LDM; i += 256) Ss[i] = 0.f;

  for (int step = 0; step < T; ++step) {
    const int t = dir ? T - 1 - step : step;
    const int64_t fi = bh * T + t;
    const float* mt = M + fi * D * D;
    __syncthreads();
    for (int e = tid * 4; e < D * D; e += 1024) {
      const float4 x = *reinterpret_cast<const float4*>(mt + e);
      *reinterpret_cast<float4*>(Ms + (e / D) * LDM + (e % D)) = x;
    }
    __syncthreads();
    const float g = gamma[fi];
    float acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
    for (int q = 0; q < D; ++q) {
      const float sv = Ss[row * LDM + q];
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[c] += sv * Ms[q * LDM + col0 + c];
    }
    const float* crow = Cm + fi * D * D + (int64_t)(r0 + row) * D + col0;
    float* srow = states + dir * bhtdd + fi * D * D + (int64_t)(r0 + row) * D + col0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const float nv = g * acc[c] + crow[c];
      Ss[row * LDM + col0 + c] = nv;
      srow[c] = nv;
    }
  }
}

// ---------------------------------------------------------------------------
// readout: for a tile of tokens of one frame, u = S_t q for both directions
// (U = Q S^T on MFMA with S staged in LDS in the I/O precision), RMSNorm of
// each over head_dim, summed, times rms weight and gate.
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_readout_kernel(
    const T* __restrict__ q, const float* __restrict__ states, const float* __restrict__ rms_w,
    const T* __restrict__ gate, int64_t ldg, T* __restrict__ out, int64_t ldo, int H, int T_,
    int N, float eps, int tiles_per_frame, int64_t bhtdd) {
  using MM = Mma<T>;
  constexpr int KP = MM::kPack, KS = MM::kStep;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int LDSS = D + EPC;
  constexpr int CT = D / 16;
  constexpr int KSTEPS = D / KS;
  __shared__ __attribute__((aligned(16))) T Sf[D * LDSS];
  __shared__ __attribute__((aligned(16))) T Sb[D * LDSS];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane % 16, lg = lane / 16;
  const int tile = blockIdx.x % tiles_per_frame;
  const int64_t fi = blockIdx.x / tiles_per_frame;     // (b*H + h)*T + t
  const int t = (int)(fi % T_);
  const int64_t bh = fi / T_;
  const int h = (int)(bh % H);
  const int64_t b = bh / H;
  const float* sf = states + fi * D * D;
  const float* sb = states + bhtdd + fi * D * D;
  for (int e = tid * 4; e < D * D; e += 1024) {
    const float4 x = *reinterpret_cast<const float4*>(sf + e);
    const float4 y = *reinterpret_cast<const float4*>(sb + e);
    T* pf = Sf + (e / D) * LDSS + (e % D);
    T* pb = Sb + (e / D) * LDSS + (e % D);
    pf[0] = from_f32<T>(x.x); pf[1] = from_f32<T>(x.y); pf[2] = from_f32<T>(x.z); pf[3] = from_f32<T>(x.w);
    pb[0] = from_f32<T>(y.x); pb[1] = from_f32<T>(y.y); pb[2] = from_f32<T>(y.z); pb[3] = from_f32<T>(y.w);
  }
  __syncthreads();

  const int n0 = tile * kReadoutBT + wave * 16;
  const int n = n0 + li;
  const T* qrow = q + (fi * N + n) * D;
  typename MM::Frag qa[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    qa[ks] = (n < N) ? MM::load(qrow + ks * KS + lg * KP) : MM::zero();

  f32x4 uf[CT], ub[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    uf[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    ub[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uf[ct] = MM::run(qa[ks], MM::load(Sf + (ct * 16 + li) * LDSS + ks * KS + lg * KP), uf[ct]);
      ub[ct] = MM::run(qa[ks], MM::load(Sb + (ct * 16 + li) * LDSS + ks * KS + lg * KP), ub[ct]);
    }
  }
  // uf[ct][r] = u_fwd(token n0 + lg*4 + r)[ct*16 + li]
  float rf[4], rb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float sf2 = 0.f, sb2 = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      sf2 += uf[ct][r] * uf[ct][r];
      sb2 += ub[ct][r] * ub[ct][r];
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      sf2 += __shfl_xor(sf2, m);
      sb2 += __shfl_xor(sb2, m);
    }
    rf[r] = 1.f / sqrtf(sf2 / D + eps);
    rb[r] = 1.f / sqrtf(sb2 / D + eps);
  }
  const int64_t NL = (int64_t)T_ * N;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int nn = n0 + lg * 4 + r;
    if (nn >= N) continue;
    const int64_t orow = b * NL + (int64_t)t * N + nn;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int i = ct * 16 + li;
      const float w = rms_w ? rms_w[h * D + i] : 1.f;
      float val = (uf[ct][r] * rf[r] + ub[ct][r] * rb[r]) * w;
      if (gate) val *= to_f32(gate[orow * ldg + h * D + i]);
      out[orow * ldo + h * D + i] = from_f32<T>(val);
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T>
static hipError_t gram_t(int d, const void* k, const void* v, const float* beta, float* A,
                         float* Bm, int nframes, int N, hipStream_t st) {
  if (d == 32)
    vda_gram_kernel<T, 32><<<nframes, 256, 0, st>>>((const T*)k, (const T*)v, beta, A, Bm, N);
  else if (d == 64)
    vda_gram_kernel<T, 64><<<nframes, 256, 0, st>>>((const T*)k, (const T*)v, beta, A, Bm, N);
  else
    vda_gram_kernel<T, 128><<<nframes, 256, 0, st>>>((const T*)k, (const T*)v, beta, A, Bm, N);
  return hipGetLastError();
}

hipError_t launch_vda_gram(int dtype, int d, const void* k, const void* v, const float* beta,
                           float* A, float* Bm, int nframes, int N, hipStream_t st) {
  if (nframes == 0) return hipSuccess;
  return dtype == 1 ? gram_t<bf16>(d, k, v, beta, A, Bm, nframes, N, st)
                    : gram_t<float>(d, k, v, beta, A, Bm, nframes, N, st);
}

hipError_t launch_vda_solve(int d, float* AM, float* BC, int nframes, hipStream_t st) {
  if (nframes == 0) return hipSuccess;
  if (d == 32) vda_solve_kernel<32><<<nframes, 256, 0, st>>>(AM, BC);
  else if (d == 64) vda_solve_kernel<64><<<nframes, 256, 0, st>>>(AM, BC);
  else vda_solve_kernel<128><<<nframes, 256, 0, st>>>(AM, BC);
  return hipGetLastError();
}

hipError_t launch_vda_scan(int d, const float* M, const float* Cm, const float* gamma,
                           float* states, int BH, int T, hipStream_t st) {
  if (BH == 0) return hipSuccess;
  const int64_t bhtdd = (int64_t)BH * T * d * d;
  dim3 grid(d / kScanRows, BH, 2);
  if (d == 32) vda_scan_kernel<32, kScanRows><<<grid, 256, 0, st>>>(M, Cm, gamma, states, T, bhtdd);
  else if (d == 64) vda_scan_kernel<64, kScanRows><<<grid, 256, 0, st>>>(M, Cm, gamma, states, T, bhtdd);
  else vda_scan_kernel<128, kScanRows><<<grid, 256, 0, st>>>(M, Cm, gamma, states, T, bhtdd);
  return hipGetLastError();
}

template <typename T>
static hipError_t readout_t(int d, const void* q, const float* states, const float* rms_w,
                            const void* gate, int64_t ldg, void* out, int64_t ldo, int B, int H,
                            int T_, int N, float eps, hipStream_t st) {
  const int tpf = (N + kReadoutBT - 1) / kReadoutBT;
  const int64_t blocks = (int64_t)B * H * T_ * tpf;
  const int64_t bhtdd = (int64_t)B * H * T_ * d * d;
  if (blocks == 0) return hipSuccess;
#define VDN_READOUT(DD)                                                                   \
  vda_readout_kernel<T, DD><<<(unsigned)blocks, 256, 0, st>>>(                            \
      (const T*)q, states, rms_w, (const T*)gate, ldg, (T*)out, ldo, H, T_, N, eps, tpf, \
      bhtdd)
  if (d == 32) VDN_READOUT(32);
  else if (d == 64) VDN_READOUT(64);
  else VDN_READOUT(128);
#undef VDN_READOUT
  return hipGetLastError();
}

hipError_t launch_vda_readout(int dtype, int d, const void* q, const float* states,
                              const float* rms_w, const void* gate, int64_t ldg, void* out,
                              int64_t ldo, int B, int H, int T, int N, float eps,
                              hipStream_t st) {
  return dtype == 1 ? readout_t<bf16>(d, q, states, rms_w, gate, ldg, out, ldo, B, H, T, N, eps, st)
                    : readout_t<float>(d, q, states, rms_w, gate, ldg, out, ldo, B, H, T, N, eps, st);
}

}  // namespace vdn
