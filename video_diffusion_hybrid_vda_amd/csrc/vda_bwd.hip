// Gradient of the VDA linear branch (10100.com article on Video DeltaNet,
// 方法概述 part 2: the frame-level delta rule; part 3: RMSNorm per direction
// and the staged adaptation that trains this branch).  The pages give the
// forward rule only; the kernels below evaluate its derivative, step by step
// in reverse:
//   readout  u = S_t q, r = u / rho, o = w (r_f + r_b):
//            du = (w do - r mean(w do r)) / rho,  dq = S_f^T du_f + S_b^T du_b,
//            dS_t = sum over the frame's tokens of du q^T,  dw = sum (r_f + r_b) do
//   scan     S_t = X_t M_t, X_t = gamma_t S_prev + B_t:  G_t = dS_t + gamma_next dX_next,
//            dX_t = G_t M_t^T,  dM_t = sum_dir X_t^T G_t,  dB_t = sum_dir dX_t,
//            dgamma_t = sum_dir <dX_t, S_prev>
//   solve    M_t = (I + A_t)^-1:  dA_t = -M_t^T dM_t M_t^T
//   Gram     dK_t = beta_t (K_t (dA_t + dA_t^T) + V_t dB_t),  dV_t = beta_t K_t dB_t^T,
//            dbeta_t = <dA_t, K_t^T K_t> + <dB_t, V_t^T K_t>
//
// Kernels:
//   bgemm        batched fp32-accumulate product with strided, two-segment
//                operands: every contraction above (token-side products and the
//                per-frame d x d products); fp32 FMA, or fp32 MFMA when both
//                operands and the result are fp32
//   bgemm_mfma   the same on bf16 MFMA with fp32 operands split into hi + lo
//                bf16: the token-side products of bf16 I/O
//   rms_bwd      per token and direction: du from u (in place) and partial dw
//   scan_bwd     per (batch, head, direction, 16 state rows): the T-step adjoint chain
//   frame_bwd    per frame: X_t of both directions, dB_t and dgamma_t
//   sym_dbeta    per frame: dA_t + dA_t^T next to dB_t, and dbeta_t
//   dw_reduce    sum of the partial RMSNorm-weight gradients
#include <math.h>

#include <type_traits>

#include "vda_bwd.h"
#include "vdn_common.h"

namespace vdn {

// ---------------------------------------------------------------------------
// bgemm: C[z] = alpha * alpha_z[z] * sum_k A[z](m, k) B[z](k, n)  (+ C[z] if accumulate)
// 64 x 64 output tile per workgroup of 256 threads (4 x 4 outputs per thread,
// spread 16 apart so that LDS reads are conflict-free and each row of the
// store is 16 consecutive elements), 16-deep k slabs staged through LDS in
// fp32, the next slab loaded into registers while the current one is used.
// Operand elements are fetched along the operand's unit-stride axis.
namespace bg {
constexpr int BM = 64, BN = 64, BK = 16, LDT = 64 + 4;
typedef float f32x16 __attribute__((ext_vector_type(16)));
}

__device__ __forceinline__ void batch_index(const BGemm& p, int64_t z, int64_t& z0, int64_t& z1,
                                            int64_t& z2) {
  z0 = z % p.n0;
  z1 = (z / p.n0) % p.n1;
  z2 = z / ((int64_t)p.n0 * p.n1);
}

template <typename TA, typename TB, typename TC, bool MF>
__global__ __launch_bounds__(256) void bgemm_kernel(BGemm p) {
  using namespace bg;
  static_assert(!MF || (std::is_same<TA, float>::value && std::is_same<TB, float>::value), "fp32 MFMA takes fp32");
  // fp32 MFMA reads k and k + 1 of one column in the two lane halves: rows 32 banks apart
  constexpr int LD = MF ? 64 + 32 : LDT;
  constexpr int KB = BK;                         // k slab (32 deep measured slower on the matrix unit)
  constexpr int PER = BM * KB / 256;             // slab elements per thread and operand
  __shared__ float As[KB][LD];
  __shared__ float Bs[KB][LD];
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles = ((p.M + BM - 1) / BM) * tiles_n;
  const int64_t z = blockIdx.x / tiles;
  const int tile = blockIdx.x % tiles;
  const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
  int64_t z0, z1, z2;
  batch_index(p, z, z0, z1, z2);
  const int64_t oa = z0 * p.sa[0] + z1 * p.sa[1] + z2 * p.sa[2];
  const int64_t ob = z0 * p.sb[0] + z1 * p.sb[1] + z2 * p.sb[2];
  const int64_t oc = z0 * p.sc[0] + z1 * p.sc[1] + z2 * p.sc[2];
  const TA* a0 = (const TA*)p.a0 + oa;
  const TA* a1 = (const TA*)(p.a1 ? p.a1 : p.a0) + oa;
  const TB* b0 = (const TB*)p.b0 + ob;
  const TB* b1 = (const TB*)(p.b1 ? p.b1 : p.b0) + ob;
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;

  // element r of this thread's share of a slab: (row of the tile, k in the slab)
  auto a_pos = [&](int r, int& mm, int& kk) {
    const int e = tid + 256 * r;
    if (p.a_kfast) { kk = e % KB; mm = e / KB; } else { mm = e % BM; kk = e / BM; }
  };
  auto b_pos = [&](int r, int& nn, int& kk) {
    const int e = tid + 256 * r;
    if (p.b_nfast) { nn = e % BN; kk = e / BN; } else { kk = e % KB; nn = e / KB; }
  };
  float ra[PER], rb[PER];
  auto load = [&](int k0) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      int mm, kk;
      a_pos(r, mm, kk);
      const int m = m0 + mm, k = k0 + kk;
      float x = 0.f;
      if (m < p.M && k < p.K) {
        const bool s1 = k >= p.ks;
        x = to_f32((s1 ? a1 : a0)[m * p.sam + (s1 ? k - p.ks : k) * p.sak]);
      }
      ra[r] = x;
      int nn;
      b_pos(r, nn, kk);
      const int n = n0 + nn, kb = k0 + kk;
      float y = 0.f;
      if (n < p.N && kb < p.K) {
        const bool s1 = kb >= p.ks;
        y = to_f32((s1 ? b1 : b0)[(s1 ? kb - p.ks : kb) * p.sbk + n * p.sbn]);
      }
      rb[r] = y;
    }
  };

  // FMA path: 4 x 4 outputs per thread.  MFMA path: wave w forms the 32 x 32
  // block (32 (w / 2), 32 (w % 2)) with v_mfma_f32_32x32x2_f32 (lane l: row or
  // column l % 32, k = l / 32 of each pair)
  float acc[4][4];
  f32x16 accm = {};
  const int wave = tid / kWave, lane = tid % kWave, l32 = lane % 32, h = lane / 32;
  const int wm = 32 * (wave / 2), wn = 32 * (wave % 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  load(0);
  for (int k0 = 0; k0 < p.K; k0 += KB) {
    __syncthreads();   // the previous slab has been read
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      int mm, kk;
      a_pos(r, mm, kk);
      As[kk][mm] = ra[r];
      int nn;
      b_pos(r, nn, kk);
      Bs[kk][nn] = rb[r];
    }
    __syncthreads();
    if (k0 + KB < p.K) load(k0 + KB);
    if constexpr (MF) {
#pragma unroll
      for (int s2 = 0; s2 < KB / 2; ++s2)
        accm = __builtin_amdgcn_mfma_f32_32x32x2f32(As[2 * s2 + h][wm + l32], Bs[2 * s2 + h][wn + l32], accm, 0, 0, 0);
    } else {
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        float av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = As[kk][ty + 16 * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx + 16 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
      }
    }
  }

  const float alpha = p.alpha * (p.alpha_z ? p.alpha_z[z] : 1.f);
  TC* c = (TC*)p.c + oc;
  auto put = [&](int m, int n, float v) {
    if (m >= p.M || n >= p.N) return;
    const int64_t idx = m * p.ldc + n;
    float val = alpha * v;
    if (p.accumulate) val += to_f32(c[idx]);
    c[idx] = from_f32<TC>(val);
  };
  if constexpr (MF) {
    // accm[r] = block element (row 8 (r / 4) + 4 h + r % 4, column l32)
#pragma unroll
    for (int r = 0; r < 16; ++r) put(m0 + wm + 8 * (r / 4) + 4 * h + r % 4, n0 + wn + l32, accm[r]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) put(m0 + ty + 16 * i, n0 + tx + 16 * j, acc[i][j]);
  }
}

// ---------------------------------------------------------------------------
// bgemm_mfma: the same product on bf16 MFMA (v_mfma_f32_16x16x32_bf16) for the
// token-side contractions of bf16 I/O.  An fp32 operand enters as the
// unevaluated pair hi + lo of bf16 values (hi = bf16(x), lo = bf16(x - hi),
// ~16 significant bits); a bf16 operand is exact.  Each product sums
// hi*hi, and hi*lo / lo*hi for each split operand (lo*lo, ~2^-16 relative, is
// dropped).  64 x BN output tile per workgroup (BN = 128 when the output is
// that wide, so that each token row is read once), four waves of 32 x BN/2,
// 64-deep k slabs staged in LDS as [row][k] bf16 (k contiguous,
// rows padded to 144 bytes) so that each lane's 8-element fragment is one
// 16-byte read; the next slab is loaded into registers while the current one
// is multiplied.
namespace bm {
constexpr int BM = 64, BK = 64, LDK = BK + 8;   // output tile BM x BN, BN = 64 or 128
}

template <typename TA, typename TB, typename TC, int BN>
__global__ __launch_bounds__(256) void bgemm_mfma_kernel(BGemm p) {
  using bm::BM;
  using bm::BK;
  using bm::LDK;
  constexpr int JT = BN / 32;   // 16-column MFMA tiles per wave (a wave covers BN / 2 columns)
  constexpr int RB = BN / 64;   // 16-element runs of the B slab per thread
  constexpr bool SA = sizeof(TA) == 4, SB = sizeof(TB) == 4;   // fp32 operands are split
  // operand slabs; after the last slab the same bytes hold the fp32 output tile
  constexpr int kOpBytes = (BM * LDK + BN * LDK + (SA ? BM * LDK : 0) + (SB ? BN * LDK : 0)) * 2;
  constexpr int LDC = BN + 4;
  constexpr int kCBytes = BM * LDC * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kOpBytes > kCBytes ? kOpBytes : kCBytes];
  bf16* Ah = reinterpret_cast<bf16*>(smem);
  bf16* Bh = Ah + BM * LDK;
  bf16* Al = Bh + BN * LDK;
  bf16* Bl = Al + (SA ? BM * LDK : 0);
  float* Cs = reinterpret_cast<float*>(smem);
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles = ((p.M + BM - 1) / BM) * tiles_n;
  const int64_t z = blockIdx.x / tiles;
  const int tile = blockIdx.x % tiles;
  const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
  int64_t z0, z1, z2;
  batch_index(p, z, z0, z1, z2);
  const int64_t oa = z0 * p.sa[0] + z1 * p.sa[1] + z2 * p.sa[2];
  const int64_t ob = z0 * p.sb[0] + z1 * p.sb[1] + z2 * p.sb[2];
  const int64_t oc = z0 * p.sc[0] + z1 * p.sc[1] + z2 * p.sc[2];
  const TA* a0 = (const TA*)p.a0 + oa;
  const TA* a1 = (const TA*)(p.a1 ? p.a1 : p.a0) + oa;
  const TB* b0 = (const TB*)p.b0 + ob;
  const TB* b1 = (const TB*)(p.b1 ? p.b1 : p.b0) + ob;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  // element j < 16 of this thread's share of a slab: 16 consecutive elements
  // along the operand's unit-stride axis
  auto a_pos = [&](int j, int& mm, int& kk) {
    if (p.a_kfast) { mm = tid / 4; kk = (tid % 4) * 16 + j; } else { kk = tid / 4; mm = (tid % 4) * 16 + j; }
  };
  // run u of the B slab: along n (BN / 16 runs per k) or along k (4 runs per n)
  auto b_run = [&](int u, int& nn, int& kk) {
    if (p.b_nfast) { kk = u / (BN / 16); nn = (u % (BN / 16)) * 16; } else { nn = u / 4; kk = (u % 4) * 16; }
  };
  float ra[16], rb[RB][16];
  // 16 consecutive elements from p[0..15] (16-byte aligned; checked on the host)
  auto vload = [](const auto* ptr, float (&r)[16]) {
    if constexpr (sizeof(*ptr) == 4) {
      const float4* v = reinterpret_cast<const float4*>(ptr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = v[i];
        r[4 * i] = x.x; r[4 * i + 1] = x.y; r[4 * i + 2] = x.z; r[4 * i + 3] = x.w;
      }
    } else {
      const bf16x8* v = reinterpret_cast<const bf16x8*>(ptr);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bf16x8 x = v[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) r[8 * i + e] = (float)x[e];
      }
    }
  };
  auto load = [&](int k0) {
    // A: the thread's run is along k (a_kfast) or along m
    {
      const int mm = p.a_kfast ? tid / 4 : (tid % 4) * 16;
      const int kk = p.a_kfast ? (tid % 4) * 16 : tid / 4;
      const int m = m0 + mm, k = k0 + kk;
      const bool s1 = k >= p.ks;
      const int kl = s1 ? k - p.ks : k;
      const bool whole = p.vec && (p.a_kfast ? (m < p.M && k + 16 <= p.K && (s1 || k + 16 <= p.ks))
                                             : (k < p.K && m + 16 <= p.M));
      if (whole) {
        vload((s1 ? a1 : a0) + m * p.sam + kl * p.sak, ra);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          int jm, jk;
          a_pos(j, jm, jk);
          const int mj = m0 + jm, kj = k0 + jk;
          float x = 0.f;
          if (mj < p.M && kj < p.K) {
            const bool t1 = kj >= p.ks;
            x = to_f32((t1 ? a1 : a0)[mj * p.sam + (t1 ? kj - p.ks : kj) * p.sak]);
          }
          ra[j] = x;
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      int nn, kk;
      b_run(tid + 256 * rr, nn, kk);
      const int n = n0 + nn, k = k0 + kk;
      const bool s1 = k >= p.ks;
      const int kl = s1 ? k - p.ks : k;
      const bool whole = p.vec && (p.b_nfast ? (k < p.K && n + 16 <= p.N)
                                             : (n < p.N && k + 16 <= p.K && (s1 || k + 16 <= p.ks)));
      if (whole) {
        vload((s1 ? b1 : b0) + kl * p.sbk + n * p.sbn, rb[rr]);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int nj = n + (p.b_nfast ? j : 0), kj = k + (p.b_nfast ? 0 : j);
          float y = 0.f;
          if (nj < p.N && kj < p.K) {
            const bool t1 = kj >= p.ks;
            y = to_f32((t1 ? b1 : b0)[(t1 ? kj - p.ks : kj) * p.sbk + nj * p.sbn]);
          }
          rb[rr][j] = y;
        }
      }
    }
  };

  f32x4 acc[2][JT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < JT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load(0);
  for (int k0 = 0; k0 < p.K; k0 += BK) {
    __syncthreads();   // the previous slab has been read
    // runs along k go to LDS as two 16-byte stores, runs along m / n element by element
    auto put = [&](const float (&r)[16], bool kfast, int row, int kk, bf16* hi, bf16* lo, auto split) {
      if (kfast) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 vh, vl;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            vh[e] = (bf16)r[8 * h + e];
            if constexpr (decltype(split)::value) vl[e] = (bf16)(r[8 * h + e] - (float)vh[e]);
          }
          *reinterpret_cast<bf16x8*>(&hi[row * LDK + kk + 8 * h]) = vh;
          if constexpr (decltype(split)::value) *reinterpret_cast<bf16x8*>(&lo[row * LDK + kk + 8 * h]) = vl;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const bf16 h = (bf16)r[j];
          hi[(row + j) * LDK + kk] = h;
          if constexpr (decltype(split)::value) lo[(row + j) * LDK + kk] = (bf16)(r[j] - (float)h);
        }
      }
    };
    put(ra, p.a_kfast, p.a_kfast ? tid / 4 : (tid % 4) * 16, p.a_kfast ? (tid % 4) * 16 : tid / 4, Ah, Al,
        std::integral_constant<bool, SA>());
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      int nn, kk;
      b_run(tid + 256 * rr, nn, kk);
      put(rb[rr], !p.b_nfast, nn, kk, Bh, Bl, std::integral_constant<bool, SB>());
    }
    __syncthreads();
    if (k0 + BK < p.K) load(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int kof = ks * 32 + (lane / 16) * 8;
      bf16x8 ah[2], al[2], bh[JT], bl[JT];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 32 + i * 16 + lane % 16;
        ah[i] = *reinterpret_cast<const bf16x8*>(&Ah[row * LDK + kof]);
        if constexpr (SA) al[i] = *reinterpret_cast<const bf16x8*>(&Al[row * LDK + kof]);
      }
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const int col = wn * (BN / 2) + j * 16 + lane % 16;
        bh[j] = *reinterpret_cast<const bf16x8*>(&Bh[col * LDK + kof]);
        if constexpr (SB) bl[j] = *reinterpret_cast<const bf16x8*>(&Bl[col * LDK + kof]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
          if constexpr (SB) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
          if constexpr (SA) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
        }
    }
  }

  // acc[i][j][r] = C[wm*32 + i*16 + (lane/16)*4 + r][wn*BN/2 + j*16 + lane%16]: through
  // LDS, then each thread writes 16-byte row chunks
  const float alpha = p.alpha * (p.alpha_z ? p.alpha_z[z] : 1.f);
  __syncthreads();   // every wave is done with the operand slabs
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < JT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Cs[(wm * 32 + i * 16 + (lane / 16) * 4 + r) * LDC + wn * (BN / 2) + j * 16 + lane % 16] =
            alpha * acc[i][j][r];
  __syncthreads();
  TC* c = (TC*)p.c + oc;
  constexpr int CH = 16 / sizeof(TC);   // elements per 16-byte chunk
  for (int u = tid; u < BM * (BN / CH); u += 256) {
    const int mm = u / (BN / CH), nn = (u % (BN / CH)) * CH;
    const int m = m0 + mm, n = n0 + nn;
    if (m >= p.M) continue;
    const float* cs = Cs + mm * LDC + nn;
    TC* dst = c + m * p.ldc + n;
    if (p.vec && n + CH <= p.N) {
      float v[CH];
#pragma unroll
      for (int e = 0; e < CH; ++e) v[e] = cs[e];
      if constexpr (sizeof(TC) == 4) {
        float4 o = make_float4(v[0], v[1], v[2], v[3]);
        if (p.accumulate) {
          const float4 x = *reinterpret_cast<const float4*>(dst);
          o.x += x.x; o.y += x.y; o.z += x.z; o.w += x.w;
        }
        *reinterpret_cast<float4*>(dst) = o;
      } else {
        bf16x8 o;
        const bf16x8 x = p.accumulate ? *reinterpret_cast<const bf16x8*>(dst) : bf16x8{};
#pragma unroll
        for (int e = 0; e < CH; ++e) o[e] = (bf16)(v[e] + (p.accumulate ? (float)x[e] : 0.f));
        *reinterpret_cast<bf16x8*>(dst) = o;
      }
    } else {
      for (int e = 0; e < CH && n + e < p.N; ++e) {
        float val = cs[e];
        if (p.accumulate) val += to_f32(dst[e]);
        dst[e] = from_f32<TC>(val);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bgemm_mfma_resident: the bf16-MFMA product for outputs 128 columns wide with
// K = KK (128 or 256): the whole K x 128 B operand (a frame's d x d matrices)
// is staged into LDS once, as hi/lo bf16 pairs, and `tiles_per_wg` consecutive
// 64-row tiles of A stream through it, 64-deep k slabs at a time.  Staging B
// once per tile is what bounds the tiled kernel above.
namespace br {
constexpr int BM = 64, BN = 128, BK = 64, LDK = BK + 8;
}

template <typename TA, typename TB, typename TC, int KK>
__global__ __launch_bounds__(256) void bgemm_mfma_resident_kernel(BGemm p, int tiles_per_wg) {
  using namespace br;
  constexpr bool SA = sizeof(TA) == 4, SB = sizeof(TB) == 4;
  constexpr int LDB = KK + 8;   // B row pitch in LDS (bf16): 16-byte multiple
  __shared__ __attribute__((aligned(16))) bf16 Bh[BN * LDB];
  __shared__ __attribute__((aligned(16))) bf16 Bl[SB ? BN * LDB : 8];
  __shared__ __attribute__((aligned(16))) bf16 Ah[BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Al[SA ? BM * LDK : 8];
  const int tiles_m = (p.M + BM - 1) / BM;
  const int chunks = (tiles_m + tiles_per_wg - 1) / tiles_per_wg;
  const int64_t z = blockIdx.x / chunks;
  const int tm0 = (int)(blockIdx.x % chunks) * tiles_per_wg;
  int64_t z0, z1, z2;
  batch_index(p, z, z0, z1, z2);
  const int64_t oa = z0 * p.sa[0] + z1 * p.sa[1] + z2 * p.sa[2];
  const int64_t ob = z0 * p.sb[0] + z1 * p.sb[1] + z2 * p.sb[2];
  const int64_t oc = z0 * p.sc[0] + z1 * p.sc[1] + z2 * p.sc[2];
  const TA* a0 = (const TA*)p.a0 + oa;
  const TA* a1 = (const TA*)(p.a1 ? p.a1 : p.a0) + oa;
  const TB* b0 = (const TB*)p.b0 + ob;
  const TB* b1 = (const TB*)(p.b1 ? p.b1 : p.b0) + ob;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  auto vload = [](const auto* ptr, float (&r)[16]) {
    if constexpr (sizeof(*ptr) == 4) {
      const float4* v = reinterpret_cast<const float4*>(ptr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = v[i];
        r[4 * i] = x.x; r[4 * i + 1] = x.y; r[4 * i + 2] = x.z; r[4 * i + 3] = x.w;
      }
    } else {
      const bf16x8* v = reinterpret_cast<const bf16x8*>(ptr);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bf16x8 x = v[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) r[8 * i + e] = (float)x[e];
      }
    }
  };
  // runs along k go to LDS as two 16-byte stores, runs along m / n element by element
  auto put = [](const float (&r)[16], bool kfast, int row, int kk, int pitch, bf16* hi, bf16* lo, auto split) {
    if (kfast) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 vh, vl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vh[e] = (bf16)r[8 * h + e];
          if constexpr (decltype(split)::value) vl[e] = (bf16)(r[8 * h + e] - (float)vh[e]);
        }
        *reinterpret_cast<bf16x8*>(&hi[row * pitch + kk + 8 * h]) = vh;
        if constexpr (decltype(split)::value) *reinterpret_cast<bf16x8*>(&lo[row * pitch + kk + 8 * h]) = vl;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bf16 h = (bf16)r[j];
        hi[(row + j) * pitch + kk] = h;
        if constexpr (decltype(split)::value) lo[(row + j) * pitch + kk] = (bf16)(r[j] - (float)h);
      }
    }
  };

  // the whole B operand: KK x 128 in runs of 16 along its unit-stride axis
  for (int u = tid; u < KK * BN / 16; u += 256) {
    int nn, kk;
    if (p.b_nfast) { kk = u / (BN / 16); nn = (u % (BN / 16)) * 16; } else { nn = u / (KK / 16); kk = (u % (KK / 16)) * 16; }
    const bool s1 = kk >= p.ks;
    const int kl = s1 ? kk - p.ks : kk;
    float rb[16];
    const bool whole = p.vec && (p.b_nfast ? (nn + 16 <= p.N) : (nn < p.N && (s1 || kk + 16 <= p.ks)));
    if (whole) {
      vload((s1 ? b1 : b0) + kl * p.sbk + nn * p.sbn, rb);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int nj = nn + (p.b_nfast ? j : 0), kj = kk + (p.b_nfast ? 0 : j);
        float y = 0.f;
        if (nj < p.N && kj < p.K) {
          const bool t1 = kj >= p.ks;
          y = to_f32((t1 ? b1 : b0)[(t1 ? kj - p.ks : kj) * p.sbk + nj * p.sbn]);
        }
        rb[j] = y;
      }
    }
    put(rb, !p.b_nfast, nn, kk, LDB, Bh, Bl, std::integral_constant<bool, SB>());
  }

  const float alpha = p.alpha * (p.alpha_z ? p.alpha_z[z] : 1.f);
  TC* c = (TC*)p.c + oc;
  const int amm = p.a_kfast ? tid / 4 : (tid % 4) * 16;   // this thread's A run in a slab
  const int akk = p.a_kfast ? (tid % 4) * 16 : tid / 4;
  float ra[16];
  for (int ti = 0; ti < tiles_per_wg; ++ti) {
    const int tm = tm0 + ti;
    if (tm >= tiles_m) break;
    const int m0 = tm * BM;
    auto load = [&](int k0) {
      const int m = m0 + amm, k = k0 + akk;
      const bool s1 = k >= p.ks;
      const int kl = s1 ? k - p.ks : k;
      const bool whole = p.vec && (p.a_kfast ? (m < p.M && (s1 || k + 16 <= p.ks)) : (m + 16 <= p.M));
      if (whole) {
        vload((s1 ? a1 : a0) + m * p.sam + kl * p.sak, ra);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int mj = m + (p.a_kfast ? 0 : j), kj = k + (p.a_kfast ? j : 0);
          float x = 0.f;
          if (mj < p.M && kj < p.K) {
            const bool t1 = kj >= p.ks;
            x = to_f32((t1 ? a1 : a0)[mj * p.sam + (t1 ? kj - p.ks : kj) * p.sak]);
          }
          ra[j] = x;
        }
      }
    };
    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    load(0);
    for (int k0 = 0; k0 < KK; k0 += BK) {
      __syncthreads();   // B staged (first slab) / the previous A slab has been read
      put(ra, p.a_kfast, amm, akk, LDK, Ah, Al, std::integral_constant<bool, SA>());
      __syncthreads();
      if (k0 + BK < KK) load(k0 + BK);
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        const int kof = ks * 32 + (lane / 16) * 8;
        bf16x8 ah[2], al[2], bh[4], bl[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = wm * 32 + i * 16 + lane % 16;
          ah[i] = *reinterpret_cast<const bf16x8*>(&Ah[row * LDK + kof]);
          if constexpr (SA) al[i] = *reinterpret_cast<const bf16x8*>(&Al[row * LDK + kof]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = wn * 64 + j * 16 + lane % 16;
          bh[j] = *reinterpret_cast<const bf16x8*>(&Bh[col * LDB + k0 + kof]);
          if constexpr (SB) bl[j] = *reinterpret_cast<const bf16x8*>(&Bl[col * LDB + k0 + kof]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
            if constexpr (SB) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
            if constexpr (SA) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
          }
      }
    }
    // acc[i][j][r] = C[wm*32 + i*16 + (lane/16)*4 + r][wn*64 + j*16 + lane%16]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = wn * 64 + j * 16 + lane % 16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * 32 + i * 16 + (lane / 16) * 4 + r;
          if (m >= p.M || n >= p.N) continue;
          const int64_t idx = m * p.ldc + n;
          float val = alpha * acc[i][j][r];
          if (p.accumulate) val += to_f32(c[idx]);
          c[idx] = from_f32<TC>(val);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// kv_grad_bf16_d128: the Gram adjoint of one frame, bf16 tokens, head_dim 128:
//   dK_t = beta_t (K_t C1 + V_t C2),  dV_t = beta_t K_t C2^T,
// C1 = dA_t + dA_t^T (symmetric) and C2 = dB_t from cdb[frame][0 / 1] (fp32).
// One workgroup per frame reads K_t and V_t once and writes dK_t and dV_t once.
// C1 and C2 sit in LDS as bf16 hi + lo pairs (four 32 KB matrices, 16-byte
// chunk c of row r at c ^ (((r & 7) << 1) | ((r >> 3) & 1))).  Eight waves (two
// per SIMD) take 16-token tiles and compute the transposed outputs dK^T, dV^T
// (rows = output dimension, columns = tokens) on v_mfma_f32_16x16x32_bf16,
// the token rows of K and V being the B operand straight from HBM (the next
// tile's rows are loaded while the current one is multiplied).  The A operand
// is a 16-byte row read of C1 or C2 (C1 = C1^T) for the K terms and, for
// V C2, two transposed reads of C2 (ds_read_b64_tr_b16: lane group g gets rows
// 32 ks + 4 g + 0..3 and 32 ks + 16 + 4 g + 0..3 of one column), so V is loaded
// in that dimension order.  Every fp32 operand gives two products (hi, lo);
// K and V are exact in bf16.  (Four waves of 32-token tiles on 32x32x16
// products read C1 and C2 half as often per token, but need 482 registers,
// one wave per SIMD.)
namespace kvg {
constexpr int D = 128, ROWB = D * 2, MATB = D * ROWB, TT = 16, NW = 8;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r & 7) << 1) | ((r >> 3) & 1)); }
}

__global__ __launch_bounds__(512) void kv_grad_bf16_d128_kernel(const bf16* __restrict__ k,
                                                                const bf16* __restrict__ v,
                                                                const float* __restrict__ cdb,
                                                                const float* __restrict__ beta,
                                                                bf16* __restrict__ dk, bf16* __restrict__ dv,
                                                                int T, int N, int Lt) {
  using namespace kvg;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * MATB];   // C1 hi, C1 lo, C2 hi, C2 lo
  const int f = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = lane / 16, j16 = lane % 16;

  // C1, C2 -> hi / lo bf16 in LDS, 8 elements (one 16-byte chunk) per step
  const float* c1 = cdb + (int64_t)f * 2 * D * D;
  for (int u = tid; u < 2 * D * (D / 8); u += 512) {
    const int m = u / (D * D / 8), rem = u % (D * D / 8), r = rem / 16, c = rem % 16;
    const float* src = c1 + m * D * D + r * D + c * 8;
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = (bf16)x[e];
      lo[e] = (bf16)(x[e] - (float)hi[e]);
    }
    const int off = r * ROWB + swz(r, c) * 16;
    *reinterpret_cast<bf16x8*>(lds + (2 * m) * MATB + off) = hi;
    *reinterpret_cast<bf16x8*>(lds + (2 * m + 1) * MATB + off) = lo;
  }
  __syncthreads();

  const float bt = beta[f];
  const int64_t row0 = (int64_t)(f / T) * Lt + (int64_t)(f % T) * N;   // first token row of the frame
  const bf16* kf = k + row0 * D;
  const bf16* vf = v + row0 * D;
  const int ntile = (N + TT - 1) / TT;

  // A-operand addresses (bytes into lds): row reads of row 16 nb + j16, chunk
  // 4 ks + g (the swizzle depends on the row mod 16, so nb moves the address by
  // a constant); transposed reads: lane j16 of group g reads row 4 g + j16 / 4
  // of a 16-row step, columns 16 nb + 4 (j16 % 4) .. + 3, and receives column
  // 16 nb + j16 of rows 4 g .. 4 g + 3
  int aoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) aoff[ks] = j16 * ROWB + swz(j16, 4 * ks + g) * 16;
  int toff[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int r = 4 * g + j16 / 4;
    toff[nb] = 2 * MATB + r * ROWB + swz(r, 2 * nb + (j16 % 4) / 2) * 16 + 8 * (j16 % 2);
  }
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  auto tr = [&](int off) { return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((__attribute__((address_space(3))) unsigned char*)lds + off)); };
  auto rd = [&](int off) { return *reinterpret_cast<const bf16x8*>(lds + off); };

  // token operands of one tile: K dims 32 ks + 8 g .. + 7, V dims 32 ks + 4 g .. + 3
  // and 32 ks + 16 + 4 g .. + 3 (the transposed reads' order)
  bf16x8 kb[2][4];
  u32x2 va[2][4], vb[2][4];
  auto load = [&](int buf, int tile) {
    const int t = min(TT * tile + j16, N - 1);   // rows past the frame repeat its last row (not stored)
    const bf16* kr = kf + (int64_t)t * D;
    const bf16* vr = vf + (int64_t)t * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kb[buf][ks] = *reinterpret_cast<const bf16x8*>(kr + 32 * ks + 8 * g);
      va[buf][ks] = *reinterpret_cast<const u32x2*>(vr + 32 * ks + 4 * g);
      vb[buf][ks] = *reinterpret_cast<const u32x2*>(vr + 32 * ks + 16 + 4 * g);
    }
  };
  auto compute = [&](int buf, int tile) {
    f32x4 ak[8], av[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      ak[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      av[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 kk = kb[buf][ks];
      const bf16x8 vv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va[buf][ks], vb[buf][ks], 0, 1, 2, 3));
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        // keep each step's LDS reads next to its products
        asm volatile("" ::: "memory");
        const int ao = aoff[ks] + nb * 16 * ROWB;
        const bf16x8 c1h = rd(ao), c1l = rd(MATB + ao), c2h = rd(2 * MATB + ao), c2l = rd(3 * MATB + ao);
        const int to = toff[nb] + ks * 32 * ROWB;
        const i16x4 th0 = tr(to), th1 = tr(to + 16 * ROWB);
        const i16x4 tl0 = tr(to + MATB), tl1 = tr(to + MATB + 16 * ROWB);
        const bf16x8 c2th = __builtin_bit_cast(bf16x8, __builtin_shufflevector(th0, th1, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 c2tl = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tl0, tl1, 0, 1, 2, 3, 4, 5, 6, 7));
        ak[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c1h, kk, ak[nb], 0, 0, 0);
        av[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c2h, kk, av[nb], 0, 0, 0);
        ak[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c2th, vv, ak[nb], 0, 0, 0);
        av[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c2l, kk, av[nb], 0, 0, 0);
        ak[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c1l, kk, ak[nb], 0, 0, 0);
        ak[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c2tl, vv, ak[nb], 0, 0, 0);
      }
    }
    // ak[nb][e] = dK^T(n = 16 nb + 4 g + e, token 16 tile + j16)
    const int t = TT * tile + j16;
    if (t < N) {
      bf16* dkr = dk + (row0 + t) * D;
      bf16* dvr = dv + (row0 + t) * D;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int n = 16 * nb + 4 * g;
        bf16x4 ok, ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ok[e] = (bf16)(bt * ak[nb][e]);
          ov[e] = (bf16)(bt * av[nb][e]);
        }
        *reinterpret_cast<bf16x4*>(dkr + n) = ok;
        *reinterpret_cast<bf16x4*>(dvr + n) = ov;
      }
    }
  };
  int tile = wave;
  if (tile < ntile) load(0, tile);
  for (; tile < ntile; tile += 2 * NW) {
    if (tile + NW < ntile) load(1, tile + NW);
    compute(0, tile);
    if (tile + NW >= ntile) break;
    if (tile + 2 * NW < ntile) load(0, tile + 2 * NW);
    compute(1, tile + NW);
  }
}

// RMSNorm weight of ones, for callers that pass none
__device__ float kUnitWeight[128] = {   // global (not constant) memory: loads stay global, not flat
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};

// ---------------------------------------------------------------------------
// tok_grad_bf16_d128<SECOND>: the token side of the readout adjoint, one scan
// direction of one frame per workgroup (bf16 tokens, head_dim 128):
//   u = S q,  rho = sqrt(mean u^2 + eps),  r = u / rho,  g = w do,
//   du = (g - r mean(g r)) / rho,  dq += S^T du,
//   dS = sum over the frame's tokens of du q^T,  dw = sum of r do.
// Nothing token-sized but q, do and dq leaves the chip: u and du stay in
// registers.  The first direction writes its share of dq in fp32 (to the
// workspace); the second adds its own and writes dq in bf16.
// Eight waves (two per SIMD, so that one wave's vector and LDS work runs
// beside the other's matrix products) each take a 16-token tile per round:
//   u^T = S q^T      v_mfma_f32_16x16x32_bf16, A = rows of S (hi, lo) from LDS,
//                    B = q straight from HBM (lane: token l%16, dims 8(l/16)..+7
//                    of each 32-dim step); the result holds, per lane, token
//                    l%16 at dims 16 ib + 4(l/16) + 0..3, so a token's 128 values
//                    sit in four lanes and the RMSNorm sums take two cross-lane
//                    adds;
//   dq^T = S^T du^T  same product shape; du is already the B operand if the
//                    32-dim step's k order is taken as dims 4(l/16) + 0..3 then
//                    16 + 4(l/16) + 0..3, and A (columns of S) comes from two
//                    ds_read_b64_tr_b16 reads of four rows each in that order;
//   dS = du^T q      after the round's barrier, wave w forms dS rows
//                    16 w .. 16 w + 15 over the round's tiles on
//                    v_mfma_f32_16x16x16_bf16 (one tile = one 16-token step),
//                    both operands transposed reads of the staged rows.
// LDS: S as bf16 hi + lo (64 KB, rows of 256 bytes, chunk c of row r at
// c ^ (((r & 7) << 1) | ((r >> 3) & 1))) and, per wave, the tile's du hi, du lo
// and q rows (12 KB): 160 KB, one workgroup per CU.  (With 32-token tiles on
// 32x32x16 products, which read S half as often, one wave per SIMD needs all
// 512 registers and runs the phases one after another: 8.6 against 7.5 ms.)
// x summed over lanes l, l ^ 16, l ^ 32 and l ^ 48 with two lane swaps (each
// returns the pair {own, partner} in some order, so their sum is exact and
// the same in every lane of the group)
__device__ __forceinline__ float sum_lanes_16_32(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
namespace tkg {
constexpr int D = 128, ROWB = 256, MATB = D * ROWB, TT = 16, TILEB = TT * ROWB;
constexpr int NW = 8, STG = 2 * MATB, STGW = 3 * TILEB;
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r & 7) << 1) | ((r >> 3) & 1)); }
static_assert(STG + NW * STGW == 160 * 1024, "LDS budget");
}

template <bool SECOND>
__global__ __launch_bounds__(512) void tok_grad_bf16_d128_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ d_out, int64_t ldo, const float* __restrict__ states,
    const float* __restrict__ rms_w, float* __restrict__ dqp, bf16* __restrict__ dq, float* __restrict__ dsg,
    float* __restrict__ dwp, int dir, int64_t nf, int H, int T, int N, int Lt, float eps) {
  using namespace tkg;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[STG + NW * STGW];   // 160 KB
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int64_t f = blockIdx.x;
  const int64_t bh = f / T;
  const int t = (int)(f % T);
  const int64_t b = bh / H;
  const int hh = (int)(bh % H);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = lane / 16, j16 = lane % 16;

  // S -> hi / lo bf16, rows of 256 bytes with swizzled 16-byte chunks
  const float* S = states + ((int64_t)dir * nf + f) * D * D;
  for (int u = tid; u < D * (D / 8); u += 512) {
    const int r = u / 16, c = u % 16;
    const float* src = S + r * D + c * 8;
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b4 = *reinterpret_cast<const float4*>(src + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, b4.x, b4.y, b4.z, b4.w};
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = (bf16)x[e];
      lo[e] = (bf16)(x[e] - (float)hi[e]);
    }
    const int off = r * ROWB + swz(r, c) * 16;
    *reinterpret_cast<bf16x8*>(lds + off) = hi;
    *reinterpret_cast<bf16x8*>(lds + MATB + off) = lo;
  }

  auto tr = [&](int off) { return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)lds + off)); };
  auto rd = [&](int off) { return *reinterpret_cast<const bf16x8*>(lds + off); };
  auto cat = [](i16x4 a, i16x4 c) { return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7)); };
  // row reads of S for the u product: row 16 ib + j16, chunk 4 ks + g (the
  // swizzle depends on the row mod 16, so ib moves the address by a constant)
  int aoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) aoff[ks] = j16 * ROWB + swz(j16, 4 * ks + g) * 16;
  // transposed reads of a row-major [rows][128] matrix, four rows from row r0:
  // lane j16 of group g reads row r0 + 4 g + j16 / 4, columns 16 cb + 4 (j16 % 4)
  // .. + 3, and receives column 16 cb + j16 of rows r0 + 4 g .. + 3
  int toff[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const int r = 4 * g + j16 / 4;
    toff[cb] = r * ROWB + swz(r, 2 * cb + (j16 % 4) / 2) * 16 + 8 * (j16 % 2);
  }

  const bf16* qf = q + (bh * Lt + (int64_t)t * N) * D;
  const bf16* dof = d_out + (b * Lt + (int64_t)t * N) * ldo + (int64_t)hh * D;
  const float* wf = rms_w ? rms_w + (int64_t)hh * D : kUnitWeight;
  float* dqpf = dqp + f * (int64_t)N * D;
  bf16* dqf = dq + (bh * Lt + (int64_t)t * N) * D;
  const int ntile = (N + TT - 1) / TT, nround = (ntile + NW - 1) / NW;

  float dw[8][4];        // sum over this lane's tokens of r do at dims 16 ib + 4 g + e
  f32x4 dsa[8];          // dS rows 16 wave + 4 g + e, column 16 cb + j16
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dsa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) dw[i][e] = 0.f;
  }
  __syncthreads();

  for (int round = 0; round < nround; ++round) {
    const int tile = round * NW + wave;
    unsigned char* sdh = lds + STG + wave * STGW;   // du hi rows of this wave's tile
    unsigned char* sdl = sdh + TILEB;                // du lo rows
    unsigned char* sq = sdl + TILEB;                 // q rows
    if (tile < ntile) {
      const int n = TT * tile + j16;
      const bool valid = n < N;
      const int nn = valid ? n : N - 1;
      // q: B operand of u^T = S q^T, also staged as rows for dS
      bf16x8 qb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        qb[ks] = *reinterpret_cast<const bf16x8*>(qf + (int64_t)nn * D + 32 * ks + 8 * g);
        *reinterpret_cast<bf16x8*>(sq + j16 * ROWB + swz(j16, 4 * ks + g) * 16) = qb[ks];
      }
      bf16x4 dob[8];
      float4 wv[8];   // the RMSNorm weight at the same dims, loaded here so that the u products cover it
#pragma unroll
      for (int ib = 0; ib < 8; ++ib) {
        dob[ib] = *reinterpret_cast<const bf16x4*>(dof + (int64_t)nn * ldo + 16 * ib + 4 * g);
        wv[ib] = *reinterpret_cast<const float4*>(wf + 16 * ib + 4 * g);
      }
      // u^T; ua[ib][e] = u(token j16, dim 16 ib + 4 g + e)
      f32x4 ua[8];
#pragma unroll
      for (int ib = 0; ib < 8; ++ib) ua[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
          asm volatile("" ::: "memory");   // keeps each step's LDS reads next to its products
          const int ao = aoff[ks] + ib * 16 * ROWB;
          ua[ib] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rd(ao), qb[ks], ua[ib], 0, 0, 0);
          ua[ib] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rd(MATB + ao), qb[ks], ua[ib], 0, 0, 0);
        }
      // RMSNorm adjoint (the four lanes j16 + 16 g' hold the token's 128 values)
      float ss = 0.f;
#pragma unroll
      for (int ib = 0; ib < 8; ++ib)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += ua[ib][e] * ua[ib][e];
      ss = sum_lanes_16_32(ss);
      const float inv = 1.f / sqrtf(ss * (1.f / D) + eps);
      const float vm = valid ? inv : 0.f;      // tokens past the frame contribute nothing
      float gw[8][4];
      float gr = 0.f;
#pragma unroll
      for (int ib = 0; ib < 8; ++ib) {
        const float w4[4] = {wv[ib].x, wv[ib].y, wv[ib].z, wv[ib].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dv = (float)dob[ib][e];
          const float u = ua[ib][e];
          gw[ib][e] = w4[e] * dv;
          gr += gw[ib][e] * u;
          const float rr = u * vm;                // r = u / rho (zero past the frame)
          ua[ib][e] = rr;
          dw[ib][e] += rr * dv;
        }
      }
      gr = sum_lanes_16_32(gr);
      const float c = gr * inv * inv * (1.f / D);   // mean(g r) / rho
      // du = (g - r mean(g r)) / rho as hi / lo bf16: B operand of dq^T for the
      // 32-dim step ks in the k order (dims 32 ks + 4 g + 0..3, 32 ks + 16 + 4 g + 0..3),
      // and staged as rows for dS (8-byte pieces at dims 16 ib + 4 g)
      bf16x8 duh[4], dul[4];
#pragma unroll
      for (int ib = 0; ib < 8; ++ib) {
        bf16x4 hv, lv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = gw[ib][e] * vm - ua[ib][e] * c;
          hv[e] = (bf16)x;
          lv[e] = (bf16)(x - (float)hv[e]);
          duh[ib / 2][4 * (ib % 2) + e] = hv[e];
          dul[ib / 2][4 * (ib % 2) + e] = lv[e];
        }
        const int off = j16 * ROWB + swz(j16, 2 * ib + g / 2) * 16 + 8 * (g % 2);
        *reinterpret_cast<bf16x4*>(sdh + off) = hv;
        *reinterpret_cast<bf16x4*>(sdl + off) = lv;
      }
      // the first direction's dq share, loaded before the products so that they
      // cover its latency (rows past the frame read the last row and are not stored)
      float4 prev[8];
      if constexpr (SECOND) {
#pragma unroll
        for (int ib = 0; ib < 8; ++ib)
          prev[ib] = *reinterpret_cast<const float4*>(dqpf + (int64_t)nn * D + 16 * ib + 4 * g);
      }
      // dq^T = S^T du^T: A = transposed reads of S (hi, lo), B = du (hi, lo); lo x lo dropped
      f32x4 qa[8];
#pragma unroll
      for (int ib = 0; ib < 8; ++ib) qa[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
          asm volatile("" ::: "memory");
          const int to = ks * 32 * ROWB + toff[ib];
          const bf16x8 ah = cat(tr(to), tr(to + 16 * ROWB));
          const bf16x8 al = cat(tr(MATB + to), tr(MATB + to + 16 * ROWB));
          qa[ib] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, duh[ks], qa[ib], 0, 0, 0);
          qa[ib] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, dul[ks], qa[ib], 0, 0, 0);
          qa[ib] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, duh[ks], qa[ib], 0, 0, 0);
        }
      // qa[ib][e] = dq(token j16, dim 16 ib + 4 g + e) of this direction
      if (valid) {
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
          const int j = 16 * ib + 4 * g;
          if constexpr (SECOND) {
            bf16x4 o;
            o[0] = (bf16)(prev[ib].x + qa[ib][0]);
            o[1] = (bf16)(prev[ib].y + qa[ib][1]);
            o[2] = (bf16)(prev[ib].z + qa[ib][2]);
            o[3] = (bf16)(prev[ib].w + qa[ib][3]);
            *reinterpret_cast<bf16x4*>(dqf + (int64_t)n * D + j) = o;
          } else {
            *reinterpret_cast<float4*>(dqpf + (int64_t)n * D + j) = make_float4(qa[ib][0], qa[ib][1], qa[ib][2], qa[ib][3]);
          }
        }
      }
    }
    __syncthreads();
    // dS rows 16 wave .. + 15 over the tiles of this round (one 16-token step
    // each): A = du^T (transposed reads of the staged du rows, column block =
    // wave), B = q (transposed reads, column block cb)
    for (int tt = 0; tt < NW; ++tt) {
      if (round * NW + tt >= ntile) break;
      const int base = STG + tt * STGW;
      const i16x4 ah = tr(base + toff[wave]);
      const i16x4 al = tr(base + TILEB + toff[wave]);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        asm volatile("" ::: "memory");
        const i16x4 bq = tr(base + 2 * TILEB + toff[cb]);
        dsa[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bq, dsa[cb], 0, 0, 0);
        dsa[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bq, dsa[cb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // dS: dsa[cb][e] = dS(row 16 wave + 4 g + e, column 16 cb + j16)
  float* ds = dsg + (f * 2 + dir) * D * D;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int e = 0; e < 4; ++e) ds[(16 * wave + 4 * g + e) * D + 16 * cb + j16] = dsa[cb][e];
  // dw: sum the 16 lanes of each group (they hold the same dims), then the eight waves
#pragma unroll
  for (int ib = 0; ib < 8; ++ib)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = dw[ib][e];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, kWave);
      dw[ib][e] = x;
    }
  float* red = reinterpret_cast<float*>(lds);   // S is no longer read
  if (j16 == 0) {
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave * D + 16 * ib + 4 * g + e] = dw[ib][e];
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w * D + tid];
    dwp[(f * 2 + dir) * D + tid] = s;
  }
}

hipError_t launch_tok_grad(const void* q, const void* d_out, int64_t ldo, const float* states, const float* rms_w,
                           float* dqp, void* dq, float* dsg, float* dwp, int64_t nf, int H, int T, int N, int Lt,
                           float eps, hipStream_t st) {
  if (nf <= 0) return hipSuccess;
  if (nf > 0x7FFFFFFF) return hipErrorInvalidValue;
  tok_grad_bf16_d128_kernel<false><<<(unsigned)nf, 512, 0, st>>>(
      (const bf16*)q, (const bf16*)d_out, ldo, states, rms_w, dqp, (bf16*)dq, dsg, dwp, 0, nf, H, T, N, Lt, eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tok_grad_bf16_d128_kernel<true><<<(unsigned)nf, 512, 0, st>>>(
      (const bf16*)q, (const bf16*)d_out, ldo, states, rms_w, dqp, (bf16*)dq, dsg, dwp, 1, nf, H, T, N, Lt, eps);
  return hipGetLastError();
}

hipError_t launch_kv_grad(const void* k, const void* v, const float* cdb, const float* beta, void* dk, void* dv,
                          int64_t nf, int T, int N, int Lt, hipStream_t st) {
  if (nf <= 0) return hipSuccess;
  if (nf > 0x7FFFFFFF) return hipErrorInvalidValue;
  kv_grad_bf16_d128_kernel<<<(unsigned)nf, 512, 0, st>>>((const bf16*)k, (const bf16*)v, cdb, beta, (bf16*)dk,
                                                         (bf16*)dv, T, N, Lt);
  return hipGetLastError();
}

hipError_t launch_bgemm(int ta, int tb, int tc, BGemm p, hipStream_t st, bool mfma) {
  if (p.M <= 0 || p.N <= 0 || p.batch <= 0) return hipSuccess;
  if (p.ks <= 0) p.ks = p.K;
  p.a_kfast = p.sak == 1;
  p.b_nfast = p.sbn == 1;
  const int64_t tiles = (int64_t)((p.M + bg::BM - 1) / bg::BM) * ((p.N + bg::BN - 1) / bg::BN);
  const int64_t blocks = tiles * p.batch;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (mfma) {
    // 16-element runs load as 16-byte vectors when every base pointer and every
    // non-unit stride keeps them 16-byte aligned (8 elements covers both types)
    auto al16 = [](const void* q) { return ((uintptr_t)q & 15u) == 0; };
    bool vec = al16(p.a0) && al16(p.b0) && al16(p.c) && (!p.a1 || al16(p.a1)) && (!p.b1 || al16(p.b1)) &&
               p.ks % 16 == 0 && (p.sak == 1 || p.sam == 1) && (p.sbn == 1 || p.sbk == 1);
    for (int64_t x : {p.sam, p.sak, p.sbk, p.sbn, p.sa[0], p.sa[1], p.sa[2], p.sb[0], p.sb[1], p.sb[2], p.ldc,
                      p.sc[0], p.sc[1], p.sc[2]})
      vec = vec && (x == 1 || x % 8 == 0);
    p.vec = vec;
    if (p.vec && p.N == 128 && (p.K == 128 || p.K == 256)) {
      // the B operand resident in LDS, eight 64-row tiles of A per workgroup
      constexpr int kTilesPerWg = 8;
      const int64_t tm = (p.M + br::BM - 1) / br::BM;
      const int64_t wgs = (tm + kTilesPerWg - 1) / kTilesPerWg * p.batch;
      if (wgs > 0x7FFFFFFFLL) return hipErrorInvalidValue;
#define VDN_BR(A, B, C)                                                                               \
  (p.K == 128 ? bgemm_mfma_resident_kernel<A, B, C, 128><<<(unsigned)wgs, 256, 0, st>>>(p, kTilesPerWg) \
              : bgemm_mfma_resident_kernel<A, B, C, 256><<<(unsigned)wgs, 256, 0, st>>>(p, kTilesPerWg))
      if (ta == 1 && tb == 0 && tc == 0) VDN_BR(bf16, float, float);
      else if (ta == 0 && tb == 1 && tc == 0) VDN_BR(float, bf16, float);
      else if (ta == 0 && tb == 0 && tc == 1) VDN_BR(float, float, bf16);
      else if (ta == 1 && tb == 0 && tc == 1) VDN_BR(bf16, float, bf16);
      else return hipErrorInvalidValue;
#undef VDN_BR
      return hipGetLastError();
    }
    // 128-column tiles when the output is that wide: each token row of A is then read once
    const bool wide = p.N > 64;
    const int bn = wide ? 128 : 64;
    const int64_t mtiles = (int64_t)((p.M + bm::BM - 1) / bm::BM) * ((p.N + bn - 1) / bn) * p.batch;
    if (mtiles > 0x7FFFFFFFLL) return hipErrorInvalidValue;
#define VDN_BM(A, B, C)                                                                  \
  (wide ? bgemm_mfma_kernel<A, B, C, 128><<<(unsigned)mtiles, 256, 0, st>>>(p)         \
        : bgemm_mfma_kernel<A, B, C, 64><<<(unsigned)mtiles, 256, 0, st>>>(p))
    if (ta == 1 && tb == 0 && tc == 0) VDN_BM(bf16, float, float);
    else if (ta == 0 && tb == 1 && tc == 0) VDN_BM(float, bf16, float);
    else if (ta == 0 && tb == 0 && tc == 1) VDN_BM(float, float, bf16);
    else if (ta == 1 && tb == 0 && tc == 1) VDN_BM(bf16, float, bf16);
    else return hipErrorInvalidValue;
#undef VDN_BM
    return hipGetLastError();
  }
#define VDN_BG(A, B, C) bgemm_kernel<A, B, C, false><<<(unsigned)blocks, 256, 0, st>>>(p)
  // the combinations the gradient uses: bf16 or fp32 tokens against fp32 matrices
  if (ta == 1 && tb == 0 && tc == 0) VDN_BG(bf16, float, float);
  else if (ta == 0 && tb == 1 && tc == 0) VDN_BG(float, bf16, float);
  else if (ta == 0 && tb == 0 && tc == 1) VDN_BG(float, float, bf16);
  else if (ta == 1 && tb == 0 && tc == 1) VDN_BG(bf16, float, bf16);
  // fp32 operands and result: fp32 MFMA
  else if (ta == 0 && tb == 0 && tc == 0) bgemm_kernel<float, float, float, true><<<(unsigned)blocks, 256, 0, st>>>(p);
  else return hipErrorInvalidValue;
#undef VDN_BG
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sum over a workgroup of 256 threads (four waves); every thread gets the sum.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// ---------------------------------------------------------------------------
// fill and per-frame scaling of the recomputed Gram products:
// A_t = beta_t (K^T K)_t, B_t = beta_t (V^T K)_t
__global__ __launch_bounds__(256) void fill_kernel(float* x, float v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = v;
}

__global__ __launch_bounds__(256) void scale_frames_kernel(const float* __restrict__ kk,
                                                           const float* __restrict__ vk,
                                                           const float* __restrict__ beta,
                                                           float* __restrict__ am, float* __restrict__ bm,
                                                           int64_t dd, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const float b = beta[i / dd];
  am[i] = b * kk[i];
  bm[i] = b * vk[i];
}

// ---------------------------------------------------------------------------
// rms_bwd: workgroup (frame f, direction) walks the frame's N tokens, one wave
// per token.  U holds u = S_t q on entry and du on exit, [frame][dir][N][D].
// dw_part[f][dir][i] = sum over the frame's tokens of r_i do_i.
template <typename T, int D>
__global__ __launch_bounds__(256) void rms_bwd_kernel(float* __restrict__ U, const T* __restrict__ d_out,
                                                      int64_t ldo, const float* __restrict__ rms_w,
                                                      float* __restrict__ dw_part, int H, int T_, int N,
                                                      int Lt, float eps) {
  constexpr int PL = (D + kWave - 1) / kWave;   // elements per lane
  __shared__ float red[4][D];
  const int64_t f = blockIdx.x / 2;
  const int dir = blockIdx.x % 2;
  const int64_t bh = f / T_;
  const int t = (int)(f % T_);
  const int64_t b = bh / H;
  const int h = (int)(bh % H);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  float w[PL], dw[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) {
    const int c = lane + kWave * e;
    w[e] = c < D ? (rms_w ? rms_w[h * D + c] : 1.f) : 0.f;
    dw[e] = 0.f;
  }
  for (int n = wave; n < N; n += 4) {
    float* u = U + ((f * 2 + dir) * N + n) * D;
    const T* dor = d_out + (b * Lt + (int64_t)t * N + n) * ldo + (int64_t)h * D;
    float uv[PL], dv[PL];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < PL; ++e) {
      const int c = lane + kWave * e;
      uv[e] = c < D ? u[c] : 0.f;
      dv[e] = c < D ? to_f32(dor[c]) : 0.f;
      ss += uv[e] * uv[e];
    }
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss / D + eps);
    float gr = 0.f;
#pragma unroll
    for (int e = 0; e < PL; ++e) gr += w[e] * dv[e] * uv[e] * inv;
    const float mgr = wave_sum(gr) / D;
#pragma unroll
    for (int e = 0; e < PL; ++e) {
      const int c = lane + kWave * e;
      const float r = uv[e] * inv;
      dw[e] += r * dv[e];
      if (c < D) u[c] = (w[e] * dv[e] - r * mgr) * inv;
    }
  }
#pragma unroll
  for (int e = 0; e < PL; ++e) {
    const int c = lane + kWave * e;
    if (c < D) red[wave][c] = dw[e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += 256)
    dw_part[(f * 2 + dir) * D + c] = red[0][c] + red[1][c] + red[2][c] + red[3][c];
}

// ---------------------------------------------------------------------------
// scan_bwd: rows of G are independent given the M_t, as in the forward scan.
// Workgroup (row block, batch-head, direction) walks the frames against the
// direction that scan wrote them in.  dsg holds dS_t on entry and G_t on exit;
// dx receives dX_t = G_t M_t^T; both [frame][dir][D][D].  Mt holds M_t^T.
template <int D, int R>
__global__ __launch_bounds__(256) void scan_bwd_kernel(const float* __restrict__ Mt,
                                                       const float* __restrict__ gamma,
                                                       float* __restrict__ dsg, float* __restrict__ dx,
                                                       int T_) {
  constexpr int TPR = 256 / R;     // threads per row
  constexpr int CPT = D / TPR;     // columns per thread
  __shared__ float Gs[R][D + 4];
  const int tid = threadIdx.x;
  const int row = tid / TPR, col0 = (tid % TPR) * CPT;
  const int r0 = blockIdx.x * R;
  const int64_t bh = blockIdx.y;
  const int dir = blockIdx.z;
  float carry[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) carry[c] = 0.f;
  for (int step = 0; step < T_; ++step) {
    const int t = dir ? step : T_ - 1 - step;
    const int64_t f = bh * T_ + t;
    const int64_t off = ((f * 2 + dir) * D + r0 + row) * D + col0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const float g = dsg[off + c] + carry[c];
      dsg[off + c] = g;
      Gs[row][col0 + c] = g;
    }
    __syncthreads();
    const float* mt = Mt + f * D * D + col0;
    float acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
    for (int j = 0; j < D; ++j) {
      const float gj = Gs[row][j];
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[c] = fmaf(gj, mt[j * D + c], acc[c]);
    }
    const float gm = gamma[f];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      dx[off + c] = acc[c];
      carry[c] = gm * acc[c];
    }
    __syncthreads();   // Gs is rewritten by the next frame
  }
}

// ---------------------------------------------------------------------------
// scan_bwd on fp32 MFMA for head_dim 64 and 128: the same row-parallel scheme
// as the forward scan (one workgroup of D/32 waves per 32 state rows of one
// (batch, head, direction); G_t in LDS; wave w forms the 32 x 32 block of
// columns 32w.. of dX_t = G_t M_t^T with v_mfma_f32_32x32x2f32; M_t rows, the
// next frames' dS two frames ahead and the next M one frame ahead are loaded
// while a frame's products run).  M_t is the inverse of the symmetric matrix
// I + A_t, so M_t^T = M_t: the B operand is read from the stored M_t^T in the
// forward scan's row order (16-byte loads) rather than down its columns.  The
// epilogue writes dX_t and G_next = dS_next + gamma_t dX_t (over dS_next, which
// the later stages read as G).
namespace sb {
constexpr int R = 32;
typedef float f32x16 __attribute__((ext_vector_type(16)));
}  // namespace sb

template <int D>
__global__ __launch_bounds__(2 * D) void scan_bwd_mfma_kernel(const float* __restrict__ Mt,
                                                             const float* __restrict__ gamma,
                                                             float* __restrict__ dsg, float* __restrict__ dx,
                                                             int T, int total) {
  using namespace sb;
  constexpr int LD = D + 4, NRB = D / R, KG = D / 8;
  __shared__ __attribute__((aligned(16))) float P[2][R * LD];   // G_t and dX_t, rows r0 .. r0+31
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int l32 = lane % 32, h = lane / 32;
  const int lid = xcd_remap(blockIdx.x, total);
  const int dir = lid & 1, rb = (lid >> 1) % NRB;
  const int64_t bh = lid / (2 * NRB);
  const int r0 = rb * R, n0 = wave * 32;
  const int crow = tid / (D / 4), ccol = 4 * (tid % (D / 4));

  // frame of adjoint step `step` (the forward direction runs backwards in time and
  // vice versa), clamped to the last step (loads past the end are not used)
  auto fidx = [&](int step) -> int64_t {
    const int c = step < T ? step : T - 1;
    return bh * T + (dir ? c : T - 1 - c);
  };
  // element (r0 + row, col) of frame f's matrix of this direction in dsg / dx
  auto eoff = [&](int64_t f, int row, int col) { return ((f * 2 + dir) * D + r0 + row) * (int64_t)D + col; };
  auto load_m = [&](float4 (&m)[KG], int step) {
    const float* mp = Mt + fidx(step) * D * D + (int64_t)(n0 + l32) * D + 4 * h;
#pragma unroll
    for (int i = 0; i < KG; ++i) m[i] = *reinterpret_cast<const float4*>(mp + 8 * i);
  };
  auto load_g = [&](float4 (&b)[4], int step) {
    const float* bp = dsg + eoff(fidx(step), crow, ccol);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const float4*>(bp + 8 * j * D);
  };

  // one adjoint step: mc = M_s, mn <- M_{s+1}, bl <- dS_{s+2}, be = dS_{s+1};
  // G_s in X, dX_s and then G_{s+1} go to Y
  auto step = [&](int s, float4 (&mc)[KG], float4 (&mn)[KG], float4 (&bl)[4], const float4 (&be)[4],
                  const float* X, float* Y) {
    const int64_t fi = fidx(s), fn = fidx(s + 1);
    const float gc = gamma[fi];
    load_m(mn, s + 1);
    load_g(bl, s + 2);
    __builtin_amdgcn_sched_barrier(0);   // the next frames' loads go out before this frame's products
    const float* xrow = X + l32 * LD + 4 * h;
    float4 xv[KG];
#pragma unroll
    for (int i = 0; i < KG; ++i) xv[i] = *reinterpret_cast<const float4*>(xrow + 8 * i);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < KG; ++i) {
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xv[i].x, mc[i].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xv[i].y, mc[i].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xv[i].z, mc[i].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xv[i].w, mc[i].w, acc, 0, 0, 0);
    }
    // acc[r] = dX_s[r0 + 8 (r/4) + 4h + r%4][n0 + l32]
#pragma unroll
    for (int r = 0; r < 16; ++r) Y[(8 * (r / 4) + 4 * h + r % 4) * LD + n0 + l32] = acc[r];
    __syncthreads();   // dX_s complete in Y
    const bool more = s + 1 < T;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float* yp = Y + (crow + 8 * j) * LD + ccol;
      const float4 sv = *reinterpret_cast<const float4*>(yp);
      *reinterpret_cast<float4*>(dx + eoff(fi, crow + 8 * j, ccol)) = sv;
      float4 gn;
      gn.x = gc * sv.x + be[j].x;
      gn.y = gc * sv.y + be[j].y;
      gn.z = gc * sv.z + be[j].z;
      gn.w = gc * sv.w + be[j].w;
      if (more) *reinterpret_cast<float4*>(dsg + eoff(fn, crow + 8 * j, ccol)) = gn;
      *reinterpret_cast<float4*>(yp) = gn;
    }
    __syncthreads();   // G_{s+1} complete in Y
  };

  float4 m0[KG], m1[KG], b0[4], b1[4];
  load_m(m0, 0);
  load_g(b0, 0);
  load_g(b1, 1);
#pragma unroll
  for (int j = 0; j < 4; ++j)   // G of the first adjoint step is its dS (nothing follows it)
    *reinterpret_cast<float4*>(&P[0][(crow + 8 * j) * LD + ccol]) = b0[j];
  __syncthreads();
  int s = 0;
  for (; s + 1 < T; s += 2) {
    step(s, m0, m1, b0, b1, P[0], P[1]);
    step(s + 1, m1, m0, b1, b0, P[1], P[0]);
  }
  if (s < T) step(s, m0, m1, b0, b1, P[0], P[1]);
}

// ---------------------------------------------------------------------------
// frame_bwd: per frame f, X_t = gamma_t S_prev + B_t for both directions
// (S_prev = S_{t-1} forward, S_{t+1} backward, zero past the ends), into
// xs[f][dir]; dB_t = dX_f + dX_b into cdb[f][1]; dgamma_t.
__global__ __launch_bounds__(256) void frame_bwd_kernel(const float* __restrict__ states,
                                                        const float* __restrict__ bm,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ dx, float* __restrict__ xs,
                                                        float* __restrict__ cdb, float* __restrict__ dgamma,
                                                        int T_, int64_t nf, int64_t dd) {
  __shared__ float red[4];
  const int64_t f = blockIdx.x;
  const int t = (int)(f % T_);
  const float g = gamma[f];
  const float* sf = t > 0 ? states + (f - 1) * dd : nullptr;
  const float* sb = t < T_ - 1 ? states + (nf + f + 1) * dd : nullptr;
  float part = 0.f;
  for (int64_t e = threadIdx.x; e < dd; e += 256) {
    const float xf = dx[(f * 2) * dd + e], xb = dx[(f * 2 + 1) * dd + e];
    const float pf = sf ? sf[e] : 0.f, pb = sb ? sb[e] : 0.f;
    const float bt = bm[f * dd + e];
    xs[(f * 2) * dd + e] = g * pf + bt;
    xs[(f * 2 + 1) * dd + e] = g * pb + bt;
    cdb[(f * 2 + 1) * dd + e] = xf + xb;
    part += xf * pf + xb * pb;
  }
  part = block_sum(part, red);
  if (threadIdx.x == 0) dgamma[f] = part;
}

// ---------------------------------------------------------------------------
// sym_dbeta: per frame, cdb[f][0] = dA_t + dA_t^T and
// dbeta_t = <dA_t, K^T K> + <dB_t, V^T K> (kk, vk: the Gram products without beta).
template <int D>
__global__ __launch_bounds__(256) void sym_dbeta_kernel(const float* __restrict__ dA,
                                                        const float* __restrict__ kk,
                                                        const float* __restrict__ vk,
                                                        float* __restrict__ cdb, float* __restrict__ dbeta) {
  constexpr int DD = D * D;
  __shared__ float red[4];
  const int64_t f = blockIdx.x;
  const float* a = dA + f * DD;
  float part = 0.f;
  for (int e = threadIdx.x; e < DD; e += 256) {
    const int i = e / D, j = e % D;
    const float x = a[e];
    cdb[(f * 2) * DD + e] = x + a[j * D + i];
    part += x * kk[f * DD + e] + cdb[(f * 2 + 1) * DD + e] * vk[f * DD + e];
  }
  part = block_sum(part, red);
  if (threadIdx.x == 0) dbeta[f] = part;
}

// dw_reduce: drms_w[h*D + i] = sum over batch, frame and direction of dw_part.
__global__ __launch_bounds__(256) void dw_reduce_kernel(const float* __restrict__ part,
                                                        float* __restrict__ drms_w, int B, int H, int T_,
                                                        int D) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= H * D) return;
  const int h = idx / D, i = idx % D;
  float s = 0.f;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T_; ++t) {
      const int64_t f = ((int64_t)b * H + h) * T_ + t;
      s += part[(f * 2) * D + i] + part[(f * 2 + 1) * D + i];
    }
  drms_w[idx] = s;
}

// ---------------------------------------------------------------------------
hipError_t launch_fill(float* x, float v, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(x, v, n);
  return hipGetLastError();
}

hipError_t launch_scale_frames(const float* kk, const float* vk, const float* beta, float* am,
                               float* bm, int64_t nf, int64_t dd, hipStream_t st) {
  const int64_t total = nf * dd;
  if (total <= 0) return hipSuccess;
  scale_frames_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(kk, vk, beta, am, bm, dd, total);
  return hipGetLastError();
}

hipError_t launch_rms_bwd(int dtype, int d, float* U, const void* d_out, int64_t ldo,
                          const float* rms_w, float* dw_part, int64_t nf, int H, int T, int N, int Lt,
                          float eps, hipStream_t st) {
  if (nf <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)(nf * 2);
#define VDN_RB(TT, DD) \
  rms_bwd_kernel<TT, DD><<<blocks, 256, 0, st>>>(U, (const TT*)d_out, ldo, rms_w, dw_part, H, T, N, Lt, eps)
  if (dtype == 1) {
    if (d == 32) VDN_RB(bf16, 32); else if (d == 64) VDN_RB(bf16, 64); else VDN_RB(bf16, 128);
  } else {
    if (d == 32) VDN_RB(float, 32); else if (d == 64) VDN_RB(float, 64); else VDN_RB(float, 128);
  }
#undef VDN_RB
  return hipGetLastError();
}

hipError_t launch_scan_bwd(int d, const float* Mt, const float* gamma, float* dsg, float* dx, int BH,
                           int T, hipStream_t st) {
  if (BH <= 0) return hipSuccess;
  if (d == 64 || d == 128) {
    const int total = BH * 2 * (d / sb::R);   // d / 32 row blocks x 2 directions per (batch, head)
    if (d == 128) scan_bwd_mfma_kernel<128><<<total, 256, 0, st>>>(Mt, gamma, dsg, dx, T, total);
    else scan_bwd_mfma_kernel<64><<<total, 128, 0, st>>>(Mt, gamma, dsg, dx, T, total);
    return hipGetLastError();
  }
  constexpr int R = 16;
  dim3 grid(d / R, BH, 2);
  scan_bwd_kernel<32, R><<<grid, 256, 0, st>>>(Mt, gamma, dsg, dx, T);
  return hipGetLastError();
}

hipError_t launch_frame_bwd(const float* states, const float* bm, const float* gamma, const float* dx,
                            float* xs, float* cdb, float* dgamma, int T, int64_t nf, int d,
                            hipStream_t st) {
  if (nf <= 0) return hipSuccess;
  frame_bwd_kernel<<<(unsigned)nf, 256, 0, st>>>(states, bm, gamma, dx, xs, cdb, dgamma, T, nf,
                                                 (int64_t)d * d);
  return hipGetLastError();
}

hipError_t launch_sym_dbeta(int d, const float* dA, const float* kk, const float* vk, float* cdb,
                            float* dbeta, int64_t nf, hipStream_t st) {
  if (nf <= 0) return hipSuccess;
  if (d == 32) sym_dbeta_kernel<32><<<(unsigned)nf, 256, 0, st>>>(dA, kk, vk, cdb, dbeta);
  else if (d == 64) sym_dbeta_kernel<64><<<(unsigned)nf, 256, 0, st>>>(dA, kk, vk, cdb, dbeta);
  else sym_dbeta_kernel<128><<<(unsigned)nf, 256, 0, st>>>(dA, kk, vk, cdb, dbeta);
  return hipGetLastError();
}

hipError_t launch_dw_reduce(const float* part, float* drms_w, int B, int H, int T, int d,
                            hipStream_t st) {
  const int n = H * d;
  dw_reduce_kernel<<<(n + 255) / 256, 256, 0, st>>>(part, drms_w, B, H, T, d);
  return hipGetLastError();
}

}  // namespace vdn
