// Dense contractions of the layer: the two gate GEMMs and the summed output
// projections (10100.com article on Video DeltaNet, 方法概述 part 3: sigmoid
// gates and one output projection per branch, added).
//
// C[m][n] = epi(sum_k A[m][k] * Bt[n][k]) with both operands k-contiguous, so
// MFMA fragments come straight from LDS rows.  Weights arrive as [D_in, D_out]
// and are transposed once per call into the workspace (a few MB).
#include "vdn_common.h"
#include "vdn_internal.h"

namespace vdn {

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src,
                                                        T* __restrict__ dst, int rows, int cols,
                                                        int64_t ld_dst) {
  __shared__ T tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? src[(int64_t)r * cols + c] : from_f32<T>(0.f);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) dst[(int64_t)c * ld_dst + r] = tile[tx][i];
  }
}

// 128x128 output tile per workgroup, 4 waves in a 2x2 grid of 64x64 wave
// tiles (4x4 MFMA tiles of 16x16 each).  One K slab of 128 bytes per row is
// staged through LDS; rows are padded by 16 bytes to spread LDS banks.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const T* __restrict__ A,
                                                      const T* __restrict__ Bt,
                                                      T* __restrict__ C, int M, int N, int K,
                                                      int64_t lda, int64_t ldb, int64_t ldc,
                                                      int tiles_n, int total) {
  using MM = Mma<T>;
  constexpr int KP = MM::kPack, KS = MM::kStep;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int BM = 128, BN = 128, BK = 8 * EPC;
  constexpr int LDT = BK + EPC;
  __shared__ __attribute__((aligned(16))) T As[BM * LDT];
  __shared__ __attribute__((aligned(16))) T Bs[BN * LDT];

  const int lid = xcd_remap(blockIdx.x, total);
  const int tm = lid / tiles_n, tn = lid - tm * tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane % 16, lg = lane / 16;
  const int wr = wave / 2, wc = wave % 2;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < (BM * 8) / 256; ++it) {
      const int c = tid + it * 256;
      const int row = c / 8, kc = c % 8;
      const int gk = k0 + kc * EPC;
      const int64_t gm = m0 + row, gn = n0 + row;
      Chunk16 va = zero_chunk(), vb = zero_chunk();
      if (gm < M && gk < K) va = *reinterpret_cast<const Chunk16*>(A + gm * lda + gk);
      if (gn < N && gk < K) vb = *reinterpret_cast<const Chunk16*>(Bt + gn * ldb + gk);
      *reinterpret_cast<Chunk16*>(As + row * LDT + kc * EPC) = va;
      *reinterpret_cast<Chunk16*>(Bs + row * LDT + kc * EPC) = vb;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK / KS; ++ks) {
      typename MM::Frag a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = MM::load(As + (wr * 64 + i * 16 + li) * LDT + ks * KS + lg * KP);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = MM::load(Bs + (wc * 64 + j * 16 + li) * LDT + ks * KS + lg * KP);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = MM::run(a[i], b[j], acc[i][j]);
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wr * 64 + i * 16 + lg * 4 + r;
        const int64_t n = n0 + wc * 64 + j * 16 + li;
        if (m < M && n < N) {
          float x = acc[i][j][r];
          if (EPI == kEpiSigmoid) x = sigmoidf(x);
          C[m * ldc + n] = from_f32<T>(x);
        }
      }
}

hipError_t launch_transpose(int dtype, const void* src, void* dst, int rows, int cols,
                            int64_t ld_dst, hipStream_t st) {
  dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  if (dtype == 1)
    transpose_kernel<bf16><<<grid, 256, 0, st>>>((const bf16*)src, (bf16*)dst, rows, cols, ld_dst);
  else
    transpose_kernel<float><<<grid, 256, 0, st>>>((const float*)src, (float*)dst, rows, cols, ld_dst);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(int dtype, int epi, const void* A, const void* Bt, void* C, int M,
                          int N, int K, int64_t lda, int64_t ldb, int64_t ldc, hipStream_t st) {
  const int tiles_m = (M + 127) / 128, tiles_n = (N + 127) / 128;
  const int total = tiles_m * tiles_n;
  if (total == 0) return hipSuccess;
  if (dtype == 1) {
    if (epi == kEpiSigmoid)
      gemm_nt_kernel<bf16, kEpiSigmoid><<<total, 256, 0, st>>>(
          (const bf16*)A, (const bf16*)Bt, (bf16*)C, M, N, K, lda, ldb, ldc, tiles_n, total);
    else
      gemm_nt_kernel<bf16, kEpiStore><<<total, 256, 0, st>>>(
          (const bf16*)A, (const bf16*)Bt, (bf16*)C, M, N, K, lda, ldb, ldc, tiles_n, total);
  } else {
    if (epi == kEpiSigmoid)
      gemm_nt_kernel<float, kEpiSigmoid><<<total, 256, 0, st>>>(
          (const float*)A, (const float*)Bt, (float*)C, M, N, K, lda, ldb, ldc, tiles_n, total);
    else
      gemm_nt_kernel<float, kEpiStore><<<total, 256, 0, st>>>(
          (const float*)A, (const float*)Bt, (float*)C, M, N, K, lda, ldb, ldc, tiles_n, total);
  }
  return hipGetLastError();
}

}  // namespace vdn
