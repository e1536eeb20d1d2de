// Dense contractions of the layer: the two gate GEMMs and the summed output
// projections (10100.com article on Video DeltaNet, 方法概述 part 3: sigmoid
// gates and one output projection per branch, added).
//
// C[m][n] = epi(sum_k A[m][k] * Bt[n][k]) with both operands k-contiguous, so
// MFMA fragments come straight from LDS rows.  Weights arrive as [D_in, D_out]
// and are transposed once per call into the workspace (a few MB).
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

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

// ---------------------------------------------------------------------------
// bf16 GEMM for the layer's large shapes (M = tokens, N and K = D or 2D, K a
// multiple of 32): 256 x 256 output tile per workgroup, eight waves (two
// per SIMD, so one wave's products cover the other's LDS waits and
// barriers) of 128 x 64, 32x32x16 MFMA, 128 accumulator registers per wave.
//
// Each workgroup computes C^T for its tile (the MFMA A operand is a row
// block of Bt, the B operand a row block of A), so a lane holds four
// consecutive n of one m and stores 8 contiguous bytes.  K advances in
// 32-wide slabs (64 bytes per row) through a four-stage LDS ring filled by
// the direct-to-LDS DMA (a buffer load with the lds modifier: lane l writes
// bytes [16 l, 16 l + 16) of a 1 KB block, i.e. 16 rows of one slab); the
// 16-byte chunk c of row r sits at chunk c ^ ((r >> 2) & 3), so the sixteen
// rows a 16-lane group reads for one fragment cover all 64 banks.  Buffer
// descriptors start at the tile's first row and end at the matrix's last, so
// rows past M or N read as zero.  Tiles are visited in groups of eight M
// panels (every N tile of a group before the next group) on top of the XCD
// remap, so the workgroups that run together on one XCD share A panels and
// Bt slices in its L2.
namespace gemm_big {
constexpr int BM = 256, BN = 256, BK = 32, STAGES = 4;
constexpr int ROWB = BK * 2;                 // bytes per row of a slab
constexpr int TILEB = BM * ROWB;             // 16 KB per operand and stage
constexpr int STAGEB = 2 * TILEB;            // A slab, then Bt slab
constexpr int GROUP_M = 8;
constexpr int kWaitVm0 = 0x0F70;             // s_waitcnt vmcnt(0) (gfx9 encoding)
constexpr int kWaitVm8 = 0x0F78;             // s_waitcnt vmcnt(8): all but the last two slabs' loads (4 per slab)
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 2) & 3); }
}  // namespace gemm_big

template <int EPI>
__global__ __launch_bounds__(512) void gemm_bf16_nt_big_kernel(const bf16* __restrict__ A,
                                                               const bf16* __restrict__ Bt,
                                                               bf16* __restrict__ C, int M, int N, int K,
                                                               int64_t lda, int64_t ldb, int64_t ldc,
                                                               int tiles_m, int tiles_n) {
  using namespace gemm_big;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STAGES * STAGEB];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l32 = lane % 32, h = lane / 32;
  const int wm = wave >> 2, wn = wave & 3;   // 128-row block of A, 64-row block of Bt

  // tile of this workgroup: XCD-contiguous logical id, then grouped order
  const int total = tiles_m * tiles_n;
  const int pid = xcd_remap(blockIdx.x, total);
  const int group = pid / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = pid - group * GROUP_M * tiles_n;
  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // buffer descriptors in scalar registers
  const int tm = __builtin_amdgcn_readfirstlane(first_m + in_group % gsize);
  const int tn = __builtin_amdgcn_readfirstlane(in_group / gsize);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  // DMA: wave w fills rows 32 w .. 32 w + 31 of each slab, two 16-row blocks;
  // lane l of block i loads row 32 w + 16 i + l/4, global chunk swz^-1
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + m0 * lda), (short)0, (int)(min((int64_t)BM, M - m0) * lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Bt + n0 * ldb), (short)0, (int)(min((int64_t)BN, N - n0) * ldb * 2), 0x00020000);
  int offa[2], offb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 32 * wave + 16 * i + lane / 4;
    const int c = swz(row, lane % 4);
    offa[i] = (int)(row * lda * 2) + 16 * c;
    offb[i] = (int)(row * ldb * 2) + 16 * c;
  }
  const int nk = K / BK;
  // The DMA is an opaque instruction for the compiler (its wait insertion
  // cannot tell ring stages apart); the loop waits for each slab explicitly.
  auto issue = [&](int kt, int stage) {
    const int lds = (int)(size_t)(__attribute__((address_space(3))) unsigned char*)(ring + stage * STAGEB);
    const int kb = kt * ROWB;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = 2 * wave + i;
      asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(offa[i]), "s"(ra), "s"(kb),
                   "{m0}"(lds + blk * 1024)
                   : "memory");
      asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(offb[i]), "s"(rb), "s"(kb),
                   "{m0}"(lds + TILEB + blk * 1024)
                   : "memory");
    }
  };

  f32x16 acc[2][4];   // acc[jn][im]: C^T block (n: 32 jn.., m: 32 im..) of this wave's 128 x 64
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x16{};

  // fragments of one 16-column step ks of a slab: fb[j] rows 64 wn + 32 j + l32
  // of Bt, fa[i] rows 128 wm + 32 i + l32 of A, chunk 2 ks + h
  auto read_frags = [&](int stage, int ks, bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {
    const unsigned char* sa = ring + stage * STAGEB;
    const unsigned char* sb = sa + TILEB;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rb_row = 64 * wn + 32 * j + l32;
      fb[j] = *reinterpret_cast<const bf16x8*>(sb + rb_row * ROWB + 16 * swz(rb_row, 2 * ks + h));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra_row = 128 * wm + 32 * i + l32;
      fa[i] = *reinterpret_cast<const bf16x8*>(sa + ra_row * ROWB + 16 * swz(ra_row, 2 * ks + h));
    }
  };
  auto products = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[j][i], 0, 0, 0);
  };
  auto fence = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  for (int s = 0; s < 3; ++s)
    if (s < nk) issue(s, s);
  if (nk > 2) __builtin_amdgcn_s_waitcnt(kWaitVm8);
  else __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  // Fragment reads run half a slab ahead of their products: the second
  // step's fragments of slab kt are read at the top of step kt (covered by
  // the first step's products); then each wave waits for its share of slab
  // kt+1, the barrier publishes it (and, being a full barrier, waits for
  // every wave's outstanding LDS reads), and the first step's fragments of
  // slab kt+1 are read beside the second step's products.  A ring slot is
  // refilled (slab kt+3 at the top of step kt) after the barrier of step
  // kt-1, past every read of its previous slab.
  bf16x8 fa0[4], fb0[2], fa1[4], fb1[2];
  read_frags(0, 0, fa0, fb0);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 3 < nk) issue(kt + 3, (kt + 3) % STAGES);
    read_frags(kt % STAGES, 1, fa1, fb1);
    fence();
    products(fa0, fb0);
    fence();
    if (kt + 3 < nk) __builtin_amdgcn_s_waitcnt(kWaitVm8);
    else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (kt + 1 < nk) read_frags((kt + 1) % STAGES, 0, fa0, fb0);
    fence();
    products(fa1, fb1);
  }

  // epilogue: acc[jn][im][4 r4 + e] = C[m0 + 128 wm + 32 im + l32][n0 + 64 wn + 32 jn + 8 r4 + 4 h + e]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + 128 * wm + 32 * i + l32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int64_t n = n0 + 64 * wn + 32 * j + 8 * r4 + 4 * h;
        if (n >= N) continue;
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = acc[j][i][4 * r4 + e];
          if (EPI == kEpiSigmoid) x = sigmoidf(x);
          v[e] = (bf16)x;
        }
        *reinterpret_cast<bf16x4*>(C + m * ldc + n) = v;
      }
  }
}

// Eight waves as above with 64-wide K slabs in a two-stage ring (the same
// 128 KB of LDS): half the barriers per product.  Rows of a slab are 128 bytes
// (eight 16-byte chunks); chunk c of row r sits at c ^ ((r >> 1) & 7), so the
// sixteen rows a 16-lane fragment read touches cover all 64 banks.  Slab
// kt+2 is issued right after the barrier that retires slab kt, so its loads
// have one slab of products to land.
namespace gemm_k64 {
constexpr int BK = 64, ROWB = BK * 2, TILEB = 256 * ROWB, STAGEB = 2 * TILEB;
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }
}  // namespace gemm_k64

template <int EPI>
__global__ __launch_bounds__(512) void gemm_bf16_nt_k64_kernel(const bf16* __restrict__ A,
                                                               const bf16* __restrict__ Bt,
                                                               bf16* __restrict__ C, int M, int N, int K,
                                                               int64_t lda, int64_t ldb, int64_t ldc,
                                                               int tiles_m, int tiles_n) {
  using namespace gemm_k64;
  using gemm_big::BM;
  using gemm_big::BN;
  using gemm_big::GROUP_M;
  using gemm_big::f32x16;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[2 * STAGEB];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l32 = lane % 32, h = lane / 32;
  const int wm = wave >> 2, wn = wave & 3;   // 128-row block of A, 64-row block of Bt

  const int total = tiles_m * tiles_n;
  const int pid = xcd_remap(blockIdx.x, total);
  const int group = pid / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = pid - group * GROUP_M * tiles_n;
  const int tm = __builtin_amdgcn_readfirstlane(first_m + in_group % gsize);
  const int tn = __builtin_amdgcn_readfirstlane(in_group / gsize);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  // DMA: wave w fills rows 32 w .. 32 w + 31 of each slab, four 8-row blocks;
  // lane l of block i loads row 32 w + 8 i + l/8, global chunk swz^-1
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + m0 * lda), (short)0, (int)(min((int64_t)BM, M - m0) * lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Bt + n0 * ldb), (short)0, (int)(min((int64_t)BN, N - n0) * ldb * 2), 0x00020000);
  int offa[4], offb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + lane / 8;
    const int c = swz(row, lane % 8);
    offa[i] = (int)(row * lda * 2) + 16 * c;
    offb[i] = (int)(row * ldb * 2) + 16 * c;
  }
  const int nk = K / BK;
  auto issue = [&](int kt, int stage) {
    const int lds = (int)(size_t)(__attribute__((address_space(3))) unsigned char*)(ring + stage * STAGEB);
    const int kb = kt * ROWB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int blk = 4 * wave + i;
      asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(offa[i]), "s"(ra), "s"(kb),
                   "{m0}"(lds + blk * 1024)
                   : "memory");
      asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(offb[i]), "s"(rb), "s"(kb),
                   "{m0}"(lds + TILEB + blk * 1024)
                   : "memory");
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x16{};

  auto read_frags = [&](int stage, int ks, bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {
    const unsigned char* sa = ring + stage * STAGEB;
    const unsigned char* sb = sa + TILEB;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rb_row = 64 * wn + 32 * j + l32;
      fb[j] = *reinterpret_cast<const bf16x8*>(sb + rb_row * ROWB + 16 * swz(rb_row, 2 * ks + h));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra_row = 128 * wm + 32 * i + l32;
      fa[i] = *reinterpret_cast<const bf16x8*>(sa + ra_row * ROWB + 16 * swz(ra_row, 2 * ks + h));
    }
  };
  auto products = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[j][i], 0, 0, 0);
  };
  auto fence = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 1) __builtin_amdgcn_s_waitcnt(gemm_big::kWaitVm8);
  else __builtin_amdgcn_s_waitcnt(gemm_big::kWaitVm0);
  __syncthreads();

  bf16x8 fa0[4], fb0[2], fa1[4], fb1[2];
  read_frags(0, 0, fa0, fb0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    read_frags(st, 1, fa1, fb1);
    fence();
    products(fa0, fb0);
    fence();
    read_frags(st, 2, fa0, fb0);
    fence();
    products(fa1, fb1);
    fence();
    read_frags(st, 3, fa1, fb1);
    fence();
    products(fa0, fb0);
    fence();
    // slab kt+1 resident, everyone done reading slab kt: its stage takes slab kt+2
    __builtin_amdgcn_s_waitcnt(gemm_big::kWaitVm0);
    __syncthreads();
    if (kt + 2 < nk) issue(kt + 2, st);
    if (kt + 1 < nk) read_frags(st ^ 1, 0, fa0, fb0);
    fence();
    products(fa1, fb1);
  }

  // epilogue: acc[jn][im][4 r4 + e] = C[m0 + 128 wm + 32 im + l32][n0 + 64 wn + 32 jn + 8 r4 + 4 h + e]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + 128 * wm + 32 * i + l32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int64_t n = n0 + 64 * wn + 32 * j + 8 * r4 + 4 * h;
        if (n >= N) continue;
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = acc[j][i][4 * r4 + e];
          if (EPI == kEpiSigmoid) x = sigmoidf(x);
          v[e] = (bf16)x;
        }
        *reinterpret_cast<bf16x4*>(C + m * ldc + n) = v;
      }
  }
}

// bf16, K a multiple of 128: the layer's two projections.  256x256 output
// tile, four waves (one per SIMD) of 128x128, v_mfma_f32_16x16x32_bf16: the
// wave's block is 8 x 8 products of 16 x 16 (256 accumulator registers).  K
// advances in 64-wide slabs through a two-stage LDS ring filled by the
// direct-to-LDS DMA; a slab is two 32-deep steps.  As in the softmax kernel, a
// step is a fixed list of 64 slots, one product each, every instruction its
// own asm statement so that the order holds: the 16 fragment reads of the next
// step go out one every fourth slot (each product waits, with an explicit
// lgkmcnt, for exactly the reads it needs), and the slab after next's 16 DMA
// loads go out every fourth slot of the step after the barrier.  The barrier
// that retires a slab sits between its two steps: the second step's fragments
// were read during the first (in its first 16 slots), so its products run
// while the next slab's first fragments are read and the slab after it streams
// into the freed stage.  The kernel is persistent (one workgroup per compute
// unit): the slab stream runs on from one output tile into the next, so a
// tile's epilogue overlaps the next tile's first loads instead of a fresh
// workgroup's start-up.  A fragment (16 rows x 32 k) is one 16-byte read per
// lane: row l % 16 of the tile, logical chunk 4 ks + l / 16 of the slab row;
// the swizzle's row term, (row >> 1) & 7, is the same for every 16-row tile of
// a lane, so tile t's address is the lane's base plus the constant 2048 t.
// (The same kernel on 32x32x16 products, 16 per 16-deep step, ran 12% slower.)
namespace gemm_s {
constexpr int BM = 256, BN = 256, BK = 64, ROWB = BK * 2;   // 128-byte slab rows
constexpr int TILEB = BM * ROWB;                              // 32 KB per operand and stage
constexpr int BBASE = 2 * TILEB;                              // A slabs of both stages, then Bt slabs
constexpr int GROUP_M = 8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
// chunk c of row r at c ^ ((r >> 1) & 7): the sixteen rows of a 16-lane
// fragment read cover all 64 banks
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }
template <int V>
using IC = std::integral_constant<int, V>;
template <int B, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(IC<B + I>{}), ...);
}
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (E > B) static_for_impl<B>(f, std::make_integer_sequence<int, E - B>{});
}
// Fragment reads of a step, in issue order: Bt tile 0, A tiles 0-7, Bt tiles
// 1-7; read r goes out in slot 4 r of the step before, or in slot r when that
// step is the one before a barrier (early), so that its reads are in when the
// barrier's lgkmcnt(0) comes.  Product (jn, im) is slot 8 jn + im.  The first
// product that uses read r waits until at most (15 - r) reads of its own step
// plus the next step's reads issued before slot s are outstanding, capped at
// 15: a wave has at most 15 LDS operations outstanding, so a larger count is
// only met once the read is in.
constexpr bool first_use(int s) { return s <= 8 || s % 8 == 0; }
constexpr int first_use_read(int s) { return s == 0 ? 1 : s <= 7 ? s + 1 : 8 + s / 8; }
constexpr int reads_before(int s, bool early) { return early ? (s < 16 ? s : 16) : (s + 3) / 4; }
constexpr int first_use_wait(int s, bool early) {
  return 15 - first_use_read(s) + reads_before(s, early) < 15 ? 15 - first_use_read(s) + reads_before(s, early) : 15;
}
static_assert(first_use_wait(0, false) == 14 && first_use_wait(1, false) == 14 && first_use_wait(7, false) == 9 &&
              first_use_wait(8, false) == 8 && first_use_wait(56, false) == 14 && first_use_wait(8, true) == 14 &&
              first_use_wait(56, true) == 15, "lgkmcnt table");
__device__ __forceinline__ void mma(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// the first product of a tile: C operand zero, so no accumulator is cleared
__device__ __forceinline__ void mma_zero(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
}
template <int OFF>
__device__ __forceinline__ void ds_frag(bf16x8& d, int addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
}
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(bf16)lo, (bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}
}  // namespace gemm_s

template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_nt_slot_kernel(const bf16* __restrict__ A,
                                                                const bf16* __restrict__ Bt,
                                                                bf16* __restrict__ C, int M, int N, int K,
                                                                int64_t lda, int64_t ldb, int64_t ldc,
                                                                int tiles_m, int tiles_n) {
  using namespace gemm_s;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[4 * TILEB];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l16 = lane % 16, g = lane / 16;
  const int wm = wave >> 1, wn = wave & 1;   // 128-row block of A, 128-row block of Bt

  const int total = tiles_m * tiles_n, G = gridDim.x;
  auto coords = [&](int l, int& tm, int& tn) {
    const int group = l / (GROUP_M * tiles_n);
    const int first_m = group * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_group = l - group * GROUP_M * tiles_n;
    tm = __builtin_amdgcn_readfirstlane(first_m + in_group % gsize);
    tn = __builtin_amdgcn_readfirstlane(in_group / gsize);
  };
  auto rsrc_a = [&](int tm) {
    const int64_t m0 = (int64_t)tm * BM;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * lda), (short)0,
                                             (int)(min((int64_t)BM, M - m0) * lda * 2), 0x00020000);
  };
  auto rsrc_b = [&](int tn) {
    const int64_t n0 = (int64_t)tn * BN;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(Bt + n0 * ldb), (short)0,
                                             (int)(min((int64_t)BN, N - n0) * ldb * 2), 0x00020000);
  };

  const int lds0 = (int)(size_t)(__attribute__((address_space(3))) unsigned char*)ring;
  int offa[8], offb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 64 * wave + 8 * i + lane / 8;
    const int c = swz(row, lane % 8);
    offa[i] = (int)(row * lda * 2) + 16 * c;
    offb[i] = (int)(row * ldb * 2) + 16 * c;
  }
  auto issue_one = [&](__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int kb, int st, int i) {
    if (i < 8)
      asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(offa[i]), "s"(ra), "s"(kb),
                   "{m0}"(lds0 + st * TILEB + (8 * wave + i) * 1024)
                   : "memory");
    else
      asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(offb[i - 8]), "s"(rb), "s"(kb),
                   "{m0}"(lds0 + BBASE + st * TILEB + (8 * wave + i - 8) * 1024)
                   : "memory");
  };
  // fragment base addresses (stage 0, tile 0) of step ks: row 128 w + l16, chunk 4 ks + g
  int adA[2], adB[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int rA = 128 * wm + l16, rB = 128 * wn + l16;
    adA[ks] = lds0 + rA * ROWB + 16 * swz(rA, 4 * ks + g);
    adB[ks] = lds0 + BBASE + rB * ROWB + 16 * swz(rB, 4 * ks + g);
  }

  int li = xcd_remap(blockIdx.x, G);
  int tm, tn;
  coords(li, tm, tn);
  __amdgpu_buffer_rsrc_t ra = rsrc_a(tm), rb = rsrc_b(tn);
  const int nk = K / BK;   // even
#pragma unroll
  for (int i = 0; i < 16; ++i) issue_one(ra, rb, 0, 0, i);
#pragma unroll
  for (int i = 0; i < 16; ++i) issue_one(ra, rb, ROWB, 1, i);
  __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16): slab 0 landed
  asm volatile("s_barrier" ::: "memory");

  f32x4 acc[8][8];              // [Bt tile jn][A tile im]: C^T tile
  bf16x8 fa[2][8], fb[2][8];    // fragments of two steps: [step parity][tile]
  auto read = [&](auto ST, auto KS, auto P, auto R) {
    constexpr int st = decltype(ST)::value, ks = decltype(KS)::value, p = decltype(P)::value;
    constexpr int r = decltype(R)::value;
    if constexpr (r == 0) ds_frag<st * TILEB>(fb[p][0], adB[ks]);
    else if constexpr (r <= 8) ds_frag<st * TILEB + (r - 1) * 2048>(fa[p][r - 1], adA[ks]);
    else ds_frag<st * TILEB + (r - 8) * 2048>(fb[p][r - 8], adB[ks]);
  };
  static_for<0, 16>([&](auto R) { read(IC<0>{}, IC<0>{}, IC<0>{}, R); });

  for (;;) {
    const int lnext = li + G;
    const bool has_next = lnext < total;
    int ntm = tm, ntn = tn;   // past the last tile: reload this tile's first slabs (never read)
    if (has_next) coords(lnext, ntm, ntn);
    const __amdgpu_buffer_rsrc_t nra = rsrc_a(ntm), nrb = rsrc_b(ntn);

    // one 32-deep step: 64 products on fragment set P, the next step's reads (stage NST,
    // step NKS) into set P ^ 1, and after a barrier the DMA of the slab two ahead
    auto step = [&](auto P, auto NST, auto NKS, auto ZERO, auto DMA, auto EARLY, __amdgpu_buffer_rsrc_t da,
                    __amdgpu_buffer_rsrc_t db, int dkb, int dst) __attribute__((always_inline)) {
      constexpr int p = decltype(P)::value;
      static_for<0, 64>([&](auto S) {
        constexpr int sl = decltype(S)::value, jn = sl / 8, im = sl % 8;
        constexpr bool early = decltype(EARLY)::value;
        if constexpr (first_use(sl)) wait_lgkm<first_use_wait(sl, early)>();
        if constexpr (decltype(ZERO)::value) mma_zero(acc[jn][im], fb[p][jn], fa[p][im]);
        else mma(acc[jn][im], fb[p][jn], fa[p][im]);
        if constexpr (early) {
          if constexpr (sl < 16) read(NST, NKS, IC<1 - p>{}, IC<sl>{});
        } else if constexpr (sl % 4 == 0) {
          read(NST, NKS, IC<1 - p>{}, IC<sl / 4>{});
        }
        if constexpr (decltype(DMA)::value && sl % 4 == 2) issue_one(da, db, dkb, dst, sl / 4);
      });
    };
    // slab kt in stage ST: step 0 (reading step 1's fragments early), the barrier that
    // publishes the next slab and frees stage ST, then step 1 with the next slab's
    // first reads and the DMA of the slab two ahead into stage ST
    auto slab = [&](int kt, auto ST, auto FIRST) __attribute__((always_inline)) {
      constexpr int st = decltype(ST)::value;
      step(IC<0>{}, ST, IC<1>{}, FIRST, IC<0>{}, IC<1>{}, ra, rb, 0, 0);
      const bool wrap = kt + 2 >= nk;
      const int dkb = (wrap ? kt + 2 - nk : kt + 2) * ROWB;
      wait_lgkm<0>();
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the next slab landed
      asm volatile("s_barrier" ::: "memory");
      step(IC<1>{}, IC<1 - st>{}, IC<0>{}, IC<0>{}, IC<1>{}, IC<0>{}, wrap ? nra : ra, wrap ? nrb : rb, dkb, st);
    };
    slab(0, IC<0>{}, IC<1>{});
    slab(1, IC<1>{}, IC<0>{});
    for (int kt = 2; kt < nk; kt += 2) {
      slab(kt, IC<0>{}, IC<0>{});
      slab(kt + 1, IC<1>{}, IC<0>{});
    }
    // the last products' results are read by vector instructions below
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // Epilogue: acc[jn][im][e] = C[m0 + 128 wm + 16 im + l16][n0 + 128 wn + 16 jn + 4 g + e].
    // v_permlane16_swap between the packed values of tiles 2 p and 2 p + 1 leaves
    // the lanes of even g with eight consecutive columns of tile 2 p and those of
    // odd g with eight of tile 2 p + 1: one 16-byte store each.
    {
      const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
      const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(C + m0 * ldc), (short)0, (int)(min((int64_t)BM, M - m0) * ldc * 2), 0x00020000);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 128 * wm + 16 * i + l16;
#pragma unroll
        for (int pj = 0; pj < 4; ++pj) {
          asm volatile("" : "+a"(acc[2 * pj][i]), "+a"(acc[2 * pj + 1][i]));
          unsigned px[2], py[2];
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            float x0 = acc[2 * pj][i][2 * e2], x1 = acc[2 * pj][i][2 * e2 + 1];
            float y0 = acc[2 * pj + 1][i][2 * e2], y1 = acc[2 * pj + 1][i][2 * e2 + 1];
            if (EPI == kEpiSigmoid) {
              x0 = sigmoidf(x0); x1 = sigmoidf(x1);
              y0 = sigmoidf(y0); y1 = sigmoidf(y1);
            }
            px[e2] = pack_bf16x2(x0, x1);
            py[e2] = pack_bf16x2(y0, y1);
          }
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const auto sw = __builtin_amdgcn_permlane16_swap(px[e2], py[e2], false, false);
            px[e2] = sw[0];
            py[e2] = sw[1];
          }
          const int64_t col = n0 + 128 * wn + 16 * (2 * pj + (g & 1)) + 4 * (g & 2);
          const int off = col < N ? (int)((row * ldc + col) * 2) : int(0x80000000u);
          const u32x4 v = {px[0], px[1], py[0], py[1]};
          __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, 0);
        }
      }
    }
    if (!has_next) break;
    li = lnext;
    tm = ntm;
    tn = ntn;
    ra = nra;
    rb = nrb;
  }
  // no load may still write this workgroup's LDS when it ends
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
}

constexpr bool kGemmSlot = true;
constexpr bool kGemmK64 = true;

// the big-tile kernel's shape contract: bf16, K a multiple of 32, N of 8, 16-byte
// aligned rows, and every operand tile's byte range below 2^31
static bool gemm_big_ok(int dtype, int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, const void* A,
                        const void* Bt, const void* C) {
  if (dtype != 1 || M <= 0 || N <= 0 || K <= 0) return false;
  if (K % 32 || N % 8 || lda % 8 || ldb % 8 || ldc % 8) return false;
  if (((uintptr_t)A | (uintptr_t)Bt | (uintptr_t)C) & 15) return false;
  if (256 * lda * 2 >= (int64_t(1) << 31) || 256 * ldb * 2 >= (int64_t(1) << 31)) return false;
  return true;
}

// compute units of the current device, looked up once per device (threads
// that race on the first lookup store the same value)
static int compute_units() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (!n) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
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
  if (gemm_big_ok(dtype, M, N, K, lda, ldb, ldc, A, Bt, C)) {
    const int tm = (M + 255) / 256, tn = (N + 255) / 256;
    if (kGemmSlot && K % 128 == 0 && 256 * ldc * 2 < (int64_t(1) << 31)) {
      // persistent: one workgroup per compute unit (its 128 KB of LDS allows no second)
      const int grid = std::min(tm * tn, compute_units());
      if (epi == kEpiSigmoid)
        gemm_bf16_nt_slot_kernel<kEpiSigmoid><<<grid, 256, 0, st>>>(
            (const bf16*)A, (const bf16*)Bt, (bf16*)C, M, N, K, lda, ldb, ldc, tm, tn);
      else
        gemm_bf16_nt_slot_kernel<kEpiStore><<<grid, 256, 0, st>>>(
            (const bf16*)A, (const bf16*)Bt, (bf16*)C, M, N, K, lda, ldb, ldc, tm, tn);
    } else if (kGemmK64 && K % 64 == 0) {
      if (epi == kEpiSigmoid)
        gemm_bf16_nt_k64_kernel<kEpiSigmoid><<<tm * tn, 512, 0, st>>>(
            (const bf16*)A, (const bf16*)Bt, (bf16*)C, M, N, K, lda, ldb, ldc, tm, tn);
      else
        gemm_bf16_nt_k64_kernel<kEpiStore><<<tm * tn, 512, 0, st>>>(
            (const bf16*)A, (const bf16*)Bt, (bf16*)C, M, N, K, lda, ldb, ldc, tm, tn);
    } else {
      if (epi == kEpiSigmoid)
        gemm_bf16_nt_big_kernel<kEpiSigmoid><<<tm * tn, 512, 0, st>>>(
            (const bf16*)A, (const bf16*)Bt, (bf16*)C, M, N, K, lda, ldb, ldc, tm, tn);
      else
        gemm_bf16_nt_big_kernel<kEpiStore><<<tm * tn, 512, 0, st>>>(
            (const bf16*)A, (const bf16*)Bt, (bf16*)C, M, N, K, lda, ldb, ldc, tm, tn);
    }
    return hipGetLastError();
  }
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
