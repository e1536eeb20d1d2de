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
//   solve   : per (frame, head) M_t = (I + A_t)^-1 by Gauss-Jordan elimination
//             with the columns in registers                    (latency)
//   scan    : S_t = (gamma_t S_prev + B_t) M_t, both directions (T-step chain)
//   readout : u = S_t q both directions, RMSNorm, sum, gate     (MFMA, HBM-bound)
#include <math.h>

#include <utility>

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
                                                       float* __restrict__ Bm, int T_, int N, int Lt) {
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
  const int64_t row0 = (f / T_) * Lt + (f % T_) * N;   // first token row of frame f
  const T* kf = k + row0 * D;
  const T* vf = v + row0 * D;
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

  // the thread's 16-byte chunks of a stage (chunk c = tid + 256 i: token row c % NC,
  // column chunk c / NC); the next stage's are loaded while this stage is multiplied
  constexpr int CH = (NC * CPR + 255) / 256;
  Chunk16 kk[CH], vv[CH];
  auto load_stage = [&](int n0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i, row = c % NC, cc = c / NC;
      kk[i] = vv[i] = zero_chunk();
      if (c < NC * CPR && n0 + row < N) {
        kk[i] = *reinterpret_cast<const Chunk16*>(kf + (int64_t)(n0 + row) * D + cc * EPC);
        vv[i] = *reinterpret_cast<const Chunk16*>(vf + (int64_t)(n0 + row) * D + cc * EPC);
      }
    }
  };
  load_stage(0);

  for (int n0 = 0; n0 < N; n0 += NC) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i, row = c % NC, cc = c / NC;
      if (c < NC * CPR) {
        const T* ke = reinterpret_cast<const T*>(&kk[i]);
        const T* ve = reinterpret_cast<const T*>(&vv[i]);
#pragma unroll
        for (int x = 0; x < EPC; ++x) {
          Sm[(cc * EPC + x) * LDT + row] = ke[x];
          Sm[D * LDT + (cc * EPC + x) * LDT + row] = ve[x];
        }
      }
    }
    if (n0 + NC < N) load_stage(n0 + NC);
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
// gram, bf16, head_dim 64 and 128 (described at 128).  One workgroup of four
// waves per (frame, head); K_t and V_t stream through a four-stage LDS ring of
// 64-token tiles by the direct-to-LDS DMA path (a buffer load with the lds
// modifier), row-major with XOR-swizzled 16-byte chunks; token rows past N
// read as zero.  Wave w consumes token rows 16w .. 16w+15 of every tile.  A
// ds_read_b64_tr_b16 pair hands each lane eight tokens of one dimension: that
// register is the A operand (row = dimension) and equally the B operand
// (column = dimension) of a 32x32x16 MFMA, so K^T K and V^T K need no other
// data movement.  Each wave accumulates the 10 upper 32x32 tiles of K^T K and
// the 16 tiles of V^T K over its quarter of the tokens (416 fp32 per lane);
// the four partial sums are added through LDS at the end, scaled by beta_t,
// and A's off-diagonal tiles are mirrored.  At head_dim 64 the same holds
// with 3 + 4 tiles and 128-byte rows.
namespace gr {
constexpr int BN = 64, STAGES = 4;
constexpr int kWaitVm0 = 0x0F70;             // s_waitcnt vmcnt(0)
template <int D>
struct Geo {
  static constexpr int ROWB = D * 2, TILEB = BN * ROWB, STAGEB = 2 * TILEB;
  static constexpr int NT = D / 32;                       // 32-wide blocks per dimension
  static constexpr int NA = NT * (NT + 1) / 2, NTILE = NA + NT * NT;   // upper A tiles, then B tiles
  static constexpr int BPW = TILEB / 1024 / 4;            // 1 KB DMA blocks per wave and tensor
  static constexpr int RPB = 1024 / ROWB;                 // token rows per DMA block
  static constexpr int CPR = ROWB / 16;                   // 16-byte chunks per row
  // tiles per reduction batch: 4 waves x TB tiles x 16 x 65 floats fit the ring
  static constexpr int TB = STAGES * STAGEB / (4 * 16 * 65 * 4);
  // s_waitcnt vmcnt(n) with n = one or two tiles' loads outstanding
  static constexpr int kWaitOne = 0x0F70 | (2 * BPW);
  static constexpr int kWaitTwo = 0x0F70 | ((4 * BPW) & 15) | (((4 * BPW) >> 4) << 14);
};
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
// Physical chunk of logical 16-byte chunk c of row r.  256-byte rows: 8 rows x
// 4 chunks of a transpose read touch every bank exactly twice.  128-byte rows:
// the 4 rows x 4 chunks of each half-wave cover the 64 banks once (rows r and
// r + 2 share banks, so bit 1 of the row flips the chunk's upper half).
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128) return c ^ (((r & 7) << 1) | ((r >> 3) & 1));
  else return c ^ (((r >> 1) & 1) << 2);
}
// (tile row block, tile column block) of output tile u: the upper tiles of
// A row by row, then the tiles of B row by row
// (branch-free: row r of the upper tiles starts at tile r NT - r (r - 1) / 2)
__device__ __forceinline__ constexpr int upper_start(int nt, int r) { return r * nt - r * (r - 1) / 2; }
template <int D>
__device__ __forceinline__ constexpr int tile_i(int u) {
  constexpr int NT = Geo<D>::NT, NA = Geo<D>::NA;
  int i = 0;
  for (int r = 1; r < NT; ++r) i += u >= upper_start(NT, r) ? 1 : 0;
  return u >= NA ? (u - NA) / NT : i;
}
template <int D>
__device__ __forceinline__ constexpr int tile_j(int u) {
  constexpr int NT = Geo<D>::NT, NA = Geo<D>::NA;
  const int i = tile_i<D>(u);
  return u >= NA ? (u - NA) % NT : i + u - upper_start(NT, i);
}
static_assert(tile_i<128>(9) == 3 && tile_j<128>(9) == 3 && tile_i<128>(5) == 1 && tile_j<128>(5) == 2 &&
                  tile_i<128>(25) == 3 && tile_j<128>(25) == 3 && tile_i<64>(1) == 0 && tile_j<64>(1) == 1 &&
                  tile_i<64>(2) == 1 && tile_j<64>(2) == 1 && tile_i<64>(5) == 1 && tile_j<64>(5) == 0,
              "tile enumeration");
static_assert(Geo<128>::TB == 7 && Geo<64>::TB == 3, "reduction batches fit the ring");
static_assert(Geo<128>::kWaitOne == 0x0F78 && Geo<128>::kWaitTwo == 0x4F70 && Geo<64>::kWaitOne == 0x0F74 &&
                  Geo<64>::kWaitTwo == 0x0F78,
              "vmcnt encodings");
// f(integral_constant<int, U>) for U = 0 .. sizeof...(U) - 1, each a compile-time constant
template <typename F, int... U>
__device__ __forceinline__ void for_each_tile(F&& f, std::integer_sequence<int, U...>) {
  (f(std::integral_constant<int, U>{}), ...);
}
// Accumulating products with the accumulator's register file fixed: the
// K^T K tiles in vector registers, the V^T K tiles in accumulator registers
// (416 fp32 per lane at head_dim 128 do not fit one file; left to itself the
// compiler shuttles tiles between the files around every product).
// The first product of a tile starts from zero, so the accumulators need no
// initialisation (and no vector-write -> matrix-read wait states).
__device__ __forceinline__ void mma_v(f32x16& d, bf16x8 a, bf16x8 b, bool first) {
  if (first) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_a(f32x16& d, bf16x8 a, bf16x8 b, bool first) {
  if (first) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&a"(d) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
}  // namespace gr

template <int D>
__global__ __launch_bounds__(256) void vda_gram_bf16_kernel(const bf16* __restrict__ k,
                                                            const bf16* __restrict__ v,
                                                            const float* __restrict__ beta,
                                                            float* __restrict__ A,
                                                            float* __restrict__ Bm, int T_, int N, int Lt) {
  using namespace gr;
  using G = Geo<D>;
  constexpr int ROWB = G::ROWB, TILEB = G::TILEB, STAGEB = G::STAGEB, NT = G::NT, NA = G::NA,
                NTILE = G::NTILE, BPW = G::BPW, TB = G::TB;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STAGES * STAGEB];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int g = lane / 16, j16 = lane % 16;
  const int64_t f = blockIdx.x;
  const int64_t row0 = (f / T_) * Lt + (f % T_) * N;   // first token row of frame f
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k + row0 * D), (short)0, N * ROWB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v + row0 * D), (short)0, N * ROWB, 0x00020000);

  // DMA: lane l of block b fills physical chunk l % CPR of tile row RPB b + l / CPR
  int lane_off[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int row = (wave * BPW + i) * G::RPB + lane / G::CPR;
    lane_off[i] = row * ROWB + swz<D>(row, lane % G::CPR) * 16;
  }
  const int ntiles = (N + BN - 1) / BN;
  auto issue = [&](int t) {
    const int lds = (int)(size_t)(__attribute__((address_space(3))) unsigned char*)(ring + (t & 3) * STAGEB);
    const int base = t * BN * ROWB;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave * BPW + i;
      const int voff = base + lane_off[i];
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rk), "{m0}"(lds + blk * 1024)
                   : "memory");
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rv),
                   "{m0}"(lds + TILEB + blk * 1024)
                   : "memory");
    }
  };
  // transpose-read offsets inside a tile: tokens 16 wave + 4 (g/2) + {0..3} and
  // {8..11}, dimension 32 dt + 16 (g%2) + j16
  int offA[NT], offB[NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) {
    const int rowA = 16 * wave + 4 * (g >> 1) + (j16 >> 2), rowB = rowA + 8;
    const int dcol = dt * 32 + 16 * (g & 1) + 4 * (j16 & 3);
    const int cch = dcol >> 3, off = (dcol & 7) * 2;
    offA[dt] = rowA * ROWB + swz<D>(rowA, cch) * 16 + off;
    offB[dt] = rowB * ROWB + swz<D>(rowB, cch) * 16 + off;
  }
  auto frag = [&](const unsigned char* base, int dt) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + offA[dt]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + offB[dt]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 accA[NA], accB[NTILE - NA];     // set by the first tile's products (N >= 1)

  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  if (ntiles > 2) issue(2);
  for (int t = 0; t < ntiles; ++t) {
    if (t + 2 < ntiles) __builtin_amdgcn_s_waitcnt(G::kWaitTwo);
    else if (t + 1 < ntiles) __builtin_amdgcn_s_waitcnt(G::kWaitOne);
    else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();                       // tile t visible; tile t-1's stage free
    if (t + 3 < ntiles) issue(t + 3);
    const unsigned char* sb = ring + (t & 3) * STAGEB;
    bf16x8 kf[NT], vf[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      kf[dt] = frag(sb, dt);
      vf[dt] = frag(sb + TILEB, dt);
    }
    const bool first = t == 0;
    for_each_tile(
        [&](auto U) {
          constexpr int u = decltype(U)::value, ti = tile_i<D>(u), tj = tile_j<D>(u);
          if constexpr (u < NA) mma_v(accA[u], kf[ti], kf[tj], first);
          else mma_a(accB[u - NA], vf[ti], kf[tj], first);
        },
        std::make_integer_sequence<int, NTILE>{});
  }
  // the last products' results are read by vector instructions below: wait
  // out the matrix pipeline (fenced so that no read is scheduled above it)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);

  // cross-wave sum through the (drained) ring: P[wave][tile][r][lane], rows padded to 65
  float* P = reinterpret_cast<float*>(ring);
  const float bt = beta[f];
  float* Af = A + f * D * D;
  float* Bf = Bm + f * D * D;
#pragma unroll
  for (int b0 = 0; b0 < NTILE; b0 += TB) {
    const int nb = NTILE - b0 < TB ? NTILE - b0 : TB;
    __syncthreads();
#pragma unroll
    for (int uu = 0; uu < TB; ++uu)
      if (uu < nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          P[((wave * TB + uu) * 16 + r) * 65 + lane] = b0 + uu < NA ? accA[b0 + uu][r] : accB[b0 + uu - NA][r];
    __syncthreads();
    for (int e = tid; e < nb * 1024; e += 256) {
      const int uu = e >> 10, u = b0 + uu, w = e & 1023, row = w >> 5, col = w & 31;
      const int ti = tile_i<D>(u), tj = tile_j<D>(u);
      auto sum4 = [&](int rr, int cc) {
        const int r = (rr >> 3) * 4 + (rr & 3), ln = cc + 32 * ((rr >> 2) & 1);
        float s = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) s += P[((wv * TB + uu) * 16 + r) * 65 + ln];
        return s;
      };
      if (u < NA) {
        Af[(ti * 32 + row) * D + tj * 32 + col] = bt * sum4(row, col);
        if (ti != tj) Af[(tj * 32 + row) * D + ti * 32 + col] = bt * sum4(col, row);
      } else {
        Bf[(ti * 32 + row) * D + tj * 32 + col] = bt * sum4(row, col);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// solve: one workgroup of 2d threads per (frame, head).  M_t = (I + A_t)^-1 by
// Gauss-Jordan elimination of the augmented [I + A_t | I]: thread c keeps
// column c in registers and every column is updated with a rank-1 step per
// pivot.  I + A_t is symmetric positive definite (beta >= 0, eigenvalues
// >= 1), for which elimination without pivoting is stable, and that symmetry
// also delivers the pivot column from the pivot row: after k steps the
// not yet eliminated block of the left half is a Schur complement of I + A_t,
// itself symmetric, so column k holds row k's left-half entries in rows >= k;
// and in rows i < k it holds minus row k's right-half entry i (the upper
// part of the left half is (I+A)_{<k,<k}^-1 (I+A)_{<k,k}, the lower part of the
// right half -(I+A)_{k,<k} (I+A)_{<k,<k}^-1, transposes of each other).  So every
// thread writes only its own pivot-row entry to LDS (right half negated), at
// the rotated position (c - k) mod 2d, and slots 0 .. d-1 of that buffer are
// the pivot column in the rotated row order each thread keeps (one barrier
// per step, double-buffered).  Columns of the left half that were already
// eliminated are never read again and are not stored.
// AM holds A_t on entry and M_t^T on exit (row j = column j of M_t, so the
// scan reads contiguous runs of a column).
template <int D>
__global__ __launch_bounds__(2 * D) __attribute__((amdgpu_waves_per_eu(3))) void vda_solve_kernel(float* __restrict__ AM) {
  __shared__ __attribute__((aligned(16))) float rowb[2][2 * D];
  const int64_t f = blockIdx.x;
  float* am = AM + f * D * D;
  const int c = threadIdx.x;

  // Every thread loads column c mod D and the right half multiplies it by 0,
  // so the D loads carry no branch and are all in flight before the first
  // wait.  Column c of [I + A | I] is keep * A[:, c mod D] + e_(c mod D).
  float a[D];
  const int cl = c & (D - 1);
  const float keep = c < D ? 1.f : 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) a[i] = am[i * D + cl];
#pragma unroll
  for (int i = 0; i < D; ++i) a[i] = fmaf(a[i], keep, i == cl ? 1.f : 0.f);
  __syncthreads();   // every column is read before any thread overwrites AM below

  // The rows rotate by one per step, so that the pivot row is always a[0]
  // (all register indices stay compile-time constants): the update writes
  // row i+1 into slot i and the normalised pivot row goes to slot D-1.  After
  // D steps every row is back in its place.
  // Each thread publishes its next pivot-row entry as soon as it is formed
  // (the first update of the step), so that the LDS write's latency runs
  // beside the rest of the step's products; the other buffer was last read
  // before this step's barrier.
  const float sgn = c < D ? 1.f : -1.f;
  rowb[0][c] = sgn * a[0];
  for (int k = 0; k < D; ++k) {
    const int buf = k & 1;
    __syncthreads();
    const float4* rb = reinterpret_cast<const float4*>(rowb[buf]);
    float* next = rowb[buf ^ 1];
    const int nslot = (c - k - 1) & (2 * D - 1);
    float x;
    if constexpr (D <= 64) {
      // all D/4 reads of the pivot column issued before the products use them
      // (one frame-head system per workgroup is latency-bound at this size)
      float4 cv[D / 4];
#pragma unroll
      for (int j = 0; j < D / 4; ++j) cv[j] = rb[j];
      x = a[0] / cv[0].x;
      a[0] = a[1] - cv[0].y * x;
      if (k + 1 < D) next[nslot] = sgn * a[0];
      a[1] = a[2] - cv[0].z * x;
      a[2] = a[3] - cv[0].w * x;
#pragma unroll
      for (int j = 1; j < D / 4; ++j) {
        const int i = 4 * j;
        a[i - 1] = a[i] - cv[j].x * x;
        a[i] = a[i + 1] - cv[j].y * x;
        a[i + 1] = a[i + 2] - cv[j].z * x;
        a[i + 2] = a[i + 3] - cv[j].w * x;
      }
      __builtin_amdgcn_sched_group_barrier(0x100, D / 4, 0);   // the reads first
      __builtin_amdgcn_sched_group_barrier(0x2, 12, 0);        // the division and the first update
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);       // its publication
      __builtin_amdgcn_sched_group_barrier(0x2, D + 16, 0);    // then the rest of the vector work
    } else {
      // at head_dim 128 the compiler's own interleave keeps 3 workgroups per
      // CU (more reads in flight cost occupancy and measured slower)
      x = a[0] / rowb[buf][0];
      {
        const float4 cv = rb[0];
        a[0] = a[1] - cv.y * x;
        if (k + 1 < D) next[nslot] = sgn * a[0];
        a[1] = a[2] - cv.z * x;
        a[2] = a[3] - cv.w * x;
      }
#pragma unroll
      for (int j = 1; j < D / 4; ++j) {
        const int i = 4 * j;
        const float4 cv = rb[j];
        a[i - 1] = a[i] - cv.x * x;
        a[i] = a[i + 1] - cv.y * x;
        a[i + 1] = a[i + 2] - cv.z * x;
        a[i + 2] = a[i + 3] - cv.w * x;
      }
    }
    a[D - 1] = x;
  }

  // thread D + j now holds column j of M = (I + A)^-1: store it as row j
  if (c >= D) {
    float* dst = am + (int64_t)(c - D) * D;
#pragma unroll
    for (int i = 0; i < D; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(a[i], a[i + 1], a[i + 2], a[i + 3]);
  }
}

// ---------------------------------------------------------------------------
// scan: S_t = (gamma_t S_{t-1} + B_t) M_t with S = 0 before the first frame,
// forward (t ascending) and backward (t descending).  Rows of S are
// independent given M_t, so each workgroup owns R rows of one (batch, head,
// direction) and walks the T frames, staging M_t in LDS (transposed back
// from the solve's M^T).  Writes every S_t in fp32 and, when `split` is
// non-null, also as an unevaluated bf16 pair hi + lo (hi = bf16(S), lo =
// bf16(S - hi)) for the bf16 readout, laid out [dir][frame][hi|lo][d][d].
// This is the path for head_dim 32; head_dim 64 and 128 use the MFMA kernel
// below.
template <int D, int R>
__global__ __launch_bounds__(256) void vda_scan_kernel(const float* __restrict__ Mt,
                                                       const float* __restrict__ Bm,
                                                       const float* __restrict__ gamma,
                                                       float* __restrict__ states,
                                                       bf16* __restrict__ split, int T,
                                                       int64_t bhtdd) {
  constexpr int TPR = 256 / R;     // threads per state row
  constexpr int CPT = D / TPR;     // columns per thread
  constexpr int LDM = D + 1;
  __shared__ float Ms[D * LDM];
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
    const float* mt = Mt + fi * D * D;
    const int64_t off = fi * D * D + (int64_t)(r0 + row) * D + col0;
    const float g = gamma[fi];
    __syncthreads();
    // Ms[q][c] = M_t[q][c] = Mt[c][q]
    for (int e = tid; e < D * D; e += 256) Ms[(e % D) * LDM + e / D] = mt[e];
    // X = gamma S_{t-1} + B_t, in place
#pragma unroll
    for (int c = 0; c < CPT; ++c) Ss[row * LDM + col0 + c] = g * Ss[row * LDM + col0 + c] + Bm[off + c];
    __syncthreads();
    float acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
    for (int q = 0; q < D; ++q) {
      const float xv = Ss[row * LDM + q];
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[c] += xv * Ms[q * LDM + col0 + c];
    }
    float* srow = states + dir * bhtdd + off;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const float nv = acc[c];
      Ss[row * LDM + col0 + c] = nv;
      srow[c] = nv;
      if (split) {
        const bf16 hi = (bf16)nv;
        const bf16 lo = (bf16)(nv - (float)hi);
        bf16* sp = split + (dir * bhtdd + fi * D * D) * 2 + (int64_t)(r0 + row) * D + col0 + c;
        sp[0] = hi;
        sp[D * D] = lo;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// scan on fp32 MFMA (instantiated for head_dim 128; head_dim 64 takes the
// 16-row kernel below).  One workgroup of D / 32 waves
// per 32 state rows of one (batch, head, direction); wave w produces columns
// 32w .. 32w+31 of those rows with D / 2 v_mfma_f32_32x32x2_f32 per frame:
// S_t = X_t M_t with
// X_t = gamma_t S_{t-1} + B_t held in LDS.  The contraction index runs through
// the products in the order k = 8i + 4h + c (i the product group, h the lane
// half, c the component), so the A operand is one 16-byte LDS read per group
// and the B operand (row 32w + l%32 of M_t^T) comes from 16-byte loads in
// which the two lane halves read adjacent bytes of each row.  After the
// products the workgroup puts S_t in LDS (double-buffered against X_t) and
// every thread takes four 16-byte chunks of it: it stores S_t (fp32 and/or
// the hi/lo bf16 pair) with whole-row coalesced stores and overwrites each
// chunk with X_{t+1} = gamma_{t+1} S_t + B_{t+1}.  M_{t+1}^T is loaded one
// frame ahead, B two frames ahead, each B element once per workgroup.  The
// 2 D / 32 workgroups of one (batch, head) share an XCD, so each M_t comes
// from HBM once per direction.  kStates / kSplit: S_t is written to `states`
// (fp32) / to `split` (hi/lo bf16).
namespace sc {
constexpr int R = 32;
typedef float f32x16 __attribute__((ext_vector_type(16)));
}  // namespace sc

template <int D, bool kStates, bool kSplit>
__global__ __launch_bounds__(2 * D) void vda_scan_mfma_kernel(const float* __restrict__ Mt,
                                                            const float* __restrict__ Bm,
                                                            const float* __restrict__ gamma,
                                                            float* __restrict__ states,
                                                            bf16* __restrict__ split, int T,
                                                            int64_t bhtdd, int total) {
  using namespace sc;
  constexpr int LD = D + 4, NRB = D / R, KG = D / 8;   // LDS row stride, row blocks, product groups
  __shared__ __attribute__((aligned(16))) float P[2][R * LD];   // X_t and S_t, rows r0 .. r0+31
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int l32 = lane % 32, h = lane / 32;
  const int lid = xcd_remap(blockIdx.x, total);
  const int dir = lid & 1, rb = (lid >> 1) % NRB;
  const int64_t bh = lid / (2 * NRB);
  const int r0 = rb * R, n0 = wave * 32;
  // the thread's chunks (2 D threads, a chunk is 4 floats of a row): rows
  // crow + 8j (j = 0..3), columns ccol .. ccol+3
  const int crow = tid / (D / 4), ccol = 4 * (tid % (D / 4));

  // frame index of scan step `step`, clamped to the last step (loads past the
  // end re-read the last frame and are not used)
  auto fidx = [&](int step) -> int64_t {
    const int c = step < T ? step : T - 1;
    return bh * T + (dir ? T - 1 - c : c);
  };
  auto load_m = [&](float4 (&m)[KG], int step) {
    const float* mp = Mt + fidx(step) * D * D + (int64_t)(n0 + l32) * D + 4 * h;
#pragma unroll
    for (int i = 0; i < KG; ++i) m[i] = *reinterpret_cast<const float4*>(mp + 8 * i);
  };
  auto load_b = [&](float4 (&b)[4], int step) {
    const float* bp = Bm + fidx(step) * D * D + (int64_t)(r0 + crow) * D + ccol;
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const float4*>(bp + 8 * j * D);
  };

  // one frame step: mc = M_s^T, mn <- M_{s+1}^T, bl <- B_{s+2}, be = B_{s+1};
  // X_s in X, S_s and then X_{s+1} go to Y
  auto step = [&](int s, float4 (&mc)[KG], float4 (&mn)[KG], float4 (&bl)[4], const float4 (&be)[4],
                  const float* X, float* Y) {
    const int64_t fi = fidx(s);
    const float gn = gamma[fidx(s + 1)];
    load_m(mn, s + 1);
    load_b(bl, s + 2);
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
    // acc[r] = S_s[r0 + 8 (r/4) + 4h + r%4][n0 + l32]
#pragma unroll
    for (int r = 0; r < 16; ++r) Y[(8 * (r / 4) + 4 * h + r % 4) * LD + n0 + l32] = acc[r];
    __syncthreads();   // S_s complete in Y
    const int64_t off = fi * D * D + (int64_t)(r0 + crow) * D + ccol;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float* yp = Y + (crow + 8 * j) * LD + ccol;
      const float4 sv = *reinterpret_cast<const float4*>(yp);
      if constexpr (kStates) *reinterpret_cast<float4*>(states + dir * bhtdd + off + 8 * j * D) = sv;
      if constexpr (kSplit) {
        bf16x4 hi, lo;
        hi[0] = (bf16)sv.x; hi[1] = (bf16)sv.y; hi[2] = (bf16)sv.z; hi[3] = (bf16)sv.w;
        lo[0] = (bf16)(sv.x - (float)hi[0]);
        lo[1] = (bf16)(sv.y - (float)hi[1]);
        lo[2] = (bf16)(sv.z - (float)hi[2]);
        lo[3] = (bf16)(sv.w - (float)hi[3]);
        bf16* sp = split + dir * bhtdd * 2 + fi * D * D * 2 + (int64_t)(r0 + crow + 8 * j) * D + ccol;
        *reinterpret_cast<bf16x4*>(sp) = hi;
        *reinterpret_cast<bf16x4*>(sp + D * D) = lo;
      }
      // (after the last frame this X is formed from clamped loads and never read)
      float4 xn;
      xn.x = gn * sv.x + be[j].x;
      xn.y = gn * sv.y + be[j].y;
      xn.z = gn * sv.z + be[j].z;
      xn.w = gn * sv.w + be[j].w;
      *reinterpret_cast<float4*>(yp) = xn;
    }
    __syncthreads();   // X_{s+1} complete in Y
  };

  float4 m0[KG], m1[KG], b0[4], b1[4];
  load_m(m0, 0);
  load_b(b0, 0);
  load_b(b1, 1);
#pragma unroll
  for (int j = 0; j < 4; ++j)   // X_0 = B_0 (S_{-1} = 0)
    *reinterpret_cast<float4*>(&P[0][(crow + 8 * j) * LD + ccol]) = b0[j];
  __syncthreads();
  int s = 0;
  for (; s + 1 < T; s += 2) {
    step(s, m0, m1, b0, b1, P[0], P[1]);
    step(s + 1, m1, m0, b1, b0, P[1], P[0]);
  }
  if (s < T) step(s, m0, m1, b0, b1, P[0], P[1]);
}

// The same scan with 16 state rows per workgroup on v_mfma_f32_16x16x4f32 (the
// head_dim 64 path): D/16 waves, wave w forming the 16 x 16 block of columns
// 16w.. of S_s = X_s M_s (D/4 products of 32 cycles instead of D/2 of 64), so a
// frame step's products are a quarter of the 32-row kernel's per wave, and twice
// as many workgroups share the chip.  Lane group g = l / 16 takes
// k = 16 g .. 16 g + 15 over the D/4 products: its X row and M_s^T row
// fragments are four 16-byte reads each.  The epilogue gives every thread one
// 16-byte chunk of the 16 rows.
namespace sc16 {
constexpr int R = 16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
}  // namespace sc16

template <int D, bool kStates, bool kSplit>
__global__ __launch_bounds__(4 * D) void vda_scan_mfma16_kernel(const float* __restrict__ Mt,
                                                              const float* __restrict__ Bm,
                                                              const float* __restrict__ gamma,
                                                              float* __restrict__ states,
                                                              bf16* __restrict__ split, int T,
                                                              int64_t bhtdd, int total) {
  using namespace sc16;
  constexpr int LD = D + 4, NRB = D / R, KQ = D / 16;   // LDS row stride, row blocks, 4-k groups per lane
  __shared__ __attribute__((aligned(16))) float P[2][R * LD];   // X_t and S_t, rows r0 .. r0+15
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int l16 = lane % 16, g = lane / 16;
  const int lid = xcd_remap(blockIdx.x, total);
  const int dir = lid & 1, rb = (lid >> 1) % NRB;
  const int64_t bh = lid / (2 * NRB);
  const int r0 = rb * R, n0 = wave * 16;
  const int crow = tid / (D / 4), ccol = 4 * (tid % (D / 4));   // the thread's chunk

  auto fidx = [&](int step) -> int64_t {
    const int c = step < T ? step : T - 1;
    return bh * T + (dir ? T - 1 - c : c);
  };
  // M_s^T row n0 + l16, columns 16 g .. 16 g + 15 (k of this lane group)
  auto load_m = [&](float4 (&m)[KQ], int step) {
    const float* mp = Mt + fidx(step) * D * D + (int64_t)(n0 + l16) * D + (D / 4) * g;
#pragma unroll
    for (int i = 0; i < KQ; ++i) m[i] = *reinterpret_cast<const float4*>(mp + 4 * i);
  };
  auto load_b = [&](float4& b, int step) {
    b = *reinterpret_cast<const float4*>(Bm + fidx(step) * D * D + (int64_t)(r0 + crow) * D + ccol);
  };

  // one frame step: mc = M_s^T, mn <- M_{s+1}^T, bl <- B_{s+2}, be = B_{s+1};
  // X_s in X, S_s and then X_{s+1} go to Y
  auto step = [&](int s, float4 (&mc)[KQ], float4 (&mn)[KQ], float4& bl, const float4& be, const float* X,
                  float* Y) {
    const int64_t fi = fidx(s);
    const float gn = gamma[fidx(s + 1)];
    load_m(mn, s + 1);
    load_b(bl, s + 2);
    __builtin_amdgcn_sched_barrier(0);   // the next frames' loads go out before this frame's products
    const float* xrow = X + l16 * LD + (D / 4) * g;
    float4 xv[KQ];
#pragma unroll
    for (int i = 0; i < KQ; ++i) xv[i] = *reinterpret_cast<const float4*>(xrow + 4 * i);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i].x, mc[i].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i].y, mc[i].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i].z, mc[i].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i].w, mc[i].w, acc, 0, 0, 0);
    }
    // acc[e] = S_s[r0 + 4 g + e][n0 + l16]
#pragma unroll
    for (int e = 0; e < 4; ++e) Y[(4 * g + e) * LD + n0 + l16] = acc[e];
    __syncthreads();   // S_s complete in Y
    float* yp = Y + crow * LD + ccol;
    const float4 sv = *reinterpret_cast<const float4*>(yp);
    const int64_t off = fi * D * D + (int64_t)(r0 + crow) * D + ccol;
    if constexpr (kStates) *reinterpret_cast<float4*>(states + dir * bhtdd + off) = sv;
    if constexpr (kSplit) {
      bf16x4 hi, lo;
      hi[0] = (bf16)sv.x; hi[1] = (bf16)sv.y; hi[2] = (bf16)sv.z; hi[3] = (bf16)sv.w;
      lo[0] = (bf16)(sv.x - (float)hi[0]);
      lo[1] = (bf16)(sv.y - (float)hi[1]);
      lo[2] = (bf16)(sv.z - (float)hi[2]);
      lo[3] = (bf16)(sv.w - (float)hi[3]);
      bf16* sp = split + dir * bhtdd * 2 + fi * D * D * 2 + (int64_t)(r0 + crow) * D + ccol;
      *reinterpret_cast<bf16x4*>(sp) = hi;
      *reinterpret_cast<bf16x4*>(sp + D * D) = lo;
    }
    // (after the last frame this X is formed from clamped loads and never read)
    float4 xn;
    xn.x = gn * sv.x + be.x;
    xn.y = gn * sv.y + be.y;
    xn.z = gn * sv.z + be.z;
    xn.w = gn * sv.w + be.w;
    *reinterpret_cast<float4*>(yp) = xn;
    __syncthreads();   // X_{s+1} complete in Y
  };

  float4 m0[KQ], m1[KQ], b0, b1;
  load_m(m0, 0);
  load_b(b0, 0);
  load_b(b1, 1);
  *reinterpret_cast<float4*>(&P[0][crow * LD + ccol]) = b0;   // X_0 = B_0 (S_{-1} = 0)
  __syncthreads();
  int s = 0;
  for (; s + 1 < T; s += 2) {
    step(s, m0, m1, b0, b1, P[0], P[1]);
    step(s + 1, m1, m0, b1, b0, P[1], P[0]);
  }
  if (s < T) step(s, m0, m1, b0, b1, P[0], P[1]);
}

// ---------------------------------------------------------------------------
// readout: for a tile of tokens of one frame, u = S_t q for both directions
// (U = Q S^T on MFMA, S staged in LDS one direction at a time), RMSNorm of
// each over head_dim, summed, times rms weight; the gate multiply and the
// store go through LDS so that every lane writes whole 16-byte chunks.
// In bf16 I/O S enters as the pair hi + lo, so U = Q S_hi^T + Q S_lo^T keeps
// ~16 mantissa bits of S: u = S q can cancel strongly when q is nearly
// orthogonal to the state's rows, and RMSNorm would amplify a bf16 rounding
// of S back to full scale.
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_readout_kernel(
    const T* __restrict__ q, const float* __restrict__ states, const bf16* __restrict__ split,
    const float* __restrict__ rms_w, const T* __restrict__ gate, int64_t ldg, T* __restrict__ out,
    int64_t ldo, int H, int T_, int N, int Lt, float eps, int tiles_per_frame, int64_t bhtdd) {
  using MM = Mma<T>;
  constexpr bool kSplit = sizeof(T) == 2;
  constexpr int KP = MM::kPack, KS = MM::kStep;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int LDSS = D + EPC;            // staged S row stride (elements of T)
  constexpr int CT = D / 16;
  constexpr int KSTEPS = D / KS;
  constexpr int RT = kReadoutBT / 64;      // 16-token row tiles per wave
  constexpr int NPART = kSplit ? 2 : 1;    // hi (+ lo)
  constexpr int LDO = D + 4;               // fp32 output staging row stride
  constexpr int SBYTES = NPART * D * LDSS * (int)sizeof(T);
  constexpr int OBYTES = kReadoutBT * LDO * (int)sizeof(float);
  __shared__ __attribute__((aligned(16))) unsigned char smem[SBYTES > OBYTES ? SBYTES : OBYTES];
  T* Sl = reinterpret_cast<T*>(smem);

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane % 16, lg = lane / 16;
  const int tile = blockIdx.x % tiles_per_frame;
  const int64_t fi = blockIdx.x / tiles_per_frame;     // (b*H + h)*T + t
  const int t = (int)(fi % T_);
  const int64_t bh = fi / T_;
  const int h = (int)(bh % H);
  const int64_t b = bh / H;
  const int n0 = tile * kReadoutBT + wave * (16 * RT);

  typename MM::Frag qa[RT][KSTEPS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = n0 + rt * 16 + li;
    const T* qrow = q + (bh * Lt + (int64_t)t * N + n) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qa[rt][ks] = (n < N) ? MM::load(qrow + ks * KS + lg * KP) : MM::zero();
  }

  f32x4 u[2][RT][CT];
#pragma unroll
  for (int dir = 0; dir < 2; ++dir) {
    __syncthreads();
    if constexpr (kSplit) {
      const bf16* src = split + (dir * bhtdd + fi * D * D) * 2;   // [hi | lo][d][d]
      for (int c = tid; c < 2 * D * D / 8; c += 256) {
        const int part = c / (D * D / 8), rem = c % (D * D / 8);
        const int i = rem / (D / 8), j = (rem % (D / 8)) * 8;
        *reinterpret_cast<Chunk16*>(Sl + (part * D + i) * LDSS + j) =
            *reinterpret_cast<const Chunk16*>(src + (int64_t)c * 8);
      }
    } else {
      const float* src = states + dir * bhtdd + fi * D * D;
      for (int c = tid; c < D * D / 4; c += 256) {
        const int i = c / (D / 4), j = (c % (D / 4)) * 4;
        *reinterpret_cast<Chunk16*>(Sl + i * LDSS + j) = *reinterpret_cast<const Chunk16*>(src + (int64_t)c * 4);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) u[dir][rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
        for (int part = 0; part < NPART; ++part) {
          const typename MM::Frag sfr = MM::load(Sl + (part * D + ct * 16 + li) * LDSS + ks * KS + lg * KP);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) u[dir][rt][ct] = MM::run(qa[rt][ks], sfr, u[dir][rt][ct]);
        }
      }
    }
  }

  // u[dir][rt][ct][r] = u_dir(token n0 + rt*16 + lg*4 + r)[ct*16 + li]
  float rn[2][RT][4];
#pragma unroll
  for (int dir = 0; dir < 2; ++dir)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float ss = 0.f;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) ss += u[dir][rt][ct][r] * u[dir][rt][ct][r];
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m);
        rn[dir][rt][r] = 1.f / sqrtf(ss / D + eps);
      }

  __syncthreads();   // S no longer needed: reuse LDS for the fp32 output tile
  float* Ol = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wave * 16 * RT + rt * 16 + lg * 4 + r;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int i = ct * 16 + li;
        const float w = rms_w ? rms_w[h * D + i] : 1.f;
        Ol[row * LDO + i] = (u[0][rt][ct][r] * rn[0][rt][r] + u[1][rt][ct][r] * rn[1][rt][r]) * w;
      }
    }
  __syncthreads();
  const int64_t NL = Lt;   // output rows per batch entry
  constexpr int CPRO = D / EPC;          // 16-byte chunks per output row
  for (int c = tid; c < kReadoutBT * CPRO; c += 256) {
    const int row = c / CPRO, cc = c % CPRO;
    const int nn = tile * kReadoutBT + row;
    if (nn >= N) continue;
    const int64_t orow = b * NL + (int64_t)t * N + nn;
    float o[EPC];
#pragma unroll
    for (int x = 0; x < EPC; x += 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(Ol + row * LDO + cc * EPC + x);
      o[x] = v4.x; o[x + 1] = v4.y; o[x + 2] = v4.z; o[x + 3] = v4.w;
    }
    if (gate) {
      const Chunk16 gv = *reinterpret_cast<const Chunk16*>(gate + orow * ldg + h * D + cc * EPC);
      const T* ge = reinterpret_cast<const T*>(&gv);
#pragma unroll
      for (int x = 0; x < EPC; ++x) o[x] *= to_f32(ge[x]);
    }
    Chunk16 val;
    T* ve = reinterpret_cast<T*>(&val);
#pragma unroll
    for (int x = 0; x < EPC; ++x) ve[x] = from_f32<T>(o[x]);   // the only rounding of the output
    *reinterpret_cast<Chunk16*>(out + orow * ldo + h * D + cc * EPC) = val;
  }
}

// ---------------------------------------------------------------------------
// readout, bf16 and head_dim D = 64 or 128 (the workload shapes).  One
// workgroup of D/32 waves per (frame, head) or per share of a frame's tokens,
// two workgroups per CU at D = 128.  Wave w owns the output dimensions
// 32w .. 32w+31: it keeps rows 32w .. 32w+31 of both directions' S_hi and S_lo
// in registers as the A operand of 32x32x16 MFMAs, and walks its tokens in
// 32-token tiles computing U^T = S Q^T, D/4 products per tile.  The workgroup
// stages each tile's Q once in LDS (coalesced 16-byte loads two tiles ahead;
// chunk c of token row r at c ^ (r mod the row's chunk count), so the
// fragment reads of a 16-lane group spread over the banks).  RMSNorm needs
// each token's sum of squares over all D dimensions: each wave leaves its
// 32-dimension partial sums in LDS, and after the tile's one barrier every
// wave adds the D/32 partials.  A lane then forms u_f rn_f + u_b rn_b for 16
// dimensions of one token (one cross-lane swap per four dimensions makes them
// two runs of eight) and stages them in LDS; two tiles later, after the
// barriers in between, the workgroup scales them by w and the gate and
// writes whole 2D-byte rows of the head's slice, so each gate load and
// output store instruction covers four full rows instead of 32 bytes of 32
// rows.  With two workgroups per CU one workgroup's products run while the
// other's vector epilogue does.  nsplit > 1 gives each frame that many
// workgroups over consecutive runs of its tiles (each loads the frame's
// states), for shapes with too few frames to fill the chip.
namespace ro {
constexpr int TT = 32;                 // tokens per tile
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ int sw(int row, int ch) { return ch ^ (row & (D / 8 - 1)); }
// 16-byte slot s of row r of a staged output tile: the 16 rows written by one
// half-wave (same slot) and the 2 rows x 8 chunks read by 16 lanes spread over
// all 64 banks
__device__ __forceinline__ int ysw(int r, int s) { return s ^ (r & 15); }
}  // namespace ro

template <int D, bool kGate>
__global__ __launch_bounds__(2 * D, 2) void vda_readout_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ split, const float* __restrict__ rms_w,
    const bf16* __restrict__ gate, int64_t ldg, bf16* __restrict__ out, int64_t ldo, int H, int T_, int N,
    int Lt, float eps, int64_t bhtdd, int nsplit) {
  using namespace ro;
  constexpr int NW = D / 32, NT = 2 * D;   // waves, threads
  constexpr int CPR = D / 8;               // 16-byte chunks per token row
  constexpr int KS = D / 16;               // 16-deep product steps
  constexpr int QROW = D * 2;              // bytes per token row of a staged Q tile
  constexpr int QTILE = TT * QROW;
  constexpr int YS = D / 4;                // 16-byte slots per row of a staged output tile (fp32)
  constexpr int NBLK = D / 64;             // 8-chunk blocks per output row
  __shared__ __attribute__((aligned(16))) unsigned char QL[2][QTILE];
  __shared__ __attribute__((aligned(16))) float4 YL[2][TT * YS];
  __shared__ __attribute__((aligned(16))) float SSX[2][2][TT][NW];   // [buffer][dir][token][wave]
  __shared__ __attribute__((aligned(16))) float wl[D];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l32 = lane % 32, h = lane / 32;
  const int64_t fi = blockIdx.x / nsplit;              // (b*H + hh)*T + t
  const int sp = blockIdx.x % nsplit;
  const int t = (int)(fi % T_);
  const int64_t bh = fi / T_;
  const int hh = (int)(bh % H);
  const int64_t b = bh / H;
  const int d0 = 32 * wave;
  const int ftiles = (N + TT - 1) / TT, tps = (ftiles + nsplit - 1) / nsplit;
  const int tile0 = sp * tps, ntile = min(ftiles, tile0 + tps);   // this workgroup's tiles: tile0 .. ntile-1
  if (tile0 >= ntile) return;   // the whole workgroup (no barrier reached)
  const bf16* qfr = q + (bh * Lt + (int64_t)t * N) * D;
  const int64_t row0 = b * (int64_t)Lt + (int64_t)t * N;   // output / gate row of the frame's token 0

  if (tid < D) wl[tid] = rms_w ? rms_w[hh * D + tid] : 1.f;
  // sf[dir][part][ks] = S_part of direction dir, row d0 + l32, columns 16 ks + 8 h .. +7
  bf16x8 sf[2][2][KS];
#pragma unroll
  for (int dir = 0; dir < 2; ++dir)
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const bf16* sp = split + (dir * bhtdd + fi * D * D) * 2 + part * D * D + (int64_t)(d0 + l32) * D + 8 * h;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sf[dir][part][ks] = *reinterpret_cast<const bf16x8*>(sp + 16 * ks);
    }

  // Global traffic goes through buffer descriptors that start at a tile's first row
  // and end at the frame's last: rows past the frame read as zero and their stores
  // are dropped, and every lane offset is a fixed 32-bit value (the host keeps a
  // frame's rows below 2^31 bytes).
  auto rows_rsrc = [&](const bf16* frame, int64_t ld, int tile) {
    const int rows = max(N - tile * TT, 0);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(frame + (int64_t)tile * TT * ld), (short)0,
                                             (int)(rows * ld * 2), 0x00020000);
  };
  // the thread's share of a Q tile: 16-byte chunks tid and tid + NT (token c / CPR,
  // chunk c % CPR), i.e. bytes 16 tid and 16 tid + 32 D of the tile
  auto load_q = [&](bf16x8 (&qv)[2], int tile) {
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(qfr, D, tile);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      qv[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, 16 * tid + 32 * D * j, 0, 0));
  };
  auto store_q = [&](const bf16x8 (&qv)[2], int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + NT * j, r = c / CPR;
      *reinterpret_cast<bf16x8*>(&QL[buf][r * QROW + sw<D>(r, c % CPR) * 16]) = qv[j];
    }
  };
  // Output emission, coalesced: a tile's normalised values go to LDS (fp32, YL) and
  // after the next barrier every thread scales two 16-byte chunks of whole token
  // rows by the RMSNorm weight and the gate and writes them, 16 lanes covering two rows x 8 chunks, with the gate chunk at the same
  // place loaded the same way.  Chunk j of thread t: row crow(t, j), columns
  // 8 ccol(t, j) .. +7 of the head's slice.
  // (the chunk coordinates are recomputed from an opaque copy of tid at each use,
  // so that the compiler does not keep them, and the weights they index, in
  // registers across the tile loop)
  auto opaque_tid = [&]() { int v = tid; asm volatile("" : "+v"(v)); return v; };
  auto crow = [&](int t, int j) { const int idx = t + NT * j; return 2 * (idx / (16 * NBLK)) + (idx / 8) % 2; };
  auto ccol = [&](int t, int j) { const int idx = t + NT * j; return 8 * ((idx / 16) % NBLK) + idx % 8; };
  const bf16* gfr = kGate ? gate + row0 * ldg + hh * D : nullptr;
  bf16* ofr = out + row0 * ldo + hh * D;
  auto load_g = [&](bf16x8 (&gv)[2], int tile) {
    const __amdgpu_buffer_rsrc_t rg = rows_rsrc(gfr, ldg, tile);
    const int t = opaque_tid();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int off = 2 * (crow(t, j) * (int)ldg + 8 * ccol(t, j));   // a tile spans 32 rows
      gv[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
    }
  };
  // write tile's staged values (gated, rounded once) to its output rows
  auto emit = [&](int tile, const bf16x8 (&gv)[2]) {
    const float4* yt = YL[tile & 1];
    const __amdgpu_buffer_rsrc_t ro = rows_rsrc(ofr, ldo, tile);
    const int t = opaque_tid();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = crow(t, j), c = ccol(t, j);
      const float4 lo = yt[r * YS + ysw(r, 2 * c)];
      const float4 hi = yt[r * YS + ysw(r, 2 * c + 1)];
      const float4 wlo = *reinterpret_cast<const float4*>(&wl[8 * c]);
      const float4 whi = *reinterpret_cast<const float4*>(&wl[8 * c + 4]);
      const float y[8] = {lo.x * wlo.x, lo.y * wlo.y, lo.z * wlo.z, lo.w * wlo.w,
                          hi.x * whi.x, hi.y * whi.y, hi.z * whi.z, hi.w * whi.w};
      bf16x8 ov;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (kGate) ov[e] = (bf16)(y[e] * (float)gv[j][e]);   // the only rounding of the output
        else ov[e] = (bf16)y[e];
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ov), ro, 2 * (r * (int)ldo + 8 * c), 0, 0);
    }
  };

  // One tile.  qv holds Q of tile + 1 (stored into LDS here, then refilled with
  // tile + 3); gv holds the gate of tile - 2, whose staged values (complete since
  // the previous barrier, overwritten only after this tile's) are emitted first,
  // then the gate of this tile: two register sets alternate, so every load has
  // two tiles' time to arrive.
  auto body = [&](int tile, bf16x8 (&qv)[2], bf16x8 (&gv)[2], auto EMIT) {
    const int buf = tile & 1;
    if constexpr (decltype(EMIT)::value) emit(tile - 2, gv);
    if constexpr (kGate) load_g(gv, tile);
    // B operand: q[token 32 tile + l32][16 ks + 8 h .. +7]
    bf16x8 bq[KS];
    const unsigned char* qrow = QL[buf] + l32 * QROW;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bq[ks] = *reinterpret_cast<const bf16x8*>(qrow + sw<D>(l32, 2 * ks + h) * 16);
    // acc_dir[r] = u_dir[dimension d0 + 8 (r/4) + 4 h + r%4] of token 32 tile + l32
    f32x16 acc0, acc1;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sf[0][part][ks], bq[ks], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sf[1][part][ks], bq[ks], acc1, 0, 0, 0);
      }
    // the next tile's Q into the other buffer (its readers have passed the previous barrier)
    store_q(qv, buf ^ 1);
    load_q(qv, tile + 3);

    float ss0 = 0.f, ss1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ss0 += acc0[r] * acc0[r];
      ss1 += acc1[r] * acc1[r];
    }
    const auto x0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss0), __float_as_uint(ss0), false, false);
    const auto x1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss1), __float_as_uint(ss1), false, false);
    if (h == 0) {
      SSX[buf][0][l32][wave] = __uint_as_float(x0[0]) + __uint_as_float(x0[1]);
      SSX[buf][1][l32][wave] = __uint_as_float(x1[0]) + __uint_as_float(x1[1]);
    }
    __syncthreads();   // partial sums and the next Q tile complete
    float s0, s1;
    if constexpr (NW == 4) {
      const float4 p0 = *reinterpret_cast<const float4*>(&SSX[buf][0][l32][0]);
      const float4 p1 = *reinterpret_cast<const float4*>(&SSX[buf][1][l32][0]);
      s0 = (p0.x + p0.y) + (p0.z + p0.w);
      s1 = (p1.x + p1.y) + (p1.z + p1.w);
    } else {
      const float2 p0 = *reinterpret_cast<const float2*>(&SSX[buf][0][l32][0]);
      const float2 p1 = *reinterpret_cast<const float2*>(&SSX[buf][1][l32][0]);
      s0 = p0.x + p0.y;
      s1 = p1.x + p1.y;
    }
    // hardware reciprocal square root (1 ulp)
    const float rn0 = __builtin_amdgcn_rsqf(s0 * (1.f / D) + eps);
    const float rn1 = __builtin_amdgcn_rsqf(s1 * (1.f / D) + eps);
    float4* yw = YL[buf] + l32 * YS;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      // ya: dims d0 + 16pp + 4h + e, yb: dims d0 + 16pp + 8 + 4h + e; after the swap
      // the lane holds dims d0 + 16pp + 8h + {0..3} in ya and + {4..7} in yb, i.e.
      // chunk 4 wave + 2 pp + h of its token's row
      float ya[4], yb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ya[e] = acc0[8 * pp + e] * rn0 + acc1[8 * pp + e] * rn1;
        yb[e] = acc0[8 * pp + 4 + e] * rn0 + acc1[8 * pp + 4 + e] * rn1;
        const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(ya[e]), __float_as_uint(yb[e]), false, false);
        ya[e] = __uint_as_float(x[0]);
        yb[e] = __uint_as_float(x[1]);
      }
      const int c = 4 * wave + 2 * pp + h;
      yw[ysw(l32, 2 * c)] = make_float4(ya[0], ya[1], ya[2], ya[3]);
      yw[ysw(l32, 2 * c + 1)] = make_float4(yb[0], yb[1], yb[2], yb[3]);
    }
  };

  bf16x8 q0[2], q1[2];
  bf16x8 g0[2], g1[2];
  load_q(q0, tile0);
  store_q(q0, tile0 & 1);
  load_q(q0, tile0 + 1);
  load_q(q1, tile0 + 2);
  __syncthreads();
  // tile t uses the register sets of parity t - tile0 (q0, g0 even)
  body(tile0, q0, g0, std::false_type{});
  if (tile0 + 1 < ntile) body(tile0 + 1, q1, g1, std::false_type{});
  int tile = tile0 + 2;
  for (; tile + 2 <= ntile; tile += 2) {
    body(tile, q0, g0, std::true_type{});
    body(tile + 1, q1, g1, std::true_type{});
  }
  if (tile < ntile) body(tile, q0, g0, std::true_type{});
  __syncthreads();   // the last tile's staged values complete
  // the last two tiles (gates in the sets of their parity)
  if (ntile - tile0 >= 2) {
    if ((ntile - tile0) & 1) {
      emit(ntile - 2, g1);
      emit(ntile - 1, g0);
    } else {
      emit(ntile - 2, g0);
      emit(ntile - 1, g1);
    }
  } else {
    emit(ntile - 1, g0);
  }
}

// ---------------------------------------------------------------------------
template <typename T>
static hipError_t gram_t(int d, const void* k, const void* v, const float* beta, float* A,
                         float* Bm, int nframes, int T_, int N, int Lt, hipStream_t st) {
  if (sizeof(T) == 2 && d == 128)
    vda_gram_bf16_kernel<128><<<nframes, 256, 0, st>>>((const bf16*)k, (const bf16*)v, beta, A, Bm, T_, N, Lt);
  else if (sizeof(T) == 2 && d == 64)
    vda_gram_bf16_kernel<64><<<nframes, 256, 0, st>>>((const bf16*)k, (const bf16*)v, beta, A, Bm, T_, N, Lt);
  else if (d == 32)
    vda_gram_kernel<T, 32><<<nframes, 256, 0, st>>>((const T*)k, (const T*)v, beta, A, Bm, T_, N, Lt);
  else if (d == 64)
    vda_gram_kernel<T, 64><<<nframes, 256, 0, st>>>((const T*)k, (const T*)v, beta, A, Bm, T_, N, Lt);
  else
    vda_gram_kernel<T, 128><<<nframes, 256, 0, st>>>((const T*)k, (const T*)v, beta, A, Bm, T_, N, Lt);
  return hipGetLastError();
}

// Range check of the per-frame parameters: beta >= 0 keeps I + A_t positive
// definite, 0 <= gamma <= 1 keeps the decay a contraction.  One workgroup; the
// result is written unconditionally, so the flag needs no clearing.
__global__ __launch_bounds__(256) void param_check_kernel(const float* gamma, const float* beta,
                                                          int n, int* flag) {
  int bad = 0;
  for (int i = threadIdx.x; i < n; i += 256) {
    const float g = gamma[i], b = beta[i];
    bad |= (b < 0.f) | (g < 0.f) | (g > 1.f);
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) flag[0] = bad ? 1 : 0;
}

hipError_t launch_param_check(const float* gamma, const float* beta, int n, int* flag,
                              hipStream_t st) {
  param_check_kernel<<<1, 256, 0, st>>>(gamma, beta, n, flag);
  return hipGetLastError();
}

hipError_t launch_vda_gram(int dtype, int d, const void* k, const void* v, const float* beta,
                           float* A, float* Bm, int nframes, int T, int N, int Lt, hipStream_t st) {
  if (nframes == 0) return hipSuccess;
  return dtype == 1 ? gram_t<bf16>(d, k, v, beta, A, Bm, nframes, T, N, Lt, st)
                    : gram_t<float>(d, k, v, beta, A, Bm, nframes, T, N, Lt, st);
}

hipError_t launch_vda_solve(int d, float* AM, int nframes, hipStream_t st) {
  if (nframes == 0) return hipSuccess;
  if (d == 32) vda_solve_kernel<32><<<nframes, 64, 0, st>>>(AM);
  else if (d == 64) vda_solve_kernel<64><<<nframes, 128, 0, st>>>(AM);
  else vda_solve_kernel<128><<<nframes, 256, 0, st>>>(AM);
  return hipGetLastError();
}

hipError_t launch_vda_scan(int d, const float* Mt, const float* Bm, const float* gamma,
                           float* states, bf16* split, int BH, int T, hipStream_t st) {
  if (BH == 0) return hipSuccess;
  const int64_t bhtdd = (int64_t)BH * T * d * d;
  if (d == 128 || d == 64) {
    const int total = BH * 2 * (d / 32);   // d / 32 row blocks x 2 directions per (batch, head)
#define VDN_SCAN(DD, WS, WH) \
  vda_scan_mfma_kernel<DD, WS, WH><<<total, 2 * DD, 0, st>>>(Mt, Bm, gamma, states, split, T, bhtdd, total)
#define VDN_SCAN16(DD, WS, WH) \
  vda_scan_mfma16_kernel<DD, WS, WH><<<total16, 4 * DD, 0, st>>>(Mt, Bm, gamma, states, split, T, bhtdd, total16)
    const int total16 = BH * 2 * (d / sc16::R);
    if (!states && !split) return hipErrorInvalidValue;
    if (d == 128) {
      if (states && split) VDN_SCAN(128, true, true);
      else if (states) VDN_SCAN(128, true, false);
      else VDN_SCAN(128, false, true);
    } else {   // 16 rows per workgroup (at d = 128 the 32-row kernel measured faster)
      if (states && split) VDN_SCAN16(64, true, true);
      else if (states) VDN_SCAN16(64, true, false);
      else VDN_SCAN16(64, false, true);
    }
#undef VDN_SCAN
#undef VDN_SCAN16
    return hipGetLastError();
  }
  dim3 grid(d / kScanRows, BH, 2);
  vda_scan_kernel<32, kScanRows><<<grid, 256, 0, st>>>(Mt, Bm, gamma, states, split, T, bhtdd);
  return hipGetLastError();
}

template <typename T>
static hipError_t readout_t(int d, const void* q, const float* states, const bf16* split,
                            const float* rms_w, const void* gate, int64_t ldg, void* out, int64_t ldo,
                            int B, int H, int T_, int N, int Lt, float eps, hipStream_t st) {
  const int64_t bhtdd = (int64_t)B * H * T_ * d * d;
  // the register-resident kernel addresses a frame's rows of q, gate and out with 32-bit offsets
  const int64_t frame_bytes = (int64_t)N * std::max<int64_t>(std::max<int64_t>(ldo, gate ? ldg : 0), d) * 2;
  if (sizeof(T) == 2 && (d == 128 || d == 64) && split && frame_bytes < (int64_t(1) << 31)) {
    const int64_t nb = (int64_t)B * H * T_;
    if (nb == 0 || N <= 0) return hipSuccess;
    // frames too few to give every workgroup slot one (two per CU at d = 128, about six at
    // d = 64) get several workgroups each, each with at least 8 tiles
    const int ftiles = (N + 31) / 32;
    const int64_t target = d == 128 ? 512 : 1536;
    int nsplit = 1;
    while (nsplit < 8 && nb * nsplit < target && ftiles >= 16 * nsplit) nsplit *= 2;
    const unsigned grid = (unsigned)(nb * nsplit);
#define VDN_RO(DD, G) \
  vda_readout_bf16_kernel<DD, G><<<grid, 2 * DD, 0, st>>>((const bf16*)q, split, rms_w, (const bf16*)gate, ldg, \
                                                          (bf16*)out, ldo, H, T_, N, Lt, eps, bhtdd, nsplit)
    if (d == 128) {
      if (gate) VDN_RO(128, true);
      else VDN_RO(128, false);
    } else {
      if (gate) VDN_RO(64, true);
      else VDN_RO(64, false);
    }
#undef VDN_RO
    return hipGetLastError();
  }
  const int tpf = (N + kReadoutBT - 1) / kReadoutBT;
  const int64_t blocks = (int64_t)B * H * T_ * tpf;
  if (blocks == 0) return hipSuccess;
#define VDN_READOUT(DD)                                                                         \
  vda_readout_kernel<T, DD><<<(unsigned)blocks, 256, 0, st>>>(                                  \
      (const T*)q, states, split, rms_w, (const T*)gate, ldg, (T*)out, ldo, H, T_, N, Lt, eps, \
      tpf, bhtdd)
  if (d == 32) VDN_READOUT(32);
  else if (d == 64) VDN_READOUT(64);
  else VDN_READOUT(128);
#undef VDN_READOUT
  return hipGetLastError();
}

hipError_t launch_vda_readout(int dtype, int d, const void* q, const float* states,
                              const bf16* split, const float* rms_w, const void* gate, int64_t ldg,
                              void* out, int64_t ldo, int B, int H, int T, int N, int Lt, float eps,
                              hipStream_t st) {
  return dtype == 1 ? readout_t<bf16>(d, q, states, split, rms_w, gate, ldg, out, ldo, B, H, T, N, Lt, eps, st)
                    : readout_t<float>(d, q, states, split, rms_w, gate, ldg, out, ldo, B, H, T, N, Lt, eps, st);
}

// Zero `cols` elements of rows [row0, row0 + nrows) of every batch entry of a
// row-major [B, rows_per_batch, ld] matrix: the linear branch's output on
// context rows.  One thread per 4-byte word.
__global__ __launch_bounds__(256) void zero_rows_kernel(uint32_t* __restrict__ base, int64_t rows_per_batch,
                                                        int64_t row0, int64_t nrows, int64_t ld_words,
                                                        int64_t words, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t w = i % words, rb = i / words;
  const int64_t r = rb % nrows, b = rb / nrows;
  base[(b * rows_per_batch + row0 + r) * ld_words + w] = 0u;
}

hipError_t launch_zero_rows(void* base, int B, int64_t rows_per_batch, int64_t row0, int64_t nrows,
                            int64_t ld, int64_t cols, int es, hipStream_t st) {
  const int64_t words = cols * es / 4, total = (int64_t)B * nrows * words;
  if (total == 0) return hipSuccess;
  zero_rows_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>((uint32_t*)base, rows_per_batch, row0, nrows,
                                                                    ld * es / 4, words, total);
  return hipGetLastError();
}

}  // namespace vdn
