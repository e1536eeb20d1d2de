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
// gram, bf16 / head_dim 128 (the workload shape).  One workgroup of four waves
// per (frame, head); K_t and V_t stream through a four-stage LDS ring of
// 64-token tiles by the direct-to-LDS DMA path (a buffer load with the lds
// modifier), row-major with XOR-swizzled 16-byte chunks; token rows past N
// read as zero.  Wave w consumes token rows 16w .. 16w+15 of every tile.  A
// ds_read_b64_tr_b16 pair hands each lane eight tokens of one dimension: that
// register is the A operand (row = dimension) and equally the B operand
// (column = dimension) of a 32x32x16 MFMA, so K^T K and V^T K need no other
// data movement.  Each wave accumulates the 10 upper 32x32 tiles of K^T K and
// the 16 tiles of V^T K over its quarter of the tokens (416 fp32 per lane);
// the four partial sums are added through LDS at the end, scaled by beta_t,
// and A's off-diagonal tiles are mirrored.
namespace gr {
constexpr int D = 128, BN = 64, ROWB = D * 2, TILEB = BN * ROWB, STAGEB = 2 * TILEB, STAGES = 4;
constexpr int NA = 10, NTILE = NA + 16;      // output tiles: upper A tiles, then B tiles
constexpr int TB = 7;                        // tiles per reduction batch (4 x 7 x 16 x 65 floats fit the ring)
constexpr int kWaitVm0 = 0x0F70;             // s_waitcnt vmcnt(0)
constexpr int kWaitVm8 = 0x0F78;             // vmcnt(8): one tile's loads may be outstanding
constexpr int kWaitVm16 = 0x4F70;            // vmcnt(16): two tiles' loads may be outstanding
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
// Physical chunk of logical 16-byte chunk c of row r: 8 rows x 4 chunks of a
// transpose read touch every bank exactly twice.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r & 7) << 1) | ((r >> 3) & 1)); }
// (tile row block, tile column block) of output tile u
__device__ __forceinline__ constexpr int tile_i(int u) {
  return u < 4 ? 0 : u < 7 ? 1 : u < 9 ? 2 : u < 10 ? 3 : (u - NA) / 4;
}
__device__ __forceinline__ constexpr int tile_j(int u) {
  return u < 4 ? u : u < 7 ? u - 3 : u < 9 ? u - 5 : u < 10 ? 3 : (u - NA) % 4;
}
// Accumulating products with the accumulator's register file fixed: the 10
// K^T K tiles in vector registers, the 16 V^T K tiles in accumulator
// registers (416 fp32 per lane do not fit one file; left to itself the
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

__global__ __launch_bounds__(256) void vda_gram_bf16_d128_kernel(const bf16* __restrict__ k,
                                                                 const bf16* __restrict__ v,
                                                                 const float* __restrict__ beta,
                                                                 float* __restrict__ A,
                                                                 float* __restrict__ Bm, int T_, int N,
                                                                 int Lt) {
  using namespace gr;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STAGES * STAGEB];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int g = lane / 16, j16 = lane % 16;
  const int64_t f = blockIdx.x;
  const int64_t row0 = (f / T_) * Lt + (f % T_) * N;   // first token row of frame f
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k + row0 * D), (short)0, N * ROWB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v + row0 * D), (short)0, N * ROWB, 0x00020000);

  // DMA: lane l of block b fills physical chunk l%16 of tile row 4b + l/16
  int lane_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wave * 4 + i) * 4 + lane / 16;
    lane_off[i] = row * ROWB + swz(row, lane % 16) * 16;
  }
  const int ntiles = (N + BN - 1) / BN;
  auto issue = [&](int t) {
    const int lds = (int)(size_t)(__attribute__((address_space(3))) unsigned char*)(ring + (t & 3) * STAGEB);
    const int base = t * BN * ROWB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int blk = wave * 4 + i;
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
  int offA[4], offB[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int rowA = 16 * wave + 4 * (g >> 1) + (j16 >> 2), rowB = rowA + 8;
    const int dcol = dt * 32 + 16 * (g & 1) + 4 * (j16 & 3);
    const int cch = dcol >> 3, off = (dcol & 7) * 2;
    offA[dt] = rowA * ROWB + swz(rowA, cch) * 16 + off;
    offB[dt] = rowB * ROWB + swz(rowB, cch) * 16 + off;
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
    if (t + 2 < ntiles) __builtin_amdgcn_s_waitcnt(kWaitVm16);
    else if (t + 1 < ntiles) __builtin_amdgcn_s_waitcnt(kWaitVm8);
    else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();                       // tile t visible; tile t-1's stage free
    if (t + 3 < ntiles) issue(t + 3);
    const unsigned char* sb = ring + (t & 3) * STAGEB;
    bf16x8 kf[4], vf[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      kf[dt] = frag(sb, dt);
      vf[dt] = frag(sb + TILEB, dt);
    }
    const bool first = t == 0;
#pragma unroll
    for (int u = 0; u < NA; ++u) mma_v(accA[u], kf[tile_i(u)], kf[tile_j(u)], first);
#pragma unroll
    for (int u = NA; u < NTILE; ++u) mma_a(accB[u - NA], vf[tile_i(u)], kf[tile_j(u)], first);
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
      const int ti = tile_i(u), tj = tile_j(u);
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
// column c in registers; at step k the pivot row and the pivot column go
// through LDS (double-buffered, one barrier per step) and every column is
// updated with a rank-1 step.  I + A_t is symmetric positive definite (beta
// >= 0, eigenvalues >= 1), for which elimination without pivoting is stable.
// AM holds A_t on entry and M_t^T on exit (row j = column j of M_t, so the
// scan reads contiguous runs of a column).
template <int D>
__global__ __launch_bounds__(2 * D) void vda_solve_kernel(float* __restrict__ AM) {
  __shared__ __attribute__((aligned(16))) float colb[2][D];
  __shared__ float rowb[2][2 * D];
  const int64_t f = blockIdx.x;
  float* am = AM + f * D * D;
  const int c = threadIdx.x;

  float a[D];
#pragma unroll
  for (int i = 0; i < D; ++i)
    a[i] = c < D ? am[i * D + c] + (i == c ? 1.f : 0.f) : (i == c - D ? 1.f : 0.f);
  __syncthreads();   // every column is read before any thread overwrites AM below

  // The rows rotate by one per step, so that the pivot row is always a[0]
  // (all register indices stay compile-time constants): the update writes
  // row i+1 into slot i and the normalised pivot row goes to slot D-1.  After
  // D steps every row is back in its place.
  for (int k = 0; k < D; ++k) {
    const int buf = k & 1;
    rowb[buf][c] = a[0];
    if (c == k) {
#pragma unroll
      for (int i = 0; i < D; i += 4)
        *reinterpret_cast<float4*>(&colb[buf][i]) = make_float4(a[i], a[i + 1], a[i + 2], a[i + 3]);
    }
    __syncthreads();
    const float x = rowb[buf][c] / rowb[buf][k];
#pragma unroll
    for (int i = 0; i < D; i += 4) {
      const float4 cv = *reinterpret_cast<const float4*>(&colb[buf][i]);
      if (i > 0) a[i - 1] = a[i] - cv.x * x;
      a[i] = a[i + 1] - cv.y * x;
      a[i + 1] = a[i + 2] - cv.z * x;
      a[i + 2] = a[i + 3] - cv.w * x;
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
// This is the path for head_dim 32 and 64; head_dim 128 uses the MFMA kernel
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
// scan, head_dim 128, on fp32 MFMA.  One workgroup of four waves per 32 state
// rows of one (batch, head, direction); wave w produces columns 32w .. 32w+31
// of those rows with 64 v_mfma_f32_32x32x2_f32 per frame.  The contraction
// index is permuted so that every operand is a contiguous run: at product s
// lane half h supplies k = 64h + s, so the A operand is row r0 + l%32 of
// X = gamma S + B, columns 64h .. 64h+63 (S from LDS, B_t from HBM), and the
// B operand is row 32w + l%32 of M_t^T, the same columns.  B_{t+1} and
// M_{t+1}^T are loaded while frame t is multiplied.  The eight workgroups of
// one (batch, head) share an XCD, so each M_t comes from HBM once per
// direction.
namespace sc {
constexpr int D = 128, R = 32, LD = D + 4;
typedef float f32x16 __attribute__((ext_vector_type(16)));
}  // namespace sc

__global__ __launch_bounds__(256) void vda_scan_d128_kernel(const float* __restrict__ Mt,
                                                            const float* __restrict__ Bm,
                                                            const float* __restrict__ gamma,
                                                            float* __restrict__ states,
                                                            bf16* __restrict__ split, int T,
                                                            int64_t bhtdd, int total) {
  using namespace sc;
  __shared__ __attribute__((aligned(16))) float Ss[R * LD];   // S_{t-1}, rows r0 .. r0+31
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int l32 = lane % 32, h = lane / 32;
  const int lid = xcd_remap(blockIdx.x, total);
  const int dir = lid & 1, rb = (lid >> 1) & 3;
  const int64_t bh = lid >> 3;
  const int r0 = rb * R, n0 = wave * 32;
  for (int i = tid; i < R * LD; i += 256) Ss[i] = 0.f;

  auto frame = [&](int step) { return dir ? T - 1 - step : step; };
  auto load = [&](float4 (&b)[16], float4 (&m)[16], int t) {
    const int64_t fi = bh * T + t;
    const float4* bp = reinterpret_cast<const float4*>(Bm + fi * D * D + (int64_t)(r0 + l32) * D + 64 * h);
    const float4* mp = reinterpret_cast<const float4*>(Mt + fi * D * D + (int64_t)(n0 + l32) * D + 64 * h);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      b[i] = bp[i];
      m[i] = mp[i];
    }
  };
  float4 bx[16], mx[16];
  load(bx, mx, frame(0));
  __syncthreads();

  for (int step = 0; step < T; ++step) {
    const int t = frame(step);
    const int64_t fi = bh * T + t;
    const float g = gamma[fi];
    float4 bn[16], mn[16];
    load(bn, mn, frame(step + 1 < T ? step + 1 : step));
    __builtin_amdgcn_sched_barrier(0);   // the next frame's loads go out before this frame's products
    const float* srow = Ss + l32 * LD + 64 * h;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 sv = *reinterpret_cast<const float4*>(srow + 4 * i);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(g * sv.x + bx[i].x, mx[i].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(g * sv.y + bx[i].y, mx[i].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(g * sv.z + bx[i].z, mx[i].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(g * sv.w + bx[i].w, mx[i].w, acc, 0, 0, 0);
    }
    __syncthreads();   // every wave has read S_{t-1}
    // acc[r] = S_t[r0 + 8 (r/4) + 4h + r%4][n0 + l32]
    float* sdst = states + dir * bhtdd + fi * D * D + (int64_t)r0 * D + n0 + l32;
    bf16* hdst = split ? split + (dir * bhtdd + fi * D * D) * 2 + (int64_t)r0 * D + n0 + l32 : nullptr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r / 4) + 4 * h + r % 4;
      Ss[row * LD + n0 + l32] = acc[r];
      sdst[row * D] = acc[r];
      if (hdst) {
        const bf16 hi = (bf16)acc[r];
        hdst[row * D] = hi;
        hdst[row * D + D * D] = (bf16)(acc[r] - (float)hi);
      }
    }
    __syncthreads();   // S_t visible
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      bx[i] = bn[i];
      mx[i] = mn[i];
    }
  }
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
// readout, bf16 and head_dim 128 (the workload shapes).  One workgroup of four
// waves per (frame, head) walks all N tokens of the frame.  Both directions'
// S_hi and S_lo are copied into LDS once by the direct-to-LDS DMA (4 x 32 KB;
// the 16-byte chunk c of row i at c ^ (i & 15), so that the sixteen rows a
// 16-lane group reads cover all banks).  Each wave then takes 64-token blocks
// (block = wave + 4k) and computes U^T = S Q^T on 32x32x16 MFMA: the state
// fragments are the A operand (one LDS read serves both 32-token tiles), the
// Q fragments come straight from HBM as the B operand.  The loads of the
// block's gate and of the next block's Q are issued before the block's 256
// products, so their latency hides behind the matrix work; the accumulators
// live in the accumulator registers.  A lane holds 64 of the 128 outputs of
// one token, its partner lane i ^ 32 the other 64: the RMSNorm needs one
// cross-lane swap, and one swap per four outputs gives each lane eight
// consecutive dimensions for 16-byte gate loads and output stores.
namespace ro {
constexpr int D = 128, SUB = 64;
constexpr int MATB = D * D * 2;   // one bf16 d x d matrix, 32 KB
constexpr int kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0)
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ int sw(int row, int ch) { return ch ^ (row & 15); }
// products with the accumulator in the accumulator registers; a chain starts from zero
__device__ __forceinline__ void mma_first(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&a"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
}  // namespace ro

__global__ __launch_bounds__(256) void vda_readout_bf16_d128_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ split, const float* __restrict__ rms_w,
    const bf16* __restrict__ gate, int64_t ldg, bf16* __restrict__ out, int64_t ldo, int H, int T_, int N,
    int Lt, float eps, int64_t bhtdd) {
  using namespace ro;
  __shared__ __attribute__((aligned(1024))) unsigned char Sl[4 * MATB];   // [dir][hi, lo][row][chunk]
  __shared__ float wl[D];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l32 = lane % 32, h = lane / 32;
  const int64_t fi = blockIdx.x;                       // (b*H + hh)*T + t
  const int t = (int)(fi % T_);
  const int64_t bh = fi / T_;
  const int hh = (int)(bh % H);
  const int64_t b = bh / H;

  // states -> LDS: 1 KB block j of a direction (j < 32: S_hi rows 4j..4j+3,
  // else S_lo) by wave j / 16; lane l fills physical chunk l % 16 of row l / 16
  {
    const int lds0 = (int)(size_t)(__attribute__((address_space(3))) unsigned char*)Sl;
#pragma unroll
    for (int dir = 0; dir < 2; ++dir) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(split + (dir * bhtdd + fi * D * D) * 2), (short)0, 2 * MATB, 0x00020000);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int blk = wave * 16 + i, part = blk / 32;
        const int row = (blk % 32) * 4 + lane / 16;
        const int voff = part * MATB + row * 256 + sw(row, lane % 16) * 16;
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
                     "{m0}"(lds0 + dir * 2 * MATB + blk * 1024)
                     : "memory");
      }
    }
  }
  if (tid < D) wl[tid] = rms_w ? rms_w[hh * D + tid] : 1.f;

  const int64_t NL = Lt;   // rows per (batch, head) of q and per batch entry of out / gate
  const bf16* qfr = q + (bh * Lt + (int64_t)t * N) * D;
  const int nblk = (N + SUB - 1) / SUB;
  // Q^T fragments of a block: lane holds q[token 32 tt + l32][16 ks + 8 h .. +7].
  // Token indices past the frame are clamped to its last token (loads stay
  // unconditional); those lanes' outputs are never stored.
  auto load_q = [&](bf16x8 (&dst)[2][8], int blk) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int n = min(blk * SUB + 32 * tt + l32, N - 1);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        dst[tt][ks] = *reinterpret_cast<const bf16x8*>(qfr + (int64_t)n * D + 16 * ks + 8 * h);
    }
  };
  bf16x8 qf[2][8];
  load_q(qf, wave);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  for (int blk = wave; blk < nblk; blk += 4) {
    bf16x8 qn[2][8];
    load_q(qn, blk + 4);
    __builtin_amdgcn_sched_barrier(0);   // the loads above go out before the products

    // acc[dir][tt][dt][r] = u_dir(token 32 tt + l32)[32 dt + 8 (r/4) + 4 h + r%4].
    // 128 steps (dir, dt, ks, part), each one state-fragment read and two
    // products; fragments are read three steps ahead and the steps are fenced,
    // so at most four fragments are live.
    f32x16 acc[2][2][4];
    auto read_sf = [&](int step) {
      const int dir = step >> 6, dt = (step >> 4) & 3, ks = (step >> 1) & 7, part = step & 1;
      const int row = 32 * dt + l32;
      return *reinterpret_cast<const bf16x8*>(Sl + (2 * dir + part) * MATB + row * 256 + sw(row, 2 * ks + h) * 16);
    };
    bf16x8 sfb[4];
#pragma unroll
    for (int i = 0; i < 3; ++i) sfb[i] = read_sf(i);
    // gate of this block (lane: dims 32 dt + 16 p + 8 h .. +7 of its token), loaded
    // halfway through the products
    bf16x8 gv[2][4][2];
#pragma unroll
    for (int step = 0; step < 128; ++step) {
      if (step == 64 && gate) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int n = min(blk * SUB + 32 * tt + l32, N - 1);
          const bf16* grow = gate + (b * NL + (int64_t)t * N + n) * ldg + hh * D + 8 * h;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) gv[tt][dt][pp] = *reinterpret_cast<const bf16x8*>(grow + 32 * dt + 16 * pp);
        }
      }
      if (step + 3 < 128) sfb[(step + 3) & 3] = read_sf(step + 3);
      const int dir = step >> 6, dt = (step >> 4) & 3, ks = (step >> 1) & 7, part = step & 1;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        if (ks == 0 && part == 0) mma_first(acc[dir][tt][dt], sfb[step & 3], qf[tt][ks]);
        else mma_acc(acc[dir][tt][dt], sfb[step & 3], qf[tt][ks]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the products' results are read by vector instructions below
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int n = blk * SUB + 32 * tt + l32;
      float rn[2];
#pragma unroll
      for (int dir = 0; dir < 2; ++dir) {
        float ss = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) ss += acc[dir][tt][dt][r] * acc[dir][tt][dt][r];
        const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        ss = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
        rn[dir] = 1.f / sqrtf(ss / D + eps);
      }
      const int64_t orow = b * NL + (int64_t)t * N + n;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          // ya: dims 32dt + 16pp + 4h + e, yb: dims 32dt + 16pp + 8 + 4h + e; after the swap
          // the lane holds dims 32dt + 16pp + 8h + {0..3} in ya and + {4..7} in yb
          float ya[4], yb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int da = 32 * dt + 16 * pp + 4 * h + e;
            ya[e] = (acc[0][tt][dt][8 * pp + e] * rn[0] + acc[1][tt][dt][8 * pp + e] * rn[1]) * wl[da];
            yb[e] = (acc[0][tt][dt][8 * pp + 4 + e] * rn[0] + acc[1][tt][dt][8 * pp + 4 + e] * rn[1]) * wl[da + 8];
            const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(ya[e]), __float_as_uint(yb[e]),
                                                            false, false);
            ya[e] = __uint_as_float(x[0]);
            yb[e] = __uint_as_float(x[1]);
          }
          bf16x8 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ga = gate ? (float)gv[tt][dt][pp][e] : 1.f;
            const float gb = gate ? (float)gv[tt][dt][pp][4 + e] : 1.f;
            ov[e] = (bf16)(ya[e] * ga);        // the only rounding of the output
            ov[4 + e] = (bf16)(yb[e] * gb);
          }
          if (n < N) *reinterpret_cast<bf16x8*>(out + orow * ldo + hh * D + 32 * dt + 16 * pp + 8 * h) = ov;
        }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[tt][ks] = qn[tt][ks];
  }
}

// ---------------------------------------------------------------------------
template <typename T>
static hipError_t gram_t(int d, const void* k, const void* v, const float* beta, float* A,
                         float* Bm, int nframes, int T_, int N, int Lt, hipStream_t st) {
  if (sizeof(T) == 2 && d == 128)
    vda_gram_bf16_d128_kernel<<<nframes, 256, 0, st>>>((const bf16*)k, (const bf16*)v, beta, A, Bm, T_, N, Lt);
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
  if (d == 128) {
    const int total = BH * 8;   // 4 row blocks x 2 directions per (batch, head)
    vda_scan_d128_kernel<<<total, 256, 0, st>>>(Mt, Bm, gamma, states, split, T, bhtdd, total);
    return hipGetLastError();
  }
  dim3 grid(d / kScanRows, BH, 2);
  if (d == 32) vda_scan_kernel<32, kScanRows><<<grid, 256, 0, st>>>(Mt, Bm, gamma, states, split, T, bhtdd);
  else vda_scan_kernel<64, kScanRows><<<grid, 256, 0, st>>>(Mt, Bm, gamma, states, split, T, bhtdd);
  return hipGetLastError();
}

template <typename T>
static hipError_t readout_t(int d, const void* q, const float* states, const bf16* split,
                            const float* rms_w, const void* gate, int64_t ldg, void* out, int64_t ldo,
                            int B, int H, int T_, int N, int Lt, float eps, hipStream_t st) {
  const int64_t bhtdd = (int64_t)B * H * T_ * d * d;
  if (sizeof(T) == 2 && d == 128 && split) {
    const int64_t nb = (int64_t)B * H * T_;
    if (nb == 0) return hipSuccess;
    vda_readout_bf16_d128_kernel<<<(unsigned)nb, 256, 0, st>>>((const bf16*)q, split, rms_w, (const bf16*)gate,
                                                               ldg, (bf16*)out, ldo, H, T_, N, Lt, eps, bhtdd);
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
