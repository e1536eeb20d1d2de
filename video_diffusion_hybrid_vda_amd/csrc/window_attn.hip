// Softmax branch of Video DeltaNet: sliding-window attention at VAE-chunk
// granularity with two-way boundary anchors (10100.com article on Video
// DeltaNet, 方法概述 part 1).  A query frame in chunk c = t / C sees the key
// frames of chunks c-W .. c+W plus the first and last frame; the first and
// last frame see every frame.  Context (text / audio) tokens, when present,
// follow the video tokens: every interaction that involves one stays on the
// full softmax (same article, part 1, last sentence), so a video query also
// sees every context token and a context query sees everything.  One softmax
// runs over the union of allowed keys; the output is multiplied by the
// branch gate.
//
// Flash-style forward on MFMA.  Each wave owns 32 queries and computes
// S^T = K Q^T so that every lane holds scores of a single query: the online
// softmax statistics are per lane, and the bf16 P^T tile feeds the P V
// product as the MFMA B operand without any register shuffle (the key order
// inside one 32-key step is permuted identically for P^T and V^T).
// Dense query groups (the anchor frames and the context tokens), whose key
// set is the whole sequence, are split along the keys; a merge kernel
// combines the partial (max, sum, output) triples.
#include <math.h>

#include "vdn_common.h"
#include "vdn_internal.h"

namespace vdn {

// One softmax work item: a tile of query tokens [qbeg, qend) of one (batch,
// head) with up to four key-token intervals [kb, ke); split != 0 marks one
// key split of a dense group's rows: its partials go to row pbase + query of
// the partial buffers (read by the merge kernel).
struct WorkItem {
  int bh, b, h, qbeg, qend, nint, split;
  int64_t pbase;   // may be negative: only pbase + query row is an index
  int kb[4], ke[4];
};

__device__ __forceinline__ WorkItem decode_work(const AttnParams& p, int BM) {
  WorkItem wi;
  const int lid = xcd_remap(blockIdx.x, p.total);
  wi.bh = lid / p.tiles_per_bh;
  const int w = lid - wi.bh * p.tiles_per_bh;
  wi.b = wi.bh / p.H;
  wi.h = wi.bh - wi.b * p.H;
  wi.nint = 0;
  wi.split = 0;
  wi.pbase = 0;
  if (w < p.n_window_tiles) {
    int c, j;
    if (p.nC == 1 || w < p.tiles0) {
      c = 0;
      j = w;
    } else if (w < p.tiles0 + (p.nC - 2) * p.tilesM) {
      const int u = w - p.tiles0;
      c = 1 + u / p.tilesM;
      j = u - (c - 1) * p.tilesM;
    } else {
      c = p.nC - 1;
      j = w - p.tiles0 - (p.nC - 2) * p.tilesM;
    }
    const int qf0 = max(c * p.C, p.a0);
    const int qf1 = min((c + 1) * p.C, p.T - p.a1);
    wi.qbeg = qf0 * p.N + j * BM;
    wi.qend = min(wi.qbeg + BM, qf1 * p.N);
    const int kf0 = max(0, (c - p.W) * p.C);
    const int kf1 = min(p.T, (c + p.W + 1) * p.C);
    if (p.a0 && kf0 > 0) { wi.kb[wi.nint] = 0; wi.ke[wi.nint] = p.N; ++wi.nint; }
    wi.kb[wi.nint] = kf0 * p.N; wi.ke[wi.nint] = kf1 * p.N; ++wi.nint;
    if (p.a1 && kf1 < p.T) { wi.kb[wi.nint] = (p.T - 1) * p.N; wi.ke[wi.nint] = p.L; ++wi.nint; }
    if (p.ctx > 0) { wi.kb[wi.nint] = p.L; wi.ke[wi.nint] = p.Lt; ++wi.nint; }
  } else {
    int u = w - p.n_window_tiles;
    int g = 0;
#pragma unroll
    for (int i = 0; i < kMaxDenseGroups - 1; ++i)
      if (g == i && i < p.nG - 1 && u >= p.nsplit * p.grp_tiles[i]) {
        u -= p.nsplit * p.grp_tiles[i];
        g = i + 1;
      }
    const int tiles_g = g == 0 ? p.grp_tiles[0] : (g == 1 ? p.grp_tiles[1] : p.grp_tiles[2]);
    const int row0 = g == 0 ? p.grp_row0[0] : (g == 1 ? p.grp_row0[1] : p.grp_row0[2]);
    const int rows = g == 0 ? p.grp_rows[0] : (g == 1 ? p.grp_rows[1] : p.grp_rows[2]);
    const int part = g == 0 ? p.grp_part[0] : (g == 1 ? p.grp_part[1] : p.grp_part[2]);
    const int s = u / tiles_g;
    const int j = u - s * tiles_g;
    wi.qbeg = row0 + j * BM;
    wi.qend = min(wi.qbeg + BM, row0 + rows);
    wi.kb[0] = s * p.keys_per_split;
    wi.ke[0] = min(wi.kb[0] + p.keys_per_split, p.Lt);
    wi.nint = 1;
    wi.split = p.nsplit > 1;
    if (wi.split)
      wi.pbase = ((int64_t)wi.bh * p.nsplit + s) * p.dense_rows + part - row0;
  }
  for (int i = wi.nint; i < 4; ++i) { wi.kb[i] = 0; wi.ke[i] = 0; }
  // Every field is uniform across the workgroup; the runtime integer divisions
  // above run on the vector unit, so pin the results to scalar registers.
  wi.bh = __builtin_amdgcn_readfirstlane(wi.bh);
  wi.b = __builtin_amdgcn_readfirstlane(wi.b);
  wi.h = __builtin_amdgcn_readfirstlane(wi.h);
  wi.qbeg = __builtin_amdgcn_readfirstlane(wi.qbeg);
  wi.qend = __builtin_amdgcn_readfirstlane(wi.qend);
  wi.nint = __builtin_amdgcn_readfirstlane(wi.nint);
  wi.split = __builtin_amdgcn_readfirstlane(wi.split);
  const int plo = __builtin_amdgcn_readfirstlane((int)(wi.pbase & 0xffffffff));
  const int phi = __builtin_amdgcn_readfirstlane((int)(wi.pbase >> 32));
  wi.pbase = ((int64_t)phi << 32) | (uint32_t)plo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wi.kb[i] = __builtin_amdgcn_readfirstlane(wi.kb[i]);
    wi.ke[i] = __builtin_amdgcn_readfirstlane(wi.ke[i]);
  }
  return wi;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void window_attn_kernel(AttnParams p) {
  using MM = Mma<T>;
  constexpr int KP = MM::kPack, KS = MM::kStep;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int BM = kAttnBM, BN = kAttnBN;   // the generic kernel's query tile
  constexpr int QW = BM / 4;           // queries per wave
  constexpr int QT = QW / 16;          // query column tiles per wave
  constexpr int KT = BN / 16;          // key row tiles per key tile
  constexpr int DT = D / 16;           // head-dim tiles
  constexpr int KSTEPS = D / KS;
  constexpr int LDK = D + EPC;         // K tile row stride (elements)
  constexpr int LDV = BN + EPC;        // V^T tile row stride (elements)
  constexpr int CPR = D / EPC;         // 16-byte chunks per token row
  __shared__ __attribute__((aligned(16))) T Ks[BN * LDK];
  __shared__ __attribute__((aligned(16))) T Vt[D * LDV];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane % 16, lg = lane / 16;

  // ---- decode the work item
  const WorkItem wi = decode_work(p, BM);
  const int bh = wi.bh, b = wi.b, h = wi.h, qbeg = wi.qbeg, qend = wi.qend, nint = wi.nint;
  const int64_t pbase = wi.pbase;
  const int split = wi.split;
  const int NL = p.Lt;   // rows per (batch, head)
  int kb[4], ke[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { kb[i] = wi.kb[i]; ke[i] = wi.ke[i]; }

  const T* Qb = (const T*)p.q + (int64_t)bh * NL * D;
  const T* Kb = (const T*)p.k + (int64_t)bh * NL * D;
  const T* Vb = (const T*)p.v + (int64_t)bh * NL * D;

  // ---- Q fragments (MFMA B operand of S^T = K Q^T), resident for the whole tile
  typename MM::Frag qf[QT][KSTEPS];
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    const int qrow = qbeg + wave * QW + j * 16 + li;
    const bool ok = qrow < qend;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[j][ks] = ok ? MM::load(Qb + (int64_t)qrow * D + ks * KS + lg * KP) : MM::zero();
  }

  f32x4 o[DT][QT];
  float mrun[QT], lrun[QT];
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    mrun[j] = -INFINITY;
    lrun[j] = 0.f;
#pragma unroll
    for (int di = 0; di < DT; ++di) o[di][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int iv = 0; iv < nint; ++iv) {
    for (int k0 = kb[iv]; k0 < ke[iv]; k0 += BN) {
      const int kn = min(BN, ke[iv] - k0);
      __syncthreads();
      // K tile row-major, V tile transposed (d-major) for the P V operand.
      for (int c = tid; c < BN * CPR; c += 256) {
        const int row = c % BN, cc = c / BN;
        Chunk16 kv = zero_chunk(), vv = zero_chunk();
        if (row < kn) {
          kv = *reinterpret_cast<const Chunk16*>(Kb + (int64_t)(k0 + row) * D + cc * EPC);
          vv = *reinterpret_cast<const Chunk16*>(Vb + (int64_t)(k0 + row) * D + cc * EPC);
        }
        *reinterpret_cast<Chunk16*>(Ks + row * LDK + cc * EPC) = kv;
        const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
        for (int x = 0; x < EPC; ++x) Vt[(cc * EPC + x) * LDV + row] = ve[x];
      }
      __syncthreads();

      // S^T tile: s[i][j][r] = score(key i*16 + lg*4 + r, query j*16 + li)
      f32x4 s[KT][QT];
#pragma unroll
      for (int i = 0; i < KT; ++i)
#pragma unroll
        for (int j = 0; j < QT; ++j) s[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int i = 0; i < KT; ++i) {
          const typename MM::Frag kf = MM::load(Ks + (i * 16 + li) * LDK + ks * KS + lg * KP);
#pragma unroll
          for (int j = 0; j < QT; ++j) s[i][j] = MM::run(kf, qf[j][ks], s[i][j]);
        }

      // online softmax, base 2, per query column
#pragma unroll
      for (int j = 0; j < QT; ++j) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < KT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (i * 16 + lg * 4 + r < kn) mx = fmaxf(mx, s[i][j][r]);
            else s[i][j][r] = -INFINITY;
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrun[j], mx * p.scale_log2);
        const float alpha = fast_exp2(mrun[j] - mnew);
        mrun[j] = mnew;
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < KT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = fast_exp2(s[i][j][r] * p.scale_log2 - mnew);
            s[i][j][r] = e;
            ps += e;
          }
        lrun[j] = lrun[j] * alpha + ps;
#pragma unroll
        for (int di = 0; di < DT; ++di) o[di][j] *= alpha;
      }

      // O^T += V^T P^T
      if constexpr (KP == 8) {
        // one 32-key step: slot lg*8+e <-> key 32*s2 + 16*(e/4) + 4*lg + e%4
#pragma unroll
        for (int s2 = 0; s2 < BN / 32; ++s2) {
          bf16x8 pf[QT];
#pragma unroll
          for (int j = 0; j < QT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pf[j][e] = (bf16)s[2 * s2][j][e];
              pf[j][4 + e] = (bf16)s[2 * s2 + 1][j][e];
            }
#pragma unroll
          for (int di = 0; di < DT; ++di) {
            const bf16* vrow = reinterpret_cast<const bf16*>(Vt) + (di * 16 + li) * LDV + 32 * s2 + lg * 4;
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 16);
            const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int j = 0; j < QT; ++j) o[di][j] = MM::run((typename MM::Frag)vf, (typename MM::Frag)pf[j], o[di][j]);
          }
        }
      } else {
        // fp32: one 4-key step per (key tile i, register r): slot lg <-> key i*16 + 4*lg + r
#pragma unroll
        for (int i = 0; i < KT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int di = 0; di < DT; ++di) {
              const typename MM::Frag vf = (typename MM::Frag)Vt[(di * 16 + li) * LDV + i * 16 + lg * 4 + r];
#pragma unroll
              for (int j = 0; j < QT; ++j)
                o[di][j] = MM::run(vf, (typename MM::Frag)s[i][j][r], o[di][j]);
            }
      }
    }
  }

  // ---- epilogue
  const T* gate = (const T*)p.gate;
  T* out = (T*)p.out;
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    float l = lrun[j];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int qrow = qbeg + wave * QW + j * 16 + li;
    if (qrow >= qend) continue;
    if (!split) {
      const float inv = 1.f / l;
      const int64_t orow = (int64_t)b * NL + qrow;
#pragma unroll
      for (int di = 0; di < DT; ++di)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int dd = di * 16 + lg * 4 + r;
          float val = o[di][j][r] * inv;
          if (gate) val *= to_f32(gate[orow * p.ldg + h * D + dd]);
          out[orow * p.ldo + h * D + dd] = from_f32<T>(val);
        }
      if (p.lse && lg == 0) p.lse[(int64_t)bh * NL + qrow] = (mrun[j] + log2f(l)) * kLn2;
    } else {
      const int64_t prow = pbase + qrow;
#pragma unroll
      for (int di = 0; di < DT; ++di)
#pragma unroll
        for (int r = 0; r < 4; ++r) p.part_o[prow * D + di * 16 + lg * 4 + r] = o[di][j][r];
      if (lg == 0) {
        p.part_ml[prow * 2] = mrun[j];
        p.part_ml[prow * 2 + 1] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16, head_dim 128: the production kernel for the workload shapes.
//
// 256 queries per workgroup: 4 waves x 64 queries (one wave per SIMD, the
// default) or 8 waves x 32 queries (two per SIMD); both measure the same on
// the workload.  64-key tiles; 32x32x16 MFMA.  K and V tiles are copied global -> LDS by the
// direct-to-LDS DMA path (a buffer load with the lds modifier: lane l writes
// bytes [16 l, 16 l + 16) of a 1 KB block) through a four-stage ring, so
// tiles t+1 .. t+3 stream in while tile t is consumed; one barrier per tile.
// Both tiles stay row-major in LDS with the 16-byte chunks of each row
// XOR-swizzled; K fragments are plain 16-byte LDS reads, V fragments are
// ds_read_b64_tr_b16 transpose reads.  Within a group of 16 lanes that
// instruction hands lane i the element i%4 of the 8-byte loads of lanes i/4,
// 4+i/4, 8+i/4, 12+i/4, so a group that loads a 4-key x 16-dim block of
// row-major V receives, per lane, four consecutive keys of one dimension:
// the MFMA A operand of O^T = V^T P^T.
//
// With one wave per SIMD the vector work of the softmax only overlaps the
// matrix work if the wave's own instruction stream interleaves them, so the
// loop is software-pipelined over half tiles of 32 keys: while the matrix
// unit computes the scores of half tile j+1 and then P V of half tile j, the
// vector unit computes the exponentials of half tile j and then the max of
// half tile j+1.  Scores are produced in vector registers (the softmax reads
// them there), O, Q and the row sums live in the accumulator registers; the
// row sums are ones^T P^T on the matrix unit, because the vector unit is the
// busier one.
//
// The running max is refreshed lazily: the output accumulators are rescaled
// only when some row max of the wave grows by more than 1 in log2 units, so
// probabilities stay <= 2.  On the near-uniform softmax of unit-norm keys this
// never triggers after the first tile; on peaked softmax it keeps the
// dominant probability at (or next to) 1, as exact as a strict running max.
namespace v2 {
constexpr int BM = 256, BN = 64, D = 128, STAGES = 4;
constexpr int kAttnQT = 2;          // query tiles of 32 per wave: 8 / kAttnQT waves per workgroup
constexpr int ROWB = D * 2;          // bytes per K/V row
constexpr int TILEB = BN * ROWB;     // 16 KB
constexpr int STAGEB = 2 * TILEB;    // K tile then V tile
constexpr float kRescaleSlack = 1.f;
constexpr int kWaitVm0 = 0x0F70;   // s_waitcnt vmcnt(0) (gfx9 encoding; expcnt and lgkmcnt not waited for)
constexpr int kWaitVm8 = 0x0F78;   // s_waitcnt vmcnt(8): at most the last 8 DMA loads outstanding
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Physical 16-byte chunk of logical chunk c in row r.  For 16 consecutive
// rows at a fixed chunk (K reads) the 16 results are distinct; for 8 aligned
// rows x 4 aligned chunks (V transpose reads) each value appears twice, i.e.
// two passes over the 64 banks, the minimum for 512 bytes.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r & 7) << 1) | ((r >> 3) & 1)); }

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Scheduling fences.  pin(x) makes x look redefined at this point, so code
// that produces x stays above it and code that consumes x stays below it;
// chunk_fence() keeps memory operations on their side and ends a machine
// scheduling region.  Both emit no instructions.
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }
template <typename T>
__device__ __forceinline__ void pin_acc(T& x) { asm volatile("" : "+a"(x)); }   // same, in the accumulator file
__device__ __forceinline__ void chunk_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Score products written out so that their results land in vector registers
// (where the softmax reads them) while O stays in the accumulator file.  The
// first step of a chain starts from zero, later steps accumulate in place
// (back-to-back accumulation into the same registers needs no wait states);
// the vector unit reads a score buffer only eight or more MFMAs after its last
// write.
__device__ __forceinline__ void mma_first(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mma_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// max of x over lanes i and i ^ 32 (the swap exchanges the upper half of the
// first operand with the lower half of the second)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
}  // namespace v2

template <int QT>
__global__ __launch_bounds__(512 / QT) void window_attn_bf16_d128_kernel(AttnParams p) {
  using namespace v2;
  constexpr int NW = 8 / QT;          // waves per workgroup
  constexpr int WQ = 32 * QT;         // queries per wave
  constexpr int BLK = 16 / NW;        // 1 KB DMA blocks per wave and operand of a tile
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STAGES * STAGEB];

  // wave index as a scalar: the DMA's LDS destination (M0) must be wave-uniform
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, h = lane / 32, g = lane / 16, j16 = lane % 16;

  const WorkItem wi = decode_work(p, BM);
  const int NL = p.Lt;   // rows per (batch, head)
  const bf16* Qb = (const bf16*)p.q + (int64_t)wi.bh * NL * D;
  const bf16* Kb = (const bf16*)p.k + (int64_t)wi.bh * NL * D;
  const bf16* Vb = (const bf16*)p.v + (int64_t)wi.bh * NL * D;

  int ntiles = 0;
#pragma unroll
  for (int iv = 0; iv < 4; ++iv)
    if (iv < wi.nint) ntiles += (wi.ke[iv] - wi.kb[iv] + BN - 1) / BN;

  // Loader.  One buffer descriptor per tensor covering this (batch, head):
  // rows past its end read as zero; rows past the end of a key interval are
  // real keys of other frames and are masked out of the softmax.  Each
  // lane's byte offset inside a 64-row tile is fixed: row blk*4 + lane/16,
  // logical chunk swz(row, lane%16) lands at physical chunk lane%16.
  int lane_off[BLK];
#pragma unroll
  for (int i = 0; i < BLK; ++i) {
    const int row = (wave * BLK + i) * 4 + lane / 16;
    lane_off[i] = row * ROWB + swz(row, lane % 16) * 16;
  }
  // interval bounds picked without dynamic indexing, as wave-uniform scalars
  const int kb0 = wi.kb[0], kb1 = wi.kb[1], kb2 = wi.kb[2], kb3 = wi.kb[3];
  const int ke0 = wi.ke[0], ke1 = wi.ke[1], ke2 = wi.ke[2], ke3 = wi.ke[3];
  auto kb_of = [&](int i) { return i == 0 ? kb0 : (i == 1 ? kb1 : (i == 2 ? kb2 : kb3)); };
  auto ke_of = [&](int i) { return i == 0 ? ke0 : (i == 1 ? ke1 : (i == 2 ? ke2 : ke3)); };
  int liv = 0, lk0 = kb_of(0), lke = ke_of(0);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)Kb, (short)0, NL * ROWB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)Vb, (short)0, NL * ROWB, 0x00020000);
  // The DMA is written as an opaque instruction: the compiler would otherwise
  // make every later LDS read wait for it (it cannot tell the stages apart);
  // the loop below waits for each tile's loads explicitly (vmcnt) before the
  // barrier that publishes the tile.
  auto issue = [&](int st) {
    const int base = lk0 * ROWB;
    const int lds = (int)(size_t)(__attribute__((address_space(3))) unsigned char*)ring;
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
      const int blk = wave * BLK + i;
      const int voff = base + lane_off[i];
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rk),
                   "{m0}"(lds + st * TILEB + blk * 1024)
                   : "memory");
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rv),
                   "{m0}"(lds + (STAGES + st) * TILEB + blk * 1024)
                   : "memory");
    }
    lk0 += BN;
    if (lk0 >= lke) {
      ++liv;
      if (liv < wi.nint) {
        lk0 = kb_of(liv);
        lke = ke_of(liv);
      }
    }
  };

  // ring of four 64-key stages: tiles t+1 .. t+3 resident or in flight while
  // tile t is consumed
  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  if (ntiles > 2) issue(2);

  // Q fragments: B operand of S^T = K Q^T; lane holds Q[query l32][16 ks + 8 h .. +7]
  bf16x8 qf[QT][8];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qrow = wi.qbeg + wave * WQ + qt * 32 + l32;
    const bool ok = qrow < wi.qend;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qf[qt][ks] = ok ? *reinterpret_cast<const bf16x8*>(Qb + (int64_t)qrow * D + ks * 16 + h * 8)
                      : bf16x8{};
  }
  // Q lives in the accumulator file (the score products read it from there)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) pin_acc(qf[qt][ks]);

  // O^T accumulators and the row sums of p: lsum[qt] = ones^T P^T on the
  // matrix unit, so every register of a lane holds the full row sum of its
  // query (of the bf16 p, the weights the P V product uses)
  f32x16 o[4][QT], lsum[QT];
  float mrun[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = -INFINITY;
    lsum[qt] = f32x16{};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt][qt] = f32x16{};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.f;
  const float c2 = p.scale_log2;
  // compute cursor: first key and interval end of the tile whose scores are
  // the most recent ones
  int civ = 0, ck0 = kb_of(0), cke = ke_of(0);
  auto advance = [&]() {
    ck0 += BN;
    if (ck0 >= cke) {
      ++civ;
      if (civ < wi.nint) {
        ck0 = kb_of(civ);
        cke = ke_of(civ);
      }
    }
  };

  // Q and the first three tiles resident; no vector-memory load is pending
  // anywhere in the loop except the DMA the loop itself waits for
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  // The softmax runs on half tiles of 32 keys.  Scores of two half tiles are
  // live at once: the current one (read by the softmax) and the next one
  // (written by the matrix unit meanwhile).  sc[qt] register r holds the
  // score of key 8(r/4) + 4h + r%4 of the half tile for query 32 qt + l32.
  f32x16 sa[QT], sb[QT];
  float mtile[QT];

  // Fragment reads.  The ring keeps the K tiles of the four stages in its
  // first 64 KB and the V tiles in the second, so every read is a per-lane
  // base register (fixed for the kernel) plus a constant below 64 KB (stage,
  // half tile, key step) that the LDS instruction carries in its offset field.
  // The swizzle depends on row % 16 only, and the constants move whole
  // 16-row groups.
  int koff[8], voffA[4], voffB[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    koff[ks] = l32 * ROWB + swz(l32, 2 * ks + h) * 16;
    pin(koff[ks]);
  }
  {
    const int rA = 4 * (g >> 1) + (j16 >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int dcol = dt * 32 + 16 * (g & 1) + 4 * (j16 & 3);
      const int cch = dcol >> 3, off = (dcol & 7) * 2;
      voffA[dt] = STAGES * TILEB + rA * ROWB + swz(rA, cch) * 16 + off;
      voffB[dt] = STAGES * TILEB + (rA + 8) * ROWB + swz(rA + 8, cch) * 16 + off;
      pin(voffA[dt]);
      pin(voffB[dt]);
    }
  }
  // K fragment of 16-column step ks, rows 32 kt + l32 of stage st
  auto load_k = [&](int st, int kt, int ks) {
    return *reinterpret_cast<const bf16x8*>(ring + koff[ks] + st * TILEB + kt * 32 * ROWB);
  };
  // V^T fragments of 16-key step s4 of stage st for the four 32-wide column blocks
  auto load_v = [&](bf16x8 (&vf)[4], int st, int s4) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int c = st * TILEB + s4 * 16 * ROWB;
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ring + voffA[dt] + c));
      const i16x4 vv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ring + voffB[dt] + c));
      vf[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vv, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // keys >= lim of a half tile get score -inf
  auto mask = [&](f32x16 (&sc)[QT], int lim) {
    const int l = lim - 4 * h;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r / 4) + (r % 4) >= l) sc[qt][r] = -INFINITY;
  };
  // raise the running max to the tile max if it outruns it by more than the
  // slack, rescaling O and the row sums
  auto refresh = [&]() {
    bool up = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) up |= mtile[qt] > mrun[qt] + kRescaleSlack;
    if (__any(up)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mnew = fmaxf(mrun[qt], mtile[qt]);
        const float alpha = fast_exp2(mrun[qt] - mnew);
        mrun[qt] = mnew;
        pin_acc(lsum[qt]);
        lsum[qt] *= alpha;
        pin_acc(lsum[qt]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          pin_acc(o[dt][qt]);   // O is copied out here, not on the common path
          o[dt][qt] *= alpha;
          pin_acc(o[dt][qt]);
        }
      }
    }
  };

  // per-query max of a half tile's scores (scaled, base 2) in mtile; the two
  // half-waves hold the two key halves of each query
  auto half_max = [&](const f32x16 (&sc)[QT]) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = sc[qt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[qt][r]);
      mtile[qt] = halves_max(mx) * c2;
      pin(mtile[qt]);
    }
  };
  // between half steps: mask a partial half tile (keys >= lim), then raise
  // the running max if needed; neither happens on most half tiles
  auto boundary = [&](f32x16 (&sc)[QT], int lim) {
    if (lim < 32) {
      asm volatile("");   // a real branch: the masking stays off the common path
      mask(sc, lim);
      half_max(sc);
    }
    refresh();
  };

  // One half step: the softmax and P V of the current half tile (scores in
  // cur, half pkt of the tile in stage pst) run beside the scores of the next
  // half tile (half skt of the tile in stage sst), which are then reduced to
  // their max; the matrix unit works while the vector unit does the
  // exponentials.  It is laid out as chunks (one 16-column step of the scores
  // or one 16-key step of P V, each with its share of vector work and the
  // operand reads of a later chunk) that are fenced against each other: the
  // score chunks carry p of the first 16 keys, the first P V chunk p of the
  // other 16, the second P V chunk the max of the next scores.  p is rounded
  // to bf16 for the products.
  auto half_step = [&](const f32x16 (&cur)[QT], f32x16 (&nxt)[QT], int sst, int skt, int pst,
                       int pkt) __attribute__((always_inline)) {
    bf16x8 kf[3], vf[2][4], pk[QT][2];
    // p of register r of query tile qt (16-key step r / 8)
    auto soft1 = [&](int qt, int r) {
      pk[qt][r >> 3][r & 7] = (bf16)fast_exp2(fmaf(cur[qt][r], c2, -mrun[qt]));
    };
    kf[0] = load_k(sst, skt, 0);
    kf[1] = load_k(sst, skt, 1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      chunk_fence();
      if (ks < 6) kf[(ks + 2) % 3] = load_k(sst, skt, ks + 2);
      if (ks == 6) load_v(vf[0], pst, 2 * pkt);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if (ks == 0) mma_first(nxt[qt], kf[ks % 3], qf[qt][ks]);
        else mma_acc(nxt[qt], kf[ks % 3], qf[qt][ks]);
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        soft1(qt, ks);
        pin(pk[qt][0]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
    chunk_fence();
    load_v(vf[1], pst, 2 * pkt + 1);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt][qt] = mma(vf[0][dt], pk[qt][0], o[dt][qt]);
      lsum[qt] = mma(ones, pk[qt][0], lsum[qt]);
    }
#pragma unroll
    for (int r = 8; r < 16; ++r)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) soft1(qt, r);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) pin(pk[qt][1]);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 5 * QT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    chunk_fence();
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt][qt] = mma(vf[1][dt], pk[qt][1], o[dt][qt]);
      lsum[qt] = mma(ones, pk[qt][1], lsum[qt]);
    }
    half_max(nxt);
#pragma unroll
    for (int i = 0; i < 5 * QT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    chunk_fence();
  };

  int kn = min(BN, cke - ck0);   // keys of tile t
  if (ntiles > 0) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 kf = load_k(0, 0, ks);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if (ks == 0) mma_first(sa[qt], kf, qf[qt][ks]);
        else mma_acc(sa[qt], kf, qf[qt][ks]);
      }
    }
    // the vector unit reads the scores next: wait for the last products
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    half_max(sa);
    boundary(sa, kn);
  }
  // One tile: its two halves; the second computes the scores of the first
  // half of tile t+1 (for the last tile they come from a stale stage and are
  // never used).  Tile t sits in ring stage t % 4; the loop is unrolled over
  // the four stages so that every stage offset is a constant (it folds into
  // the LDS instructions' offset field instead of costing an add per read).
  auto tile = [&](int t, int s0, int s1, int s3) __attribute__((always_inline)) {
    if (t + 3 < ntiles) issue(s3);
    half_step(sa, sb, s0, 1, s0, 0);
    boundary(sb, kn - 32);
    half_step(sb, sa, s1, 0, s0, 1);
    advance();
    kn = min(BN, cke - ck0);
    if (t + 3 < ntiles) __builtin_amdgcn_s_waitcnt(kWaitVm8);
    else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (t + 1 < ntiles) boundary(sa, kn);
  };
  for (int t = 0; t < ntiles; t += 4) {
    tile(t, 0, 1, 3);
    if (t + 1 >= ntiles) break;
    tile(t + 1, 1, 2, 0);
    if (t + 2 >= ntiles) break;
    tile(t + 2, 2, 3, 1);
    if (t + 3 >= ntiles) break;
    tile(t + 3, 3, 0, 2);
  }

  // ---- epilogue: o[dt][qt][r] = O(query 32 qt + l32, dim 32 dt + 8(r/4) + 4h + r%4)
  const bf16* gate = (const bf16*)p.gate;
  bf16* out = (bf16*)p.out;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = lsum[qt][0];
    const int qrow = wi.qbeg + wave * WQ + qt * 32 + l32;
    if (qrow >= wi.qend) continue;
    if (!wi.split) {
      const float inv = 1.f / lt;
      const int64_t orow = (int64_t)wi.b * NL + qrow;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = dt * 32 + 8 * r4 + 4 * h;
          float v0 = o[dt][qt][4 * r4] * inv, v1 = o[dt][qt][4 * r4 + 1] * inv;
          float v2 = o[dt][qt][4 * r4 + 2] * inv, v3 = o[dt][qt][4 * r4 + 3] * inv;
          if (gate) {
            const bf16x4 gv = *reinterpret_cast<const bf16x4*>(gate + orow * p.ldg + wi.h * D + d0);
            v0 *= (float)gv[0]; v1 *= (float)gv[1]; v2 *= (float)gv[2]; v3 *= (float)gv[3];
          }
          bf16x4 ov;
          ov[0] = (bf16)v0; ov[1] = (bf16)v1; ov[2] = (bf16)v2; ov[3] = (bf16)v3;
          *reinterpret_cast<bf16x4*>(out + orow * p.ldo + wi.h * D + d0) = ov;
        }
      if (p.lse && h == 0) p.lse[(int64_t)wi.bh * NL + qrow] = (mrun[qt] + log2f(lt)) * kLn2;
    } else {
      const int64_t prow = wi.pbase + qrow;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = dt * 32 + 8 * r4 + 4 * h;
          *reinterpret_cast<float4*>(p.part_o + prow * D + d0) =
              make_float4(o[dt][qt][4 * r4], o[dt][qt][4 * r4 + 1], o[dt][qt][4 * r4 + 2], o[dt][qt][4 * r4 + 3]);
        }
      if (h == 0) {
        p.part_ml[prow * 2] = mrun[qt];
        p.part_ml[prow * 2 + 1] = lt;
      }
    }
  }
}

// Combine the key splits of the dense query rows (anchor frames, context
// tokens): out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, then gate.
// One thread per (dense row, quarter of d).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  const int nqb = (p.dense_rows + 63) / 64;
  const int qb = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb;             // b*H + h
  const int h = bh % p.H, b = bh / p.H;
  const int n = qb * 64 + threadIdx.x / 4;     // index among the dense rows
  if (n >= p.dense_rows) return;
  // the group holding dense row n (groups are stored in row order)
  const int g = (p.nG > 2 && n >= p.grp_part[2]) ? 2 : ((p.nG > 1 && n >= p.grp_part[1]) ? 1 : 0);
  const int qrow = (g == 0 ? p.grp_row0[0] : (g == 1 ? p.grp_row0[1] : p.grp_row0[2])) + n -
                   (g == 0 ? p.grp_part[0] : (g == 1 ? p.grp_part[1] : p.grp_part[2]));
  const int dq = threadIdx.x % 4;
  constexpr int DQ = D / 4;
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s)
    M = fmaxf(M, p.part_ml[(((int64_t)bh * p.nsplit + s) * p.dense_rows + n) * 2]);
  float L = 0.f;
  float acc[DQ];
#pragma unroll
  for (int x = 0; x < DQ; ++x) acc[x] = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const int64_t prow = ((int64_t)bh * p.nsplit + s) * p.dense_rows + n;
    const float wgt = fast_exp2(p.part_ml[prow * 2] - M);
    L += wgt * p.part_ml[prow * 2 + 1];
#pragma unroll
    for (int x = 0; x < DQ; ++x) acc[x] += wgt * p.part_o[prow * D + dq * DQ + x];
  }
  const float inv = 1.f / L;
  const int64_t orow = (int64_t)b * p.Lt + qrow;
  const T* gate = (const T*)p.gate;
  T* out = (T*)p.out;
#pragma unroll
  for (int x = 0; x < DQ; ++x) {
    const int dd = dq * DQ + x;
    float val = acc[x] * inv;
    if (gate) val *= to_f32(gate[orow * p.ldg + h * D + dd]);
    out[orow * p.ldo + h * D + dd] = from_f32<T>(val);
  }
  if (p.lse && dq == 0) p.lse[(int64_t)bh * p.Lt + qrow] = (M + log2f(L)) * kLn2;
}

template <typename T, int D>
static hipError_t launch_attn_t(const AttnParams& p, hipStream_t st) {
  if (p.total > 0) {
    if (attn_uses_v2(sizeof(T) == 2 ? 1 : 0, D))
      window_attn_bf16_d128_kernel<v2::kAttnQT><<<p.total, 512 / v2::kAttnQT, 0, st>>>(p);
    else
      window_attn_kernel<T, D><<<p.total, 256, 0, st>>>(p);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_merge_t(const AttnParams& p, hipStream_t st) {
  if (p.nsplit > 1 && p.nG > 0) {
    const int blocks = p.B * p.H * ((p.dense_rows + 63) / 64);
    attn_merge_kernel<T, D><<<blocks, 256, 0, st>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_window_attn(int dtype, int d, const AttnParams& p, hipStream_t st) {
  if (p.bm != attn_query_tile(dtype, d)) return hipErrorInvalidValue;
  if (dtype == 1) {
    if (d == 32) return launch_attn_t<bf16, 32>(p, st);
    if (d == 64) return launch_attn_t<bf16, 64>(p, st);
    return launch_attn_t<bf16, 128>(p, st);
  }
  if (d == 32) return launch_attn_t<float, 32>(p, st);
  if (d == 64) return launch_attn_t<float, 64>(p, st);
  return launch_attn_t<float, 128>(p, st);
}

hipError_t launch_attn_merge(int dtype, int d, const AttnParams& p, hipStream_t st) {
  if (dtype == 1) {
    if (d == 32) return launch_merge_t<bf16, 32>(p, st);
    if (d == 64) return launch_merge_t<bf16, 64>(p, st);
    return launch_merge_t<bf16, 128>(p, st);
  }
  if (d == 32) return launch_merge_t<float, 32>(p, st);
  if (d == 64) return launch_merge_t<float, 64>(p, st);
  return launch_merge_t<float, 128>(p, st);
}

}  // namespace vdn
