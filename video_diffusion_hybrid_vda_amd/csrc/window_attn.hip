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

#include <type_traits>
#include <utility>

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

// append interval [b, e) to the item's list; the slot is picked by comparing
// with constants so that the item stays in registers (a store at a runtime
// index would put it in memory)
__device__ __forceinline__ void push(WorkItem& wi, int b, int e) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i == wi.nint) {
      wi.kb[i] = b;
      wi.ke[i] = e;
    }
  ++wi.nint;
}

__device__ __forceinline__ WorkItem decode_work(const AttnParams& p, int BM) {
  WorkItem wi;
  const int lid = xcd_remap(blockIdx.x, p.total);
  wi.bh = lid / p.tiles_per_bh;
  const int w = lid - wi.bh * p.tiles_per_bh;
  wi.b = wi.bh / p.H;
  wi.h = wi.bh - wi.b * p.H;
  wi.nint = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) { wi.kb[i] = 0; wi.ke[i] = 0; }
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
    if (p.a0 && kf0 > 0) push(wi, 0, p.N);
    push(wi, kf0 * p.N, kf1 * p.N);
    if (p.a1 && kf1 < p.T) push(wi, (p.T - 1) * p.N, p.L);
    if (p.ctx > 0) push(wi, p.L, p.Lt);
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
// 256 queries per workgroup: 4 waves x 64 queries, one wave per SIMD.  64-key
// tiles.  K and V tiles are copied global -> LDS by the direct-to-LDS DMA path
// (a buffer load with the lds modifier: lane l writes bytes [16 l, 16 l + 16)
// of a 1 KB block) through a four-stage ring, so tiles t+1 .. t+3 stream in
// while tile t is consumed; one barrier per tile.  Both tiles stay row-major
// in LDS with the 16-byte chunks of each row XOR-swizzled; K fragments are
// plain 16-byte LDS reads, V fragments ds_read_b64_tr_b16 transpose reads.
// Within a group of 16 lanes that instruction hands lane i the element i%4 of
// the 8-byte loads of lanes i/4, 4+i/4, 8+i/4, 12+i/4, so a group that loads a
// 4-key x 16-dim block of row-major V receives, per lane, four consecutive
// keys of one dimension: the MFMA A operand of O^T = V^T P^T.
//
// The wave computes S^T = K Q^T (v_mfma_f32_32x32x16_bf16, Q resident in the
// accumulator registers), so each lane holds scores of one query: the softmax
// statistics are per lane, and the bf16 P^T tile is already laid out as the B
// operand of O^T = V^T P^T (the key order inside each 16-key step is permuted
// identically for P and V).  The row sums are sel^T P^T on a 16x16x32 MFMA,
// where sel picks, for rows 0 and 1, the lanes that hold queries 0-15 and
// 16-31 of the 32-query tile.
//
// Software pipeline over half tiles of 32 keys.  One half step issues 36
// matrix products - the 16 score products of half tile j+1, the 16 P V
// products and 4 row-sum products of half tile j - and, beside them on the
// vector unit, the 32 exponentials of half tile j (p = 2^(s c - m), rounded
// to bf16 in pairs) and the max of half tile j+1's scores.  With one wave per
// SIMD the two units only overlap if the wave's own instruction stream
// alternates them, so the half step is a fixed list of slots, each one matrix
// product followed by its share of vector work and LDS fragment reads, every
// instruction an asm statement so that the compiler keeps the order.  Score
// fragments are read 6 slots ahead and V fragments 6-9 slots ahead, each
// product preceded by an explicit lgkmcnt wait for exactly the reads it
// needs; the next tile's DMA loads are spread over the second half of the
// first half step.  A probe of this instruction mix (36 products, 112 vector
// instructions, 24 LDS reads, 8 DMA loads and a barrier per 72 products)
// measured 1250 cycles per half step against 1156 for the products alone.
//
// The running max is refreshed lazily: the output accumulators are rescaled
// only when some row max of the wave grows by more than 1 in log2 units, so
// probabilities stay <= 2.  On the near-uniform softmax of unit-norm keys this
// never triggers after the first tile; on peaked softmax it keeps the
// dominant probability at (or next to) 1, as exact as a strict running max.
namespace v3 {
constexpr int BM = 256, BN = 64, D = 128, STAGES = 4;
constexpr int NW = 4, WQ = 64, QT = 2, BLK = 4;   // waves, queries per wave, 32-query tiles, DMA blocks
constexpr int ROWB = D * 2;          // bytes per K/V row
constexpr int TILEB = BN * ROWB;     // 16 KB
constexpr int VBASE = STAGES * TILEB;   // V tiles follow the four K tiles
constexpr float kRescaleSlack = 1.f;
// log2 units: the largest bound the fixed maximum takes.  A row's scores then
// lie within +-4 of 0, so no key outweighs another by more than 2^8 and no row
// is peaked; peaked rows, whose error rests on the dominant probability being
// exactly 1, keep the running maximum.
constexpr float kFixedMaxCap = 4.f;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int V>
using IC = std::integral_constant<int, V>;

// f(IC<B>{}), f(IC<B + 1>{}), ..., f(IC<E - 1>{}): every index a compile-time constant
template <int B, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(IC<B + I>{}), ...);
}
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (E > B) static_for_impl<B>(f, std::make_integer_sequence<int, E - B>{});
}

// Vector work of a half step, in units: unit 3 j + k of pair j (the two
// exponentials of p words (qt, 16-key step s4, word w), j = 8 s4 + 2 w + qt)
// is its first value (k = 0), the conversion of pair j - 1 (k = 1) or its
// second value (k = 2); unit 48 converts the last pair.  36 units (pairs
// 0-11) run beside the 16 score products, the other 13 beside the first five
// P V products.
constexpr int units_before(int m) {
  return m <= 16 ? (36 * m + 8) / 16 : (m <= 21 ? 36 + (13 * (m - 16) + 2) / 5 : 49);
}

// Issue slots of a half step's LDS fragment reads and of a tile's DMA loads.
// K fragment ks of a half step is read in slot kIssueK[ks] of it or, when
// negative, in slot 36 + kIssueK[ks] of the half step before; V half-fragment
// i = 8 s4 + 2 dt + ab (16-key step s4, 32-dim block dt, rows 0-7 / 8-15) in
// slot kIssueV[i]; DMA load i of the next tile in slot kIssueD[i] of the first
// half step of a tile.  Within a slot, K reads come before V reads.
constexpr int kIssueK[8] = {-8, -6, -4, 0, 2, 4, 6, 8};
constexpr int kIssueV[16] = {9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24};
constexpr int kIssueD[8] = {25, 26, 27, 28, 29, 30, 31, 32};
// issue order keys
constexpr int key_k(int ks) { return kIssueK[ks] * 64 + ks; }
constexpr int key_v(int i) { return kIssueV[i] * 64 + 16 + i; }
// LDS reads issued after the one with key a and before the wait point of
// slot m: this half step's reads, the next half step's K reads issued in this
// one, and the previous half step's reads shifted by one half step.  A wait
// for at most that many outstanding reads completes the read with key a
// (reads complete in order); counting fewer would only wait longer.
constexpr int younger(int a, int m) {
  int n = 0;
  for (int sh = -1; sh <= 0; ++sh) {
    for (int ks = 0; ks < 8; ++ks) {
      const int k = key_k(ks) + sh * 36 * 64;
      if (k > a && k < 64 * m) ++n;
      if (kIssueK[ks] < 0) {   // read in the half step before its own
        const int kn = (kIssueK[ks] + 36) * 64 + ks + sh * 36 * 64;
        if (kn > a && kn < 64 * m && sh == 0) ++n;
      }
    }
    for (int i = 0; i < 16; ++i) {
      const int k = key_v(i) + sh * 36 * 64;
      if (k > a && k < 64 * m) ++n;
    }
  }
  return n < 15 ? n : 15;
}
constexpr int cmax(int a, int b) { return a > b ? a : b; }
// lgkmcnt before the first score product of step ks (slot 2 ks) and before
// the first P V product of 16-key step s4, block dt (slot 16 + 10 s4 + 2 dt)
constexpr int wait_s(int ks) { return younger(key_k(ks), 2 * ks); }
constexpr int wait_p(int s4, int dt) {
  return younger(cmax(key_v(8 * s4 + 2 * dt), key_v(8 * s4 + 2 * dt + 1)), 16 + 10 * s4 + 2 * dt);
}
// every read is consumed in its own half step and issued before the next
// half step's first K read; reads that feed products are issued before them;
// a K fragment buffer (kf[ks % 4]) is rewritten only after its last product
constexpr bool schedule_ok() {
  for (int ks = 0; ks < 8; ++ks) {
    if (kIssueK[ks] >= 2 * ks) return false;
    if (ks >= 4 && kIssueK[ks] <= 2 * (ks - 4) + 1) return false;
    if (kIssueK[ks] >= 0 && kIssueK[ks] >= 36 + kIssueK[0]) return false;
  }
  for (int ks = 0; ks < 3; ++ks)
    if (kIssueK[ks] < 0 && 36 + kIssueK[ks] <= 2 * (ks + 4) + 1) return false;
  for (int i = 0; i < 16; ++i) {
    const int s4 = i / 8, dt = (i % 8) / 2;
    if (kIssueV[i] >= 16 + 10 * s4 + 2 * dt) return false;
    if (kIssueV[i] >= 36 + kIssueK[0]) return false;
    // the previous half step's use of the same registers is over
    if (kIssueV[i] < 0) return false;
  }
  return true;
}
static_assert(schedule_ok(), "LDS read schedule violates its order constraints");

// Physical 16-byte chunk of logical chunk c in row r.  For 16 consecutive
// rows at a fixed chunk (K reads) the 16 results are distinct; for 8 aligned
// rows x 4 aligned chunks (V transpose reads) each value appears twice, i.e.
// two passes over the 64 banks, the minimum for 512 bytes.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r & 7) << 1) | ((r >> 3) & 1)); }

// LDS offset of K fragment (stage st, half kt) relative to the lane's base for
// its score step; of V fragment (stage st, half pt, 16-key step s4) relative
// to the lane's base for its 32-dim block
constexpr int koffc(int st, int kt) { return st * TILEB + kt * 32 * ROWB; }
constexpr int voffc(int st, int pt, int s4) { return st * TILEB + (2 * pt + s4) * 16 * ROWB; }

// ---- the instructions of a slot, each its own asm statement so that their
// order is kept.  Hazards the hardware does not interlock are respected by
// construction: a product's scores are read by the vector unit six or more
// products later, p words are read by a product four or more slots after the
// conversion that writes them, and a conversion never directly follows the
// exponential it reads.

// score product chain in vector registers; Q (b) in the accumulator file
__device__ __forceinline__ void mma_s0(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mma_s(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// P V product into the accumulator file
__device__ __forceinline__ void mma_o(f32x16& o, bf16x8 v, bf16x8 p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}
// row sums: rows 0 and 1 of sel^T P^T
__device__ __forceinline__ void mma_l(f32x4& l, bf16x8 sel, bf16x8 p) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(l) : "v"(sel), "v"(p));
}
template <int OFF>
__device__ __forceinline__ void ds_k(bf16x8& d, int addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_tr(i16x4& d, int addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
}
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
// t = 2^(s c2 - m)
__device__ __forceinline__ void fma_exp(float& t, float s, float c2, float negm) {
  asm volatile("v_fma_f32 %0, %1, %2, %3\n\tv_exp_f32 %0, %0" : "=&v"(t) : "v"(s), "s"(c2), "v"(negm));
}
// t = 2^s (fixed-maximum path: s is already the scaled score)
__device__ __forceinline__ void exp_only(float& t, float s) {
  asm volatile("v_exp_f32 %0, %1" : "=v"(t) : "v"(s));
}
__device__ __forceinline__ void cvt_pk(unsigned& w, float a, float b) {
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(w) : "v"(a), "v"(b));
}
__device__ __forceinline__ void max3(float& m, float a, float b, float c) {
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(a), "v"(b), "v"(c));
}
__device__ __forceinline__ void max3_acc(float& m, float b, float c) {
  asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(m) : "v"(b), "v"(c));
}
__device__ __forceinline__ void max_acc(float& m, float b) {
  asm volatile("v_max_f32 %0, %0, %1" : "+v"(m) : "v"(b));
}
// lanes where max(m0 - r0, m1 - r1) > 1: a row max outran the running max
// by more than the rescale slack (1 in log2 units)
__device__ __forceinline__ unsigned long long grow_mask(float m0, float r0, float m1, float r1) {
  unsigned long long mask;
  float t0, t1;
  asm volatile(
      "v_sub_f32 %1, %3, %4\n\t"
      "v_sub_f32 %2, %5, %6\n\t"
      "v_max_f32 %1, %1, %2\n\t"
      "v_cmp_lt_f32_e64 %0, 1.0, %1"
      : "=s"(mask), "=&v"(t0), "=&v"(t1)
      : "v"(m0), "v"(r0), "v"(m1), "v"(r1));
  return mask;
}
// m = c2 * max(m over lanes i and i ^ 32)
__device__ __forceinline__ void halves_max_scaled(float& m, float c2) {
  float t;
  asm volatile(
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "v_max_f32 %0, %0, %1\n\t"
      "v_mul_f32 %0, %2, %0"
      : "+v"(m), "=&v"(t)
      : "s"(c2));
}

// max of x over lanes i and i ^ 32 (the swap exchanges the upper half of the
// first operand with the lower half of the second)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
}  // namespace v3

// FIXED: the workgroups whose bound allows it run with a fixed maximum and
// mark the others in p.fallback; !FIXED with p.fallback set runs only those.
template <bool FIXED>
__global__ __launch_bounds__(256) void window_attn_bf16_d128_kernel(AttnParams p) {
  using namespace v3;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STAGES * 2 * TILEB];

  // wave index as a scalar: the DMA's LDS destination (M0) must be wave-uniform
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, h = lane / 32, g = lane / 16, j16 = lane % 16;

  if (!FIXED && p.fallback && !p.fallback[blockIdx.x]) return;   // done by the fixed-maximum launch
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
  const int lds0 = (int)(size_t)(__attribute__((address_space(3))) unsigned char*)ring;
  // Load i of a tile (i < BLK: K block i of this wave, else V block i - BLK);
  // the last one moves the load cursor to the next tile.  The DMA is an
  // opaque instruction: the loop waits for each tile's loads explicitly
  // (vmcnt) before the barrier that publishes the tile.  Past the last tile
  // the cursor keeps moving: those loads read other keys or zeros into the
  // stage of an already consumed tile that is never read again.
  auto issue_one = [&](int st, int i) {
    const int b = i % BLK, blk = wave * BLK + b;
    const int voff = lk0 * ROWB + lane_off[b];
    if (i < BLK)
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rk),
                   "{m0}"(lds0 + st * TILEB + blk * 1024)
                   : "memory");
    else
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rv),
                   "{m0}"(lds0 + VBASE + st * TILEB + blk * 1024)
                   : "memory");
    if (i == 2 * BLK - 1) {
      lk0 += BN;
      if (lk0 >= lke) {
        ++liv;
        if (liv < wi.nint) {
          lk0 = kb_of(liv);
          lke = ke_of(liv);
        }
      }
      lk0 = __builtin_amdgcn_readfirstlane(lk0);
      lke = __builtin_amdgcn_readfirstlane(lke);
    }
  };

  // ring of four 64-key stages: tiles t+1 .. t+3 resident or in flight while
  // tile t is consumed
#pragma unroll
  for (int st = 0; st < 3; ++st)
#pragma unroll
    for (int i = 0; i < 2 * BLK; ++i) issue_one(st, i);

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
  // Fixed softmax maximum.  With the largest key norm of this (batch, head)
  // (p.kmax), every score of query q satisfies c2 |q.k| <= c2 |q| max|k| = bnd,
  // so p = 2^(c2 s - bnd) <= 1 without a running maximum, and since the row's
  // largest score is >= -bnd its largest p is >= 2^(-2 bnd).  When bnd <=
  // kFixedMaxCap for every query of the workgroup, it takes that path;
  // otherwise it marks itself for the running-maximum launch.
  const float c2 = p.scale_log2;
  float bnd[QT] = {};
  if constexpr (FIXED) {
    float k2 = 0.f;
    for (int i = 0; i < p.kmax_parts; ++i) k2 = fmaxf(k2, p.kmax[(int64_t)wi.bh * p.kmax_parts + i]);
    const float kn = sqrtf(k2);
    float worst = 0.f;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float s2 = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) s2 += (float)qf[qt][ks][e] * (float)qf[qt][ks][e];
      // lanes l and l ^ 32 hold the two halves of the query's dims
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s2), __float_as_uint(s2), false, false);
      s2 = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      bnd[qt] = c2 * sqrtf(s2) * kn;
      worst = fmaxf(worst, bnd[qt]);
    }
    // dense items (anchor-frame and context queries over every key) keep the
    // running maximum: their rows are long, and their outputs are merged
    // over key splits
    const int lid = xcd_remap(blockIdx.x, p.total);
    const bool dense = lid - (lid / p.tiles_per_bh) * p.tiles_per_bh >= p.n_window_tiles;
    const bool unsafe = dense || __syncthreads_or(worst > kFixedMaxCap);
    if (tid == 0) p.fallback[blockIdx.x] = unsafe ? 1 : 0;
    if (unsafe) {
      // this workgroup's tiles go to the running-maximum launch; no load may
      // still write its LDS when it exits
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
      return;
    }
    // Every scaled score now lies in [-bnd, bnd] with bnd <= kFixedMaxCap, so
    // 2^(c2 s) itself stays within [2^-4, 2^4]: no maximum needs subtracting
    // (softmax is shift-invariant), and with q stored as bf16(c2 q) the score
    // products deliver c2 s directly and p is one v_exp_f32 per score.  The
    // extra rounding of c2 q moves a score by at most 2^-8 bnd <= 2^-6 (log2
    // units), i.e. p by under 1.1% relative in the worst case of aligned
    // signs; sharp rows, where that would count, never get here.
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qt][ks][e] = (bf16)((float)qf[qt][ks][e] * c2);
  }
  // Q lives in the accumulator file (the score products read it from there)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+a"(qf[qt][ks]));

  // O^T accumulators (32x32 layout) and the row sums (16x16 layout: lanes 0-15
  // hold rows 0 and 1, the sums of queries l and l + 16)
  f32x16 o[4][QT];
  f32x4 lsum[QT];
  float mrun[QT], negm[QT], mtile[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = FIXED ? 0.f : -INFINITY;
    negm[qt] = FIXED ? 0.f : INFINITY;
    lsum[qt] = f32x4{};
    asm volatile("" : "+a"(lsum[qt]));
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      o[dt][qt] = f32x16{};
      asm volatile("" : "+a"(o[dt][qt]));
    }
  }
  // row-sum selector: A operand of the 16x16x32 product; lane l holds row l%16,
  // k = 8 (l/16) .. +7; row 0 takes the k groups of queries 0-15, row 1 those of 16-31
  bf16x8 sel;
  {
    const bf16 one = (bf16)(((j16 == 0) && !(g & 1)) || ((j16 == 1) && (g & 1)) ? 1.f : 0.f);
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = one;
  }
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
    ck0 = __builtin_amdgcn_readfirstlane(ck0);
    cke = __builtin_amdgcn_readfirstlane(cke);
  };

  // Fragment addresses.  The ring keeps the K tiles of the four stages in its
  // first 64 KB and the V tiles in the second, so every read is a per-lane
  // base register plus a constant below 64 KB (stage, half tile, key step)
  // that the LDS instruction carries in its offset field.  The swizzle
  // depends on row % 16 only, and the constants move whole 16-row groups.
  int koff[8], voffA[4], voffB[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = lds0 + l32 * ROWB + swz(l32, 2 * ks + h) * 16;
  {
    const int rA = 4 * (g >> 1) + (j16 >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int dcol = dt * 32 + 16 * (g & 1) + 4 * (j16 & 3);
      const int cch = dcol >> 3, off = (dcol & 7) * 2;
      voffA[dt] = lds0 + VBASE + rA * ROWB + swz(rA, cch) * 16 + off;
      voffB[dt] = lds0 + VBASE + (rA + 8) * ROWB + swz(rA + 8, cch) * 16 + off;
    }
  }
  // offset of K fragment (stage st, half kt, step ks) relative to koff[ks];
  // of V fragment (stage st, half pt, 16-key step s4) relative to voffA/B


  // keys >= lim of a half tile get score -inf
  auto mask = [&](f32x16 (&sc)[QT], int lim) {
    const int l = lim - 4 * h;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r / 4) + (r % 4) >= l) sc[qt][r] = -INFINITY;
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
    }
  };
  // raise the running max to the tile max, rescaling O and the row sums (a
  // path the compiler schedules: it waits out the products' results first and
  // leaves wait states after)
  auto rescale = [&]() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mnew = fmaxf(mrun[qt], mtile[qt]);
      const float alpha = fast_exp2(mrun[qt] - mnew);
      mrun[qt] = mnew;
      negm[qt] = -mnew;
      // lsum rows 0 / 1 of lane l < 16 belong to queries l / l + 16
      const float a_hi = __shfl(alpha, (lane & 15) + 16);
      asm volatile("" : "+a"(lsum[qt]));
      lsum[qt][0] *= alpha;
      lsum[qt][1] *= a_hi;
      asm volatile("" : "+a"(lsum[qt]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        asm volatile("" : "+a"(o[dt][qt]));
        o[dt][qt] *= alpha;
        asm volatile("" : "+a"(o[dt][qt]));
      }
    }
    asm volatile("s_nop 4" ::: "memory");
  };
  // ... if some row max outruns it by more than the slack
  static_assert(kRescaleSlack == 1.f, "grow_mask compares against 1.0");
  auto outran = [&]() {
    bool up = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) up |= mtile[qt] > mrun[qt] + kRescaleSlack;
    return __any(up);
  };
  // between half steps: mask a partial half tile (keys >= lim) and recompute
  // its max, then raise the running max if needed; grow is the half step's
  // own verdict for a full half tile.  Neither happens on most half tiles.
  auto boundary = [&](f32x16 (&sc)[QT], int lim, unsigned long long grow) {
    bool up = grow != 0;
    if (lim < 32) {
      mask(sc, lim);
      half_max(sc);
      up = outran();
    }
    if (up) rescale();
  };

  f32x16 sa[QT], sb[QT];     // scores of the current and of the next half tile
  bf16x8 kf[4];              // K fragments of score steps ks, ks + 4 share kf[ks % 4]
  i16x4 vfa[2][4], vfb[2][4];   // V^T fragments (two halves) of the two 16-key steps
  unsigned pw[QT][2][4];     // p of the current half tile as bf16 pairs: [qt][16-key step][word]
  float tt[4];               // exponentials in flight

  // One half step (see above).  cur: scores of half tile j (stage PST, half
  // PKT); nxt: scores of half tile j+1 (stage SST, half SKT), whose K
  // fragments 0-2 were read by the previous half step; NST/NKT: the half tile
  // after that, whose K fragments 0-2 this one reads; DST >= 0: issue the
  // loads of a tile into that stage.
  auto half_step = [&](const f32x16 (&cur)[QT], f32x16 (&nxt)[QT], auto SST, auto SKT, auto PST, auto PKT,
                       auto NST, auto NKT, int dst, auto FX) __attribute__((always_inline)) {
    constexpr bool kFixed = decltype(FX)::value;
    constexpr int ks_off = koffc(decltype(SST)::value, decltype(SKT)::value);
    constexpr int kn_off = koffc(decltype(NST)::value, decltype(NKT)::value);
    constexpr int v0_off = voffc(decltype(PST)::value, decltype(PKT)::value, 0);
    constexpr int v1_off = voffc(decltype(PST)::value, decltype(PKT)::value, 1);
    auto val = [&](auto J, int e) {
      constexpr int j = decltype(J)::value, s4 = j / 8, w = (j % 8) / 2, qt = j % 2;
      if constexpr (kFixed) exp_only(tt[(2 * j + e) % 4], cur[qt][8 * s4 + 2 * w + e]);
      else fma_exp(tt[(2 * j + e) % 4], cur[qt][8 * s4 + 2 * w + e], c2, negm[qt]);
    };
    auto cvt = [&](auto J) {
      constexpr int j = decltype(J)::value, s4 = j / 8, w = (j % 8) / 2, qt = j % 2;
      cvt_pk(pw[qt][s4][w], tt[(2 * j) % 4], tt[(2 * j + 1) % 4]);
    };
    auto unit = [&](auto U) {
      constexpr int u = decltype(U)::value;
      if constexpr (u == 48) {
        cvt(IC<15>{});
      } else {
        constexpr int j = u / 3, k = u % 3;
        if constexpr (k == 0) val(IC<j>{}, 0);
        else if constexpr (k == 1) {
          if constexpr (j > 0) cvt(IC<j - 1>{});
        } else {
          val(IC<j>{}, 1);
        }
      }
    };
    auto pk = [&](int qt, int s4) {
      const u32x4 w = {pw[qt][s4][0], pw[qt][s4][1], pw[qt][s4][2], pw[qt][s4][3]};
      return __builtin_bit_cast(bf16x8, w);
    };
    auto vf = [&](int s4, int dt) {
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(vfa[s4][dt], vfb[s4][dt], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    float mx[QT];
    unsigned long long grow = 0;

    auto slot = [&](auto M) {
      constexpr int m = decltype(M)::value;
      // ---- wait for this slot's operands, then its product
      if constexpr (m < 16) {
        constexpr int ks = m / 2, qt = m % 2;
        if constexpr (qt == 0) wait_lgkm<wait_s(ks)>();
        if constexpr (ks == 0) mma_s0(nxt[qt], kf[ks % 4], qf[qt][ks]);
        else mma_s(nxt[qt], kf[ks % 4], qf[qt][ks]);
      } else if constexpr (m < 24) {
        constexpr int dt = (m - 16) / 2, qt = m % 2;
        if constexpr (qt == 0) wait_lgkm<wait_p(0, dt)>();
        mma_o(o[dt][qt], vf(0, dt), pk(qt, 0));
      } else if constexpr (m < 26) {
        mma_l(lsum[m - 24], sel, pk(m - 24, 0));
      } else if constexpr (m < 34) {
        constexpr int dt = (m - 26) / 2, qt = m % 2;
        if constexpr (qt == 0) wait_lgkm<wait_p(1, dt)>();
        mma_o(o[dt][qt], vf(1, dt), pk(qt, 1));
      } else {
        mma_l(lsum[m - 34], sel, pk(m - 34, 1));
      }
      // ---- LDS fragment reads issued in this slot: K, then V
      static_for<0, 8>([&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        if constexpr (kIssueK[ks] == m) ds_k<ks_off>(kf[ks % 4], koff[ks]);
        if constexpr (kIssueK[ks] + 36 == m) ds_k<kn_off>(kf[ks % 4], koff[ks]);
      });
      static_for<0, 16>([&](auto I) {
        constexpr int i = decltype(I)::value, s4 = i / 8, dt = (i % 8) / 2, ab = i % 2;
        constexpr int off = s4 == 0 ? v0_off : v1_off;
        if constexpr (kIssueV[i] == m) {
          if constexpr (ab == 0) ds_tr<off>(vfa[s4][dt], voffA[dt]);
          else ds_tr<off>(vfb[s4][dt], voffB[dt]);
        }
      });
      // ---- DMA of a later tile
      static_for<0, 2 * BLK>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (kIssueD[i] == m) {
          if (dst >= 0) issue_one(dst, i);
        }
      });
      // ---- vector work
      if constexpr (m <= 20) static_for<units_before(m), units_before(m + 1)>(unit);
      // max of the next scores: the score chains end in slots 14 / 15
      if constexpr (kFixed) {
      } else if constexpr (m == 21) {
        max3(mx[0], nxt[0][0], nxt[0][1], nxt[0][2]);
        max3(mx[1], nxt[1][0], nxt[1][1], nxt[1][2]);
      }
      if constexpr (!kFixed && m >= 22 && m <= 28) {
        constexpr int r = 3 + 2 * (m - 22);   // 3, 5, .., 15
        if constexpr (r < 15) {
          max3_acc(mx[0], nxt[0][r], nxt[0][r + 1]);
          max3_acc(mx[1], nxt[1][r], nxt[1][r + 1]);
        } else {
          max_acc(mx[0], nxt[0][15]);
          max_acc(mx[1], nxt[1][15]);
        }
      }
      if constexpr (!kFixed && m == 29) halves_max_scaled(mx[0], c2);
      if constexpr (!kFixed && m == 30) halves_max_scaled(mx[1], c2);
      if constexpr (!kFixed && m == 32) grow = grow_mask(mx[0], mrun[0], mx[1], mrun[1]);
    };
    static_for<0, 36>(slot);
    if constexpr (!kFixed) {
      mtile[0] = mx[0];
      mtile[1] = mx[1];
    }
    return grow;
  };
  // between half steps on the fixed-maximum path: only a partial half tile's
  // masking (keys >= lim)
  auto boundary_fixed = [&](f32x16 (&sc)[QT], int lim) {
    if (lim < 32) mask(sc, lim);
  };

  // Q and the first three tiles resident
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();

  int kn = min(BN, cke - ck0);   // keys of tile t
  // first half tile's scores (stage 0, half 0), then K fragments 0-2 of the
  // first half step (stage 0, half 1)
  asm volatile("s_nop 4" ::: "memory");   // Q was just written to the accumulator file
  static_for<0, 8>([&](auto KS) {
    constexpr int ks = decltype(KS)::value;
    ds_k<koffc(0, 0)>(kf[ks % 4], koff[ks]);
    wait_lgkm<0>();
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      if constexpr (ks == 0) mma_s0(sa[qt], kf[0], qf[qt][0]);
      else mma_s(sa[qt], kf[ks % 4], qf[qt][ks]);
    }
  });
  // the vector unit reads the scores next: wait for the last products
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  if constexpr (FIXED) {
    boundary_fixed(sa, kn);
  } else {
    half_max(sa);
    boundary(sa, kn, outran() ? 1ull : 0ull);
  }
  ds_k<koffc(0, 1)>(kf[0], koff[0]);
  ds_k<koffc(0, 1)>(kf[1], koff[1]);
  ds_k<koffc(0, 1)>(kf[2], koff[2]);

  // One tile: its two halves; the second computes the scores of the first
  // half of tile t+1 (for the last tile they come from a stale stage and are
  // never used).  Tile t sits in ring stage t % 4; the loop is unrolled over
  // the four stages so that every stage offset is a constant.
  auto tile = [&](int t, auto S0, auto S1, int s3, auto FX) __attribute__((always_inline)) {
    const unsigned long long g1 = half_step(sa, sb, S0, IC<1>{}, S0, IC<0>{}, S1, IC<0>{}, s3, FX);
    if constexpr (decltype(FX)::value) boundary_fixed(sb, kn - 32);
    else boundary(sb, kn - 32, g1);
    const unsigned long long g2 = half_step(sb, sa, S1, IC<0>{}, S0, IC<1>{}, S1, IC<1>{}, -1, FX);
    advance();
    kn = min(BN, cke - ck0);
    // tile t+2's loads (issued one tile ago) are complete once at most the 8
    // of tile t+3 are outstanding; the barrier publishes tile t+2 and frees
    // the stage of tile t for the next tile's loads
    __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8)
    __builtin_amdgcn_s_barrier();
    if (t + 1 < ntiles) {
      if constexpr (decltype(FX)::value) boundary_fixed(sa, kn);
      else boundary(sa, kn, g2);
    }
  };
  auto run = [&](auto FX) __attribute__((always_inline)) {
    for (int t = 0; t < ntiles; t += 4) {
      tile(t, IC<0>{}, IC<1>{}, 3, FX);
      if (t + 1 >= ntiles) break;
      tile(t + 1, IC<1>{}, IC<2>{}, 0, FX);
      if (t + 2 >= ntiles) break;
      tile(t + 2, IC<2>{}, IC<3>{}, 1, FX);
      if (t + 3 >= ntiles) break;
      tile(t + 3, IC<3>{}, IC<0>{}, 2, FX);
    }
  };
  run(IC<FIXED>{});
  // no load may still write this workgroup's LDS when it exits; the last
  // products' results are read next
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // ---- epilogue: o[dt][qt][r] = O(query 32 qt + l32, dim 32 dt + 8(r/4) + 4h + r%4)
  const bf16* gate = (const bf16*)p.gate;
  bf16* out = (bf16*)p.out;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    // row sum of query l32: row 0 of lane l32 (l32 < 16) or row 1 of lane l32 - 16
    const float r0 = __shfl(lsum[qt][0], l32 & 15), r1 = __shfl(lsum[qt][1], l32 & 15);
    const float lt = l32 < 16 ? r0 : r1;
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

// ---------------------------------------------------------------------------
// Softmax branch with MXFP8 scores: head_dim 128, Q and K as MXFP8 (OCP E4M3
// codes, one E8M0 scale per 32 elements of a row; [P3] 实验结果 runs the
// denoiser in MXFP8), V, gate and output bf16.  The same work items, key
// intervals, running-max softmax, P V and row-sum products and epilogue as
// the bf16 kernel above; only the score product changes.
//
// S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4: 64 dims per product, so a
// 32x32 score tile is 2 products of 64 cycles instead of 8 of 32.  The
// product's K layout (probed): lane l of row i holds the 32 codes of dims
// 16 (l / 32) .. +15 and 32 + 16 (l / 32) .. +15 of its 64-dim half, and the
// scale of 32-dim block b of row i comes from lane i + 32 b.  So a lane reads
// two 16-byte chunks of its row (K from LDS, Q from global once) and one
// scale byte; the block order inside a half is the order of the dims.
//
// A half step is a fixed list of 24 slots, one product each: 4 score
// products of half tile j+1 (slots 0-3), 8 P V products and 2 row sums for
// each 16-key step of half tile j (slots 4-13 and 14-23).  The 32
// exponentials and 16 conversions of half tile j run beside the score and
// the first P V products (queries 0-31 of each step first, so the first P V
// product's words are ready early); the max of half tile j+1 beside the
// second P V step.  LDS reads: V of step 1 of half tile j in slots 0-7, the
// K codes and scales of half tile j+2 in slots 8-13, V of step 0 of half
// tile j+1 in slots 14-21; each product waits with an lgkmcnt computed from
// these tables at compile time.
namespace v8 {
using namespace v3;
constexpr int KROWB8 = D;                        // code bytes per K row
constexpr int KTILEB8 = BN * KROWB8;             // 8 KB
constexpr int VBASE8 = STAGES * KTILEB8;         // V tiles (bf16) after the K tiles
constexpr int SBASE8 = VBASE8 + STAGES * TILEB;  // then the K scales
constexpr int STILEB8 = BN * 4;                  // 4 scale bytes per key
constexpr int LDSB8 = SBASE8 + STAGES * STILEB8;
constexpr int KBLK8 = 2;                         // 1 KB K blocks per wave and tile
constexpr int NLOAD8 = KBLK8 + BLK + 1;          // K, V and one scale load per wave and tile
constexpr int NSLOT8 = 24;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// 128-byte K rows cover 32 banks: chunk c of row r at c ^ ((r >> 1) & 7), so
// a 16-lane read of one chunk in 16 consecutive rows covers all 64 banks
__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r >> 1) & 7); }
// constant parts of the K code / scale read addresses: stage st, half tile kt
constexpr int kcoff8(int st, int kt) { return st * KTILEB8 + kt * 32 * KROWB8; }
constexpr int ksoff8(int st, int kt) { return st * STILEB8 + kt * 32 * 4; }

// issue slots: K reads r = 3 kh + {codes 0-15, codes 16-31, scale} of the
// half step after this one; V half-fragments i = 2 dt + ab of 16-key step s4
constexpr int kIssueK8[6] = {8, 9, 10, 11, 12, 13};
constexpr int kIssueV8[2][8] = {{14, 15, 16, 17, 18, 19, 20, 21}, {0, 1, 2, 3, 4, 5, 6, 7}};
constexpr int kIssueD8[NLOAD8] = {4, 5, 6, 7, 8, 9, 10};
constexpr int key8_k(int r) { return kIssueK8[r] * 64 + r; }
constexpr int key8_v(int s4, int i) { return kIssueV8[s4][i] * 64 + 8 + 8 * s4 + i; }
// reads issued after the one with key a (keys of the half step before are
// shifted by one half step) and before the wait of slot m
constexpr int younger8(int a, int m) {
  int n = 0;
  for (int sh = -1; sh <= 0; ++sh) {
    for (int r = 0; r < 6; ++r) {
      const int k = key8_k(r) + sh * NSLOT8 * 64;
      if (k > a && k < 64 * m) ++n;
    }
    for (int s4 = 0; s4 < 2; ++s4)
      for (int i = 0; i < 8; ++i) {
        const int k = key8_v(s4, i) + sh * NSLOT8 * 64;
        if (k > a && k < 64 * m) ++n;
      }
  }
  return n < 15 ? n : 15;
}
// score products of dims half kh (slot 2 kh): K reads of the half step before
constexpr int wait8_s(int kh) { return younger8(key8_k(3 * kh + 2) - NSLOT8 * 64, 2 * kh); }
// P V of step 0 (slot 4 + 2 dt): V reads of the half step before; of step 1
// (slot 14 + 2 dt): this half step's
constexpr int wait8_p0(int dt) { return younger8(key8_v(0, 2 * dt + 1) - NSLOT8 * 64, 4 + 2 * dt); }
constexpr int wait8_p1(int dt) { return younger8(key8_v(1, 2 * dt + 1), 14 + 2 * dt); }
constexpr bool schedule8_ok() {
  for (int r = 0; r < 6; ++r)
    if (kIssueK8[r] < 4) return false;                      // after this half step's score products
  for (int i = 0; i < 8; ++i) {
    if (kIssueV8[0][i] < 12) return false;                  // after this half step's step-0 P V products
    if (kIssueV8[1][i] >= 14 + 2 * (i / 2)) return false;   // before its own product
  }
  return true;
}
static_assert(schedule8_ok(), "MXFP8 LDS read schedule violates its order constraints");
static_assert(wait8_s(0) == 11 && wait8_p1(0) == 12, "lgkmcnt tables");

// exponential pairs in order of use: queries 0-31 (qt 0) of each 16-key step first
constexpr int kPair8[16] = {0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15};
// 26 units (pairs 0-7 of the order and the conversion of the eighth) beside
// the 4 score products, the other 23 beside slots 4-13
constexpr int units_before8(int m) {
  return m <= 4 ? (26 * m + 2) / 4 : (m <= 14 ? 26 + (23 * (m - 4) + 5) / 10 : 49);
}

template <int SEL>   // Q scale byte (2 qt + kh)
__device__ __forceinline__ void mma8_0(f32x16& d, i32x8 k, i32x8 q, int ks, int qs) {
  asm volatile(
      "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel:[0,%5,0] op_sel_hi:[0,%6,0]"
      : "=&v"(d)
      : "v"(k), "a"(q), "v"(ks), "v"(qs), "n"(SEL & 1), "n"(SEL >> 1));
}
template <int SEL>
__device__ __forceinline__ void mma8(f32x16& d, i32x8 k, i32x8 q, int ks, int qs) {
  asm volatile(
      "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[0,%5,0] op_sel_hi:[0,%6,0]"
      : "+v"(d)
      : "v"(k), "a"(q), "v"(ks), "v"(qs), "n"(SEL & 1), "n"(SEL >> 1));
}
template <int OFF>
__device__ __forceinline__ void ds_c(i32x4& d, int addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_s(int& d, int addr) {
  asm volatile("ds_read_u8 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
}
}  // namespace v8

// Scores are the products of the decoded q and k; each is scaled into log2
// units on its way into v_exp_f32 (one v_fma_f32 with the running maximum).
__global__ __launch_bounds__(256) void window_attn_mxfp8_d128_kernel(AttnParams p) {
  using namespace v8;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[LDSB8];

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, h = lane / 32, g = lane / 16, j16 = lane % 16;

  const WorkItem wi = decode_work(p, BM);
  const int NL = p.Lt;
  const unsigned char* Qc = (const unsigned char*)p.q + (int64_t)wi.bh * NL * D;
  const unsigned char* Qs = (const unsigned char*)p.qs + (int64_t)wi.bh * NL * 4;
  const unsigned char* Kc = (const unsigned char*)p.k + (int64_t)wi.bh * NL * D;
  const unsigned char* Ks = (const unsigned char*)p.ks + (int64_t)wi.bh * NL * 4;
  const bf16* Vb = (const bf16*)p.v + (int64_t)wi.bh * NL * D;

  int ntiles = 0;
#pragma unroll
  for (int iv = 0; iv < 4; ++iv)
    if (iv < wi.nint) ntiles += (wi.ke[iv] - wi.kb[iv] + BN - 1) / BN;

  // Loader: per tile and wave 2 K blocks (8 rows of 128 code bytes; lane l
  // fills physical chunk l % 8 of row l / 8), 4 V blocks (as the bf16
  // kernel) and one 256-byte load of the tile's 64 x 4 scale bytes (every
  // wave loads the same bytes, so each wave issues the same loads).
  int koff_lane[KBLK8], voff_lane[BLK];
#pragma unroll
  for (int i = 0; i < KBLK8; ++i) {
    const int row = (wave * KBLK8 + i) * 8 + lane / 8;
    koff_lane[i] = row * KROWB8 + swz8(row, lane % 8) * 16;
  }
#pragma unroll
  for (int i = 0; i < BLK; ++i) {
    const int row = (wave * BLK + i) * 4 + lane / 16;
    voff_lane[i] = row * ROWB + swz(row, lane % 16) * 16;
  }
  const int kb0 = wi.kb[0], kb1 = wi.kb[1], kb2 = wi.kb[2], kb3 = wi.kb[3];
  const int ke0 = wi.ke[0], ke1 = wi.ke[1], ke2 = wi.ke[2], ke3 = wi.ke[3];
  auto kb_of = [&](int i) { return i == 0 ? kb0 : (i == 1 ? kb1 : (i == 2 ? kb2 : kb3)); };
  auto ke_of = [&](int i) { return i == 0 ? ke0 : (i == 1 ? ke1 : (i == 2 ? ke2 : ke3)); };
  int liv = 0, lk0 = kb_of(0), lke = ke_of(0);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)Kc, (short)0, NL * KROWB8, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)Ks, (short)0, NL * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)Vb, (short)0, NL * ROWB, 0x00020000);
  const int lds0 = (int)(size_t)(__attribute__((address_space(3))) unsigned char*)ring;
  auto issue8 = [&](int st, int i) {
    if (i < KBLK8) {
      const int voff = lk0 * KROWB8 + koff_lane[i];
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rk),
                   "{m0}"(lds0 + st * KTILEB8 + (wave * KBLK8 + i) * 1024)
                   : "memory");
    } else if (i < KBLK8 + BLK) {
      const int b = i - KBLK8;
      const int voff = lk0 * ROWB + voff_lane[b];
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rv),
                   "{m0}"(lds0 + VBASE8 + st * TILEB + (wave * BLK + b) * 1024)
                   : "memory");
    } else {
      const int voff = (lk0 + lane) * 4;
      asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
                   "{m0}"(lds0 + SBASE8 + st * STILEB8)
                   : "memory");
      lk0 += BN;
      if (lk0 >= lke) {
        ++liv;
        if (liv < wi.nint) {
          lk0 = kb_of(liv);
          lke = ke_of(liv);
        }
      }
      lk0 = __builtin_amdgcn_readfirstlane(lk0);
      lke = __builtin_amdgcn_readfirstlane(lke);
    }
  };
#pragma unroll
  for (int st = 0; st < 3; ++st)
#pragma unroll
    for (int i = 0; i < NLOAD8; ++i) issue8(st, i);

  // Q codes (B operand, in the accumulator file) and scales: lane holds
  // query l32's codes of dims 64 kh + 16 h .. +15 and 64 kh + 32 + 16 h .. +15;
  // byte 2 qt + kh of qsc is the scale of its block 2 kh + h
  i32x8 qf8[QT][2];
  int qsc = 0;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qrow = wi.qbeg + wave * WQ + qt * 32 + l32;
    const bool ok = qrow < wi.qend;
    const unsigned sw = ok ? *reinterpret_cast<const unsigned*>(Qs + (int64_t)qrow * 4) : 0u;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const unsigned char* src = Qc + (int64_t)qrow * D + 64 * kh + 16 * h;
      const i32x4 lo = ok ? *reinterpret_cast<const i32x4*>(src) : i32x4{};
      const i32x4 hi = ok ? *reinterpret_cast<const i32x4*>(src + 32) : i32x4{};
      qf8[qt][kh] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      qsc |= (int)(((sw >> (8 * (2 * kh + h))) & 0xFFu) << (8 * (2 * qt + kh)));
    }
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) asm volatile("" : "+a"(qf8[qt][kh]));

  f32x16 o[4][QT];
  f32x4 lsum[QT];
  float mrun[QT], negm[QT], mtile[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = -INFINITY;
    negm[qt] = INFINITY;
    lsum[qt] = f32x4{};
    asm volatile("" : "+a"(lsum[qt]));
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      o[dt][qt] = f32x16{};
      asm volatile("" : "+a"(o[dt][qt]));
    }
  }
  bf16x8 sel;
  {
    const bf16 one = (bf16)(((j16 == 0) && !(g & 1)) || ((j16 == 1) && (g & 1)) ? 1.f : 0.f);
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = one;
  }
  const float c2 = p.scale_log2;
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
    ck0 = __builtin_amdgcn_readfirstlane(ck0);
    cke = __builtin_amdgcn_readfirstlane(cke);
  };

  // Fragment addresses: K codes and scales of row l32 of a half tile (chunks
  // 4 kh + 2 part + h), V as the bf16 kernel
  int kcoff[2][2], ksoff[2], voffA[4], voffB[4];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) kcoff[kh][pt] = lds0 + l32 * KROWB8 + swz8(l32, 4 * kh + 2 * pt + h) * 16;
    ksoff[kh] = lds0 + SBASE8 + l32 * 4 + 2 * kh + h;
  }
  {
    const int rA = 4 * (g >> 1) + (j16 >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int dcol = dt * 32 + 16 * (g & 1) + 4 * (j16 & 3);
      const int cch = dcol >> 3, off = (dcol & 7) * 2;
      voffA[dt] = lds0 + VBASE8 + rA * ROWB + swz(rA, cch) * 16 + off;
      voffB[dt] = lds0 + VBASE8 + (rA + 8) * ROWB + swz(rA + 8, cch) * 16 + off;
    }
  }

  auto mask = [&](f32x16 (&sc)[QT], int lim) {
    const int l = lim - 4 * h;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r / 4) + (r % 4) >= l) sc[qt][r] = -INFINITY;
  };
  auto half_max = [&](const f32x16 (&sc)[QT]) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = sc[qt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[qt][r]);
      mtile[qt] = halves_max(mx) * c2;
    }
  };
  auto rescale = [&](f32x16 (&sc)[QT]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mnew = fmaxf(mrun[qt], mtile[qt]);
      const float alpha = fast_exp2(mrun[qt] - mnew);
      mrun[qt] = mnew;
      negm[qt] = -mnew;
      const float a_hi = __shfl(alpha, (lane & 15) + 16);
      asm volatile("" : "+a"(lsum[qt]));
      lsum[qt][0] *= alpha;
      lsum[qt][1] *= a_hi;
      asm volatile("" : "+a"(lsum[qt]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        asm volatile("" : "+a"(o[dt][qt]));
        o[dt][qt] *= alpha;
        asm volatile("" : "+a"(o[dt][qt]));
      }
    }
    asm volatile("s_nop 4" ::: "memory");
  };
  static_assert(kRescaleSlack == 1.f, "grow_mask compares against 1.0");
  auto outran = [&]() {
    bool up = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) up |= mtile[qt] > mrun[qt] + kRescaleSlack;
    return __any(up);
  };
  auto boundary = [&](f32x16 (&sc)[QT], int lim, unsigned long long grow) {
    bool up = grow != 0;
    if (lim < 32) {
      mask(sc, lim);
      half_max(sc);
      up = outran();
    }
    if (up) rescale(sc);
  };

  f32x16 sa[QT], sb[QT];
  i32x4 klo[2], khi[2];   // K codes of the next score products: [dims half][chunk pair part]
  int ksc[2];             // their scales (byte 0)
  i16x4 vfa[2][4], vfb[2][4];
  unsigned pw[QT][2][4];
  float tt[4];
  auto kfrag = [&](int kh) { return __builtin_shufflevector(klo[kh], khi[kh], 0, 1, 2, 3, 4, 5, 6, 7); };

  auto half_step = [&](const f32x16 (&cur)[QT], f32x16 (&nxt)[QT], auto SST, auto SKT, auto PST, auto PKT,
                       auto NST, auto NKT, int dst) __attribute__((always_inline)) {
    constexpr int kc_off = kcoff8(decltype(NST)::value, decltype(NKT)::value);
    constexpr int ks_off = ksoff8(decltype(NST)::value, decltype(NKT)::value);
    constexpr int v0_off = voffc(decltype(SST)::value, decltype(SKT)::value, 0);
    constexpr int v1_off = voffc(decltype(PST)::value, decltype(PKT)::value, 1);
    auto val = [&](auto I, int e) {
      constexpr int i = decltype(I)::value, j = kPair8[i], s4 = j / 8, w = (j % 8) / 2, qt = j % 2;
      fma_exp(tt[(2 * i + e) % 4], cur[qt][8 * s4 + 2 * w + e], c2, negm[qt]);
    };
    auto cvt = [&](auto I) {
      constexpr int i = decltype(I)::value, j = kPair8[i], s4 = j / 8, w = (j % 8) / 2, qt = j % 2;
      cvt_pk(pw[qt][s4][w], tt[(2 * i) % 4], tt[(2 * i + 1) % 4]);
    };
    auto unit = [&](auto U) {
      constexpr int u = decltype(U)::value;
      if constexpr (u == 48) {
        cvt(IC<15>{});
      } else {
        constexpr int i = u / 3, k = u % 3;
        if constexpr (k == 0) val(IC<i>{}, 0);
        else if constexpr (k == 1) {
          if constexpr (i > 0) cvt(IC<i - 1>{});
        } else {
          val(IC<i>{}, 1);
        }
      }
    };
    auto pk = [&](int qt, int s4) {
      const u32x4 w = {pw[qt][s4][0], pw[qt][s4][1], pw[qt][s4][2], pw[qt][s4][3]};
      return __builtin_bit_cast(bf16x8, w);
    };
    auto vf = [&](int s4, int dt) {
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(vfa[s4][dt], vfb[s4][dt], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    float mx[QT];
    unsigned long long grow = 0;

    auto slot = [&](auto M) {
      constexpr int m = decltype(M)::value;
      if constexpr (m < 4) {
        constexpr int kh = m / 2, qt = m % 2;
        if constexpr (qt == 0) wait_lgkm<wait8_s(kh)>();
        if constexpr (kh == 0) mma8_0<2 * qt>(nxt[qt], kfrag(0), qf8[qt][0], ksc[0], qsc);
        else mma8<2 * qt + 1>(nxt[qt], kfrag(1), qf8[qt][1], ksc[1], qsc);
      } else if constexpr (m < 12) {
        constexpr int dt = (m - 4) / 2, qt = m % 2;
        if constexpr (qt == 0) wait_lgkm<wait8_p0(dt)>();
        mma_o(o[dt][qt], vf(0, dt), pk(qt, 0));
      } else if constexpr (m < 14) {
        mma_l(lsum[m - 12], sel, pk(m - 12, 0));
      } else if constexpr (m < 22) {
        constexpr int dt = (m - 14) / 2, qt = m % 2;
        if constexpr (qt == 0) wait_lgkm<wait8_p1(dt)>();
        mma_o(o[dt][qt], vf(1, dt), pk(qt, 1));
      } else {
        mma_l(lsum[m - 22], sel, pk(m - 22, 1));
      }
      // LDS reads of this slot: K, then V
      static_for<0, 6>([&](auto R) {
        constexpr int r = decltype(R)::value, kh = r / 3, part = r % 3;
        if constexpr (kIssueK8[r] == m) {
          if constexpr (part == 0) ds_c<kc_off>(klo[kh], kcoff[kh][0]);
          else if constexpr (part == 1) ds_c<kc_off>(khi[kh], kcoff[kh][1]);
          else ds_s<ks_off>(ksc[kh], ksoff[kh]);
        }
      });
      static_for<0, 16>([&](auto I) {
        constexpr int s4 = decltype(I)::value / 8, i = decltype(I)::value % 8, dt = i / 2, ab = i % 2;
        constexpr int off = s4 == 0 ? v0_off : v1_off;
        if constexpr (kIssueV8[s4][i] == m) {
          if constexpr (ab == 0) ds_tr<off>(vfa[s4][dt], voffA[dt]);
          else ds_tr<off>(vfb[s4][dt], voffB[dt]);
        }
      });
      static_for<0, NLOAD8>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (kIssueD8[i] == m) {
          if (dst >= 0) issue8(dst, i);
        }
      });
      if constexpr (m <= 13) static_for<units_before8(m), units_before8(m + 1)>(unit);
      // max of the next scores (their products ended by slot 5)
      if constexpr (m == 12) {
        max3(mx[0], nxt[0][0], nxt[0][1], nxt[0][2]);
        max3(mx[1], nxt[1][0], nxt[1][1], nxt[1][2]);
      }
      if constexpr (m >= 13 && m <= 19) {
        constexpr int r = 3 + 2 * (m - 13);
        if constexpr (r < 15) {
          max3_acc(mx[0], nxt[0][r], nxt[0][r + 1]);
          max3_acc(mx[1], nxt[1][r], nxt[1][r + 1]);
        } else {
          max_acc(mx[0], nxt[0][15]);
          max_acc(mx[1], nxt[1][15]);
        }
      }
      if constexpr (m == 20) halves_max_scaled(mx[0], c2);
      if constexpr (m == 21) halves_max_scaled(mx[1], c2);
      if constexpr (m == 22) grow = grow_mask(mx[0], mrun[0], mx[1], mrun[1]);
    };
    static_for<0, NSLOT8>(slot);
    mtile[0] = mx[0];
    mtile[1] = mx[1];
    return grow;
  };

  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();

  int kn = min(BN, cke - ck0);
  // first half tile's scores (stage 0, half 0)
  asm volatile("s_nop 4" ::: "memory");
  ds_c<kcoff8(0, 0)>(klo[0], kcoff[0][0]);
  ds_c<kcoff8(0, 0)>(khi[0], kcoff[0][1]);
  ds_s<ksoff8(0, 0)>(ksc[0], ksoff[0]);
  ds_c<kcoff8(0, 0)>(klo[1], kcoff[1][0]);
  ds_c<kcoff8(0, 0)>(khi[1], kcoff[1][1]);
  ds_s<ksoff8(0, 0)>(ksc[1], ksoff[1]);
  wait_lgkm<0>();
  mma8_0<0>(sa[0], kfrag(0), qf8[0][0], ksc[0], qsc);
  mma8_0<2>(sa[1], kfrag(0), qf8[1][0], ksc[0], qsc);
  mma8<1>(sa[0], kfrag(1), qf8[0][1], ksc[1], qsc);
  mma8<3>(sa[1], kfrag(1), qf8[1][1], ksc[1], qsc);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  half_max(sa);
  boundary(sa, kn, outran() ? 1ull : 0ull);
  // the reads the first half step expects from a half step before it: K of
  // half tile (stage 0, half 1), then V step 0 of half tile (stage 0, half 0)
  ds_c<kcoff8(0, 1)>(klo[0], kcoff[0][0]);
  ds_c<kcoff8(0, 1)>(khi[0], kcoff[0][1]);
  ds_s<ksoff8(0, 1)>(ksc[0], ksoff[0]);
  ds_c<kcoff8(0, 1)>(klo[1], kcoff[1][0]);
  ds_c<kcoff8(0, 1)>(khi[1], kcoff[1][1]);
  ds_s<ksoff8(0, 1)>(ksc[1], ksoff[1]);
  static_for<0, 8>([&](auto I) {
    constexpr int i = decltype(I)::value, dt = i / 2;
    if constexpr (i % 2 == 0) ds_tr<voffc(0, 0, 0)>(vfa[0][dt], voffA[dt]);
    else ds_tr<voffc(0, 0, 0)>(vfb[0][dt], voffB[dt]);
  });

  auto tile = [&](int t, auto S0, auto S1, int s3) __attribute__((always_inline)) {
    const unsigned long long g1 = half_step(sa, sb, S0, IC<1>{}, S0, IC<0>{}, S1, IC<0>{}, s3);
    boundary(sb, kn - 32, g1);
    const unsigned long long g2 = half_step(sb, sa, S1, IC<0>{}, S0, IC<1>{}, S1, IC<1>{}, -1);
    advance();
    kn = min(BN, cke - ck0);
    // tile t+2's loads are complete once at most the 7 of tile t+3 are outstanding
    __builtin_amdgcn_s_waitcnt(0x0F77);   // vmcnt(7)
    __builtin_amdgcn_s_barrier();
    if (t + 1 < ntiles) boundary(sa, kn, g2);
  };
  for (int t = 0; t < ntiles; t += 4) {
    tile(t, IC<0>{}, IC<1>{}, 3);
    if (t + 1 >= ntiles) break;
    tile(t + 1, IC<1>{}, IC<2>{}, 0);
    if (t + 2 >= ntiles) break;
    tile(t + 2, IC<2>{}, IC<3>{}, 1);
    if (t + 3 >= ntiles) break;
    tile(t + 3, IC<3>{}, IC<0>{}, 2);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  const bf16* gate = (const bf16*)p.gate;
  bf16* out = (bf16*)p.out;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float r0 = __shfl(lsum[qt][0], l32 & 15), r1 = __shfl(lsum[qt][1], l32 & 15);
    const float lt = l32 < 16 ? r0 : r1;
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
// D / 8 threads per dense row, 8 consecutive dimensions each: every partial-output
// read is two 16-byte loads and every gate read and output write one 16-byte access
// (gate and output strides and head offsets are multiples of 8 elements).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;   // threads per row, rows per workgroup
  const int nqb = (p.dense_rows + RPB - 1) / RPB;
  const int qb = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb;             // b*H + h
  const int h = bh % p.H, b = bh / p.H;
  const int n = qb * RPB + threadIdx.x / TPR;  // index among the dense rows
  if (n >= p.dense_rows) return;
  // the group holding dense row n (groups are stored in row order)
  const int g = (p.nG > 2 && n >= p.grp_part[2]) ? 2 : ((p.nG > 1 && n >= p.grp_part[1]) ? 1 : 0);
  const int qrow = (g == 0 ? p.grp_row0[0] : (g == 1 ? p.grp_row0[1] : p.grp_row0[2])) + n -
                   (g == 0 ? p.grp_part[0] : (g == 1 ? p.grp_part[1] : p.grp_part[2]));
  const int d0 = (threadIdx.x % TPR) * 8;
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s)
    M = fmaxf(M, p.part_ml[(((int64_t)bh * p.nsplit + s) * p.dense_rows + n) * 2]);
  float L = 0.f;
  float acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const int64_t prow = ((int64_t)bh * p.nsplit + s) * p.dense_rows + n;
    const float wgt = fast_exp2(p.part_ml[prow * 2] - M);
    L += wgt * p.part_ml[prow * 2 + 1];
    const float4 o0 = *reinterpret_cast<const float4*>(p.part_o + prow * D + d0);
    const float4 o1 = *reinterpret_cast<const float4*>(p.part_o + prow * D + d0 + 4);
    acc[0] += wgt * o0.x; acc[1] += wgt * o0.y; acc[2] += wgt * o0.z; acc[3] += wgt * o0.w;
    acc[4] += wgt * o1.x; acc[5] += wgt * o1.y; acc[6] += wgt * o1.z; acc[7] += wgt * o1.w;
  }
  const float inv = 1.f / L;
  const int64_t orow = (int64_t)b * p.Lt + qrow;
  const T* gate = (const T*)p.gate;
  T* out = (T*)p.out;
  float val[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) val[x] = acc[x] * inv;
  if (gate) {
    const T* gp = gate + orow * p.ldg + h * D + d0;
    if constexpr (sizeof(T) == 2) {
      const Chunk16 gv = *reinterpret_cast<const Chunk16*>(gp);
      const T* ge = reinterpret_cast<const T*>(&gv);
#pragma unroll
      for (int x = 0; x < 8; ++x) val[x] *= to_f32(ge[x]);
    } else {
#pragma unroll
      for (int x = 0; x < 8; ++x) val[x] *= to_f32(gp[x]);
    }
  }
  T* op = out + orow * p.ldo + h * D + d0;
  if constexpr (sizeof(T) == 2) {
    Chunk16 ov;
    T* oe = reinterpret_cast<T*>(&ov);
#pragma unroll
    for (int x = 0; x < 8; ++x) oe[x] = from_f32<T>(val[x]);
    *reinterpret_cast<Chunk16*>(op) = ov;
  } else {
#pragma unroll
    for (int x = 0; x < 8; x += 4) *reinterpret_cast<float4*>(op + x) = make_float4(val[x], val[x + 1], val[x + 2], val[x + 3]);
  }
  if (p.lse && d0 == 0) p.lse[(int64_t)bh * p.Lt + qrow] = (M + log2f(L)) * kLn2;
}

template <typename T, int D>
static hipError_t launch_attn_t(const AttnParams& p, hipStream_t st) {
  if (p.total > 0) {
    if (attn_uses_v2(sizeof(T) == 2 ? 1 : 0, D)) {
      if (p.kmax && p.fallback) {
        // fixed maximum where the key-norm bound allows it, then the running
        // maximum for the workgroups it marked (the others return at once)
        window_attn_bf16_d128_kernel<true><<<p.total, 256, 0, st>>>(p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        window_attn_bf16_d128_kernel<false><<<p.total, 256, 0, st>>>(p);
      } else {
        AttnParams q = p;
        q.fallback = nullptr;
        window_attn_bf16_d128_kernel<false><<<p.total, 256, 0, st>>>(q);
      }
    } else
      window_attn_kernel<T, D><<<p.total, 256, 0, st>>>(p);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_merge_t(const AttnParams& p, hipStream_t st) {
  if (p.nsplit > 1 && p.nG > 0) {
    constexpr int RPB = 256 / (D / 8);   // dense rows per workgroup
    const int blocks = p.B * p.H * ((p.dense_rows + RPB - 1) / RPB);
    attn_merge_kernel<T, D><<<blocks, 256, 0, st>>>(p);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// key_norm_max: the largest squared L2 norm of the key rows (bf16, head_dim
// 128) of one part of one (batch, head), the bound behind the softmax
// kernel's fixed maximum.  Four threads per 256-byte row, each summing four
// 16-byte chunks (one 64-byte line), 64 rows per pass of the workgroup.
__global__ __launch_bounds__(256) void key_norm_max_kernel(const bf16* __restrict__ k, float* __restrict__ out,
                                                           int Lt, int parts) {
  const int64_t bh = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  const int rpp = (Lt + parts - 1) / parts;
  const int r0 = part * rpp, r1 = min(Lt, r0 + rpp);
  const int tid = threadIdx.x, quarter = tid % 4;
  const bf16* kb = k + bh * (int64_t)Lt * 128 + 32 * quarter;
  float best = 0.f;
  for (int r = r0 + tid / 4; r < r1; r += 64) {
    const bf16* row = kb + (int64_t)r * 128;
    float sq = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(row + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += (float)x[e] * (float)x[e];
    }
    sq += __shfl_xor(sq, 1, kWave);
    sq += __shfl_xor(sq, 2, kWave);
    best = fmaxf(best, sq);
  }
#pragma unroll
  for (int o = 4; o < kWave; o <<= 1) best = fmaxf(best, __shfl_xor(best, o, kWave));
  __shared__ float red[4];
  if (tid % kWave == 0) red[tid / kWave] = best;
  __syncthreads();
  if (tid == 0) out[bh * parts + part] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

hipError_t launch_key_norm_max(const void* k, float* out, int64_t bh, int Lt, int parts, hipStream_t st) {
  if (bh <= 0 || Lt <= 0) return hipSuccess;
  if (bh * parts > 0x7FFFFFFF) return hipErrorInvalidValue;
  key_norm_max_kernel<<<(unsigned)(bh * parts), 256, 0, st>>>((const bf16*)k, out, Lt, parts);
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

hipError_t launch_window_attn_mxfp8(const AttnParams& p, hipStream_t st) {
  if (p.bm != attn_query_tile(1, 128)) return hipErrorInvalidValue;
  if (p.total > 0) window_attn_mxfp8_d128_kernel<<<p.total, 256, 0, st>>>(p);
  return hipGetLastError();
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
