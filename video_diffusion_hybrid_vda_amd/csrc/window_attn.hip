// Softmax branch of Video DeltaNet: sliding-window attention at VAE-chunk
// granularity with two-way boundary anchors (10100.com article on Video
// DeltaNet, 方法概述 part 1).  A query frame in chunk c = t / C sees the key
// frames of chunks c-W .. c+W plus the first and last frame; the first and
// last frame see every frame.  One softmax runs over the union of allowed
// keys; the output is multiplied by the branch gate.
//
// Flash-style forward on MFMA.  Each wave owns 32 queries and computes
// S^T = K Q^T so that every lane holds scores of a single query: the online
// softmax statistics are per lane, and the bf16 P^T tile feeds the P V
// product as the MFMA B operand without any register shuffle (the key order
// inside one 32-key step is permuted identically for P^T and V^T).
// Anchor query frames, whose key set is the whole sequence, are split along
// the keys; a merge kernel combines the partial (max, sum, output) triples.
#include <math.h>

#include "vdn_common.h"
#include "vdn_internal.h"

namespace vdn {

template <typename T, int D>
__global__ __launch_bounds__(256) void window_attn_kernel(AttnParams p) {
  using MM = Mma<T>;
  constexpr int KP = MM::kPack, KS = MM::kStep;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int BM = kAttnBM, BN = kAttnBN;
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
  const int lid = xcd_remap(blockIdx.x, p.total);
  const int bh = lid / p.tiles_per_bh;
  const int w = lid - bh * p.tiles_per_bh;
  const int b = bh / p.H, h = bh - b * p.H;
  const int NL = p.T * p.N;
  int qbeg, qend, nint = 0, pidx = -1, afr = 0;
  int kb[3], ke[3];
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
    qbeg = qf0 * p.N + j * BM;
    qend = min(qbeg + BM, qf1 * p.N);
    const int kf0 = max(0, (c - p.W) * p.C);
    const int kf1 = min(p.T, (c + p.W + 1) * p.C);
    if (p.a0 && kf0 > 0) { kb[nint] = 0; ke[nint] = p.N; ++nint; }
    kb[nint] = kf0 * p.N; ke[nint] = kf1 * p.N; ++nint;
    if (p.a1 && kf1 < p.T) { kb[nint] = (p.T - 1) * p.N; ke[nint] = NL; ++nint; }
  } else {
    int u = w - p.n_window_tiles;
    const int per_anchor = p.nsplit * p.tiles_per_anchor;
    const int a = u / per_anchor;
    u -= a * per_anchor;
    const int s = u / p.tiles_per_anchor;
    const int j = u - s * p.tiles_per_anchor;
    afr = p.anchor_frame[a];
    qbeg = afr * p.N + j * BM;
    qend = min(qbeg + BM, (afr + 1) * p.N);
    kb[0] = s * p.keys_per_split;
    ke[0] = min(kb[0] + p.keys_per_split, NL);
    nint = 1;
    if (p.nsplit > 1) pidx = ((a * p.B + b) * p.H + h) * p.nsplit + s;
  }

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
    if (pidx < 0) {
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
      const int64_t prow = (int64_t)pidx * p.N + (qrow - afr * p.N);
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

// Combine the key splits of the anchor query rows: out = sum_s 2^(m_s - M) O_s
// / sum_s 2^(m_s - M) l_s, then gate.  One thread per (query, quarter of d).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  const int nqb = (p.N + 63) / 64;
  const int qb = blockIdx.x % nqb;
  const int abh = blockIdx.x / nqb;             // (a*B + b)*H + h
  const int h = abh % p.H;
  const int ab = abh / p.H;
  const int b = ab % p.B, a = ab / p.B;
  const int n = qb * 64 + threadIdx.x / 4;
  if (n >= p.N) return;
  const int dq = threadIdx.x % 4;
  constexpr int DQ = D / 4;
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s)
    M = fmaxf(M, p.part_ml[((int64_t)(abh * p.nsplit + s) * p.N + n) * 2]);
  float L = 0.f;
  float acc[DQ];
#pragma unroll
  for (int x = 0; x < DQ; ++x) acc[x] = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const int64_t prow = (int64_t)(abh * p.nsplit + s) * p.N + n;
    const float wgt = fast_exp2(p.part_ml[prow * 2] - M);
    L += wgt * p.part_ml[prow * 2 + 1];
#pragma unroll
    for (int x = 0; x < DQ; ++x) acc[x] += wgt * p.part_o[prow * D + dq * DQ + x];
  }
  const float inv = 1.f / L;
  const int NL = p.T * p.N;
  const int qrow = p.anchor_frame[a] * p.N + n;
  const int64_t orow = (int64_t)b * NL + qrow;
  const T* gate = (const T*)p.gate;
  T* out = (T*)p.out;
#pragma unroll
  for (int x = 0; x < DQ; ++x) {
    const int dd = dq * DQ + x;
    float val = acc[x] * inv;
    if (gate) val *= to_f32(gate[orow * p.ldg + h * D + dd]);
    out[orow * p.ldo + h * D + dd] = from_f32<T>(val);
  }
  if (p.lse && dq == 0) p.lse[(int64_t)(b * p.H + h) * NL + qrow] = (M + log2f(L)) * kLn2;
}

template <typename T, int D>
static hipError_t launch_attn_t(const AttnParams& p, hipStream_t st) {
  if (p.total > 0) window_attn_kernel<T, D><<<p.total, 256, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.nsplit > 1 && p.nA > 0) {
    const int blocks = p.nA * p.B * p.H * ((p.N + 63) / 64);
    attn_merge_kernel<T, D><<<blocks, 256, 0, st>>>(p);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_window_attn(int dtype, int d, const AttnParams& p, hipStream_t st) {
  if (dtype == 1) {
    if (d == 32) return launch_attn_t<bf16, 32>(p, st);
    if (d == 64) return launch_attn_t<bf16, 64>(p, st);
    return launch_attn_t<bf16, 128>(p, st);
  }
  if (d == 32) return launch_attn_t<float, 32>(p, st);
  if (d == 64) return launch_attn_t<float, 64>(p, st);
  return launch_attn_t<float, 128>(p, st);
}

}  // namespace vdn
