// Internal interface between the C ABI (vdn_api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vdn {

// Softmax-branch tiling of the generic kernel: queries per workgroup and keys
// per LDS tile.  bf16 with head_dim 128 runs the gfx950-specific kernel with
// 256 queries per workgroup.
constexpr int kAttnBM = 128;
constexpr int kAttnBN = 64;
constexpr int kAttnBMv2 = 256;
inline __host__ __device__ bool attn_uses_v2(int dtype, int d) { return dtype == 1 && d == 128; }
inline __host__ __device__ int attn_query_tile(int dtype, int d) {
  return attn_uses_v2(dtype, d) ? kAttnBMv2 : kAttnBM;
}
// Linear-branch readout: tokens per workgroup (4 waves x 32).
constexpr int kReadoutBT = 128;
// Linear-branch scan: state rows per workgroup.
constexpr int kScanRows = 16;

// Work decomposition of the window/anchor softmax.  Per (batch, head) the
// work items are: the query tiles of every chunk's non-anchor video frames
// (key set = the chunk window, the anchor frames outside it, and the context
// tokens), then for each dense query group - the first and the last frame
// (anchors) and the context tokens, whose key set is the whole sequence - its
// query tiles times `nsplit` key splits of that sequence.  Rows per (batch,
// head): Lt = T*N video tokens followed by ctx context tokens.
constexpr int kMaxDenseGroups = 3;
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;   // nullable, row stride ldg
  void* out;          // row stride ldo
  float* lse;         // nullable, [B, H, Lt]
  float* part_o;      // dense-row partials [B, H, nsplit, dense_rows, d] (nsplit > 1)
  float* part_ml;     // dense-row partial (max, sum) [B, H, nsplit, dense_rows, 2]
  int64_t ldg, ldo;
  int B, H, T, N;
  int L, ctx, Lt;     // video tokens, context tokens, rows per (batch, head)
  int C, W, a0, a1;
  int nC;
  int tiles0, tilesM, tilesL;
  int n_window_tiles;
  int nG;                               // dense query groups
  int grp_row0[kMaxDenseGroups];        // first row of the group
  int grp_rows[kMaxDenseGroups];        // rows of the group
  int grp_tiles[kMaxDenseGroups];       // query tiles of the group
  int grp_part[kMaxDenseGroups];        // offset of the group's rows among the dense rows
  int dense_rows;                       // rows of all dense groups
  int nsplit;
  int keys_per_split;
  int tiles_per_bh;
  int total;
  int bm;             // queries per work item (attn_query_tile)
  float scale_log2;
  const void* qs;     // MXFP8 kernel: E8M0 scales of q and k [B, H, Lt, 4] (q, k hold E4M3 codes)
  const void* ks;
  const float* kmax;  // nullable: max squared key norm of each (batch, head) in kmax_parts parts
  int kmax_parts;
  unsigned char* fallback;   // with kmax: per work item, 1 = needs the running-maximum kernel
};

enum GemmEpilogue { kEpiStore = 0, kEpiSigmoid = 1 };

// dtype: 0 = fp32, 1 = bf16 (the vdn_dtype values).
hipError_t launch_transpose(int dtype, const void* src, void* dst, int rows, int cols,
                            int64_t ld_dst, hipStream_t st);
hipError_t launch_gemm_nt(int dtype, int epi, const void* A, const void* Bt, void* C, int M,
                          int N, int K, int64_t lda, int64_t ldb, int64_t ldc, hipStream_t st);
hipError_t launch_window_attn(int dtype, int d, const AttnParams& p, hipStream_t st);
hipError_t launch_attn_merge(int dtype, int d, const AttnParams& p, hipStream_t st);
// per (batch, head) and part of its Lt rows: the largest squared L2 norm of a
// key row (bf16, head_dim 128), out [B*H, parts]
hipError_t launch_key_norm_max(const void* k, float* out, int64_t bh, int Lt, int parts, hipStream_t st);
constexpr int kKeyNormParts = 64;
// head_dim 128, bf16 v / gate / out; p.q, p.k E4M3 codes with scales p.qs, p.ks
hipError_t launch_window_attn_mxfp8(const AttnParams& p, hipStream_t st);
// MXFP8 (E4M3 codes, one E8M0 scale per 32 consecutive elements) of n_elems bf16 values
hipError_t launch_mxfp8_quantize(const void* x, int64_t n_elems, void* codes, void* scales,
                                 hipStream_t st);
// Frame f = bh*T + t of q/k/v starts at row (f / T) * Lt + (f % T) * N (Lt rows per (batch, head):
// T*N video tokens, then context tokens the linear branch does not read).
hipError_t launch_vda_gram(int dtype, int d, const void* k, const void* v, const float* beta,
                           float* A, float* Bm, int nframes, int T, int N, int Lt, hipStream_t st);
hipError_t launch_vda_solve(int d, float* AM, int nframes, hipStream_t st);   // AM: A in, M^T out
hipError_t launch_vda_scan(int d, const float* Mt, const float* Bm, const float* gamma,
                           float* states, __bf16* split, int BH, int T, hipStream_t st);
// out/gate rows: b * Lt + t * N + n; rows of context tokens are not written.
hipError_t launch_vda_readout(int dtype, int d, const void* q, const float* states,
                              const __bf16* split, const float* rms_w, const void* gate,
                              int64_t ldg, void* out, int64_t ldo, int B, int H, int T, int N,
                              int Lt, float eps, hipStream_t st);
// Zero rows [row0, row0 + nrows) of `cols` elements of every batch entry of a
// [B, rows_per_batch, ld] matrix (element size es bytes).
hipError_t launch_zero_rows(void* base, int B, int64_t rows_per_batch, int64_t row0, int64_t nrows,
                            int64_t ld, int64_t cols, int es, hipStream_t st);
// flag[0] = 1 if some beta[i] < 0 or gamma[i] outside [0, 1] (i < n), else 0.
hipError_t launch_param_check(const float* gamma, const float* beta, int n, int* flag,
                              hipStream_t st);

}  // namespace vdn
