// MXFP8 quantisation of bf16 tensors for the softmax branch's 8-bit mode.
//
// [P3] (10100.com article on Video DeltaNet, section 实验结果, the paragraph
// on scaling with sequence length) runs the 8-step denoiser in MXFP8.  The
// format is MXFP8 of the OCP Microscaling (MX) specification v1.0: blocks of
// 32 consecutive elements in OCP FP8 E4M3 (bias 7, largest finite 448) with
// one E8M0 scale 2^(code - 127) per block.  The block's exponent is
// floor(log2 max|x|) - 8 (8 = the largest E4M3 exponent), clamped to
// [-127, 127], 0 code for an all-zero block; elements are x / 2^exponent
// rounded to the nearest E4M3 value, ties to the even code, saturating at 448,
// with the sign bit of x.
//
// One thread per block: 64 bytes in, 32 code bytes and one scale byte out.
// The scaling is an exact ldexp; the rounding works on the fp32 bit pattern
// (normal range) or on a * 2^9 (subnormal range, rint is ties-to-even).
#include "vdn_common.h"
#include "vdn_internal.h"

namespace vdn {

__device__ __forceinline__ unsigned e4m3_magnitude(float a) {
  if (!(a < 448.f)) return 0x7Eu;                                  // saturate
  if (a < 0.015625f) return (unsigned)__builtin_rintf(a * 512.f);  // m * 2^-9, m = 0..8
  const unsigned bits = __float_as_uint(a);
  // round the 23-bit mantissa to 3 bits, ties to even; a carry moves into the exponent
  const unsigned r = bits + 0x7FFFFu + ((bits >> 20) & 1u);
  return (r >> 20) - (120u << 3);                                  // rebias 127 -> 7
}

__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const bf16* __restrict__ x,
                                                             unsigned char* __restrict__ codes,
                                                             unsigned char* __restrict__ scales,
                                                             int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = src[i];
    const unsigned u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int se = -127;
  if (amax > 0.f) se = max(-127, min(127, ilogbf(amax) - 8));
  scales[b] = (unsigned char)(se + 127);
  unsigned packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    unsigned w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float xv = v[4 * i + j];
      const unsigned c = e4m3_magnitude(fabsf(ldexpf(xv, -se))) | (xv < 0.f ? 0x80u : 0u);
      w |= c << (8 * j);
    }
    packed[i] = w;
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

hipError_t launch_mxfp8_quantize(const void* x, int64_t n_elems, void* codes, void* scales,
                                 hipStream_t st) {
  const int64_t nblocks = n_elems / 32;
  if (nblocks == 0) return hipSuccess;
  mxfp8_quantize_kernel<<<(unsigned)((nblocks + 255) / 256), 256, 0, st>>>(
      (const bf16*)x, (unsigned char*)codes, (unsigned char*)scales, nblocks);
  return hipGetLastError();
}

}  // namespace vdn
