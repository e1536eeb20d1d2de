// Device-side building blocks shared by the VDN kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16x16 output-tile MFMA family.  For both element types the operand layout
// is: lane l holds A[l%16][(l/16)*kPack + e] and B[(l/16)*kPack + e][l%16]
// (e < kPack); the fp32 accumulator holds C[(l/16)*4 + r][l%16] (r < 4).
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int kPack = 8;    // elements per lane per operand
  static constexpr int kStep = 32;   // reduction depth of one instruction
  typedef bf16x8 Frag;
  __device__ __forceinline__ static f32x4 run(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static Frag load(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  __device__ __forceinline__ static Frag zero() { return Frag{}; }
};

template <> struct Mma<float> {
  static constexpr int kPack = 1;
  static constexpr int kStep = 4;
  typedef float Frag;
  __device__ __forceinline__ static f32x4 run(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static Frag load(const float* p) { return *p; }
  __device__ __forceinline__ static Frag zero() { return 0.f; }
};

// Remap the hardware workgroup id so that each XCD (which owns its own L2)
// receives one contiguous range of logical work items.  Workgroup i is
// dispatched to XCD i % 8; the first (total % 8) XCDs get one extra item.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  const int xcd = pid % kNumXcd;
  const int local = pid / kNumXcd;
  const int per = total / kNumXcd;
  const int rem = total % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// logistic function with the hardware reciprocal (1 ulp) in place of the
// correctly rounded divide, which costs about ten instructions per element
__device__ __forceinline__ float sigmoidf(float x) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
}

// 16-byte global/LDS chunk helpers.
struct alignas(16) Chunk16 { uint32_t w[4]; };

__device__ __forceinline__ Chunk16 zero_chunk() { return Chunk16{{0u, 0u, 0u, 0u}}; }

}  // namespace vdn
