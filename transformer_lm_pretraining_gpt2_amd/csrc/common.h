// common.h -- device helpers shared by the gfx950 kernels of the GPT-2 step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// FP8 E4M3 (OCP encoding on gfx950) values are stored as bytes.
typedef unsigned char fp8e4;
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Eight consecutive elements along a matmul's reduction dimension: the
// per-lane operand of one (virtual) 32x32x16 MFMA step.  FP8: 32 consecutive
// elements, the per-lane operand of one 32x32x64 MFMA.
template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };
template <> struct Frag<fp8e4> { typedef i32x8 type; };
// reduction depth of one MFMA step for an operand type
template <typename T> struct KStep { static constexpr int k = 16; };
template <> struct KStep<fp8e4> { static constexpr int k = 64; };

// Four consecutive output elements (one lane's run in a 32x32 accumulator).
template <typename T> struct Quad;
template <> struct Quad<bf16> { typedef bf16x4 type; };
template <> struct Quad<float> { typedef f32x4 type; };

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 ld8(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void st8(bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ void st8(float* p, f32x8 v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// One 32x32x16 product: acc[32x32] += A(32 rows x 16 k) * B(16 k x 32 cols).
// Lane l holds row/col l%32 of its operand and 8 of the 16 k values; which 8
// is fixed by the lane group g = l/32 and the slot, identically for A and B,
// so the sum runs over all 16.  Accumulator element r of lane l sits at
// row 8*(r/4) + 4*(l/32) + r%4, col l%32 (layout checked on gfx950).
__device__ __forceinline__ void mma16(f32x16& acc, bf16x8 a, bf16x8 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
// fp32: eight 32x32x2 MFMAs; MFMA s pairs slot s of lane group 0 with slot s
// of lane group 1 (its two k values), so all 16 (group, slot) pairs are summed.
__device__ __forceinline__ void mma16(f32x16& acc, f32x8 a, f32x8 b) {
#pragma unroll
  for (int s = 0; s < 8; s++) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
}
// FP8 E4M3 x E4M3: one 32x32x64 MFMA (block scales 2^0); each lane supplies 32
// reduction values, the same 32 slots for both operands, so all 64 are summed.
__device__ __forceinline__ void mma16(f32x16& acc, i32x8 a, i32x8 b) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x) { return (T)x; }

// Index of the calling wave in its block, known to the compiler to be the same
// for every lane of the wave: branches on it (and on values derived from it)
// become scalar branches instead of masked execution of both sides.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// tanh-approximate GELU and its derivative ("Karpathy's four-hour GPT-2
// reproduction in one post", what I checked myself: GPT-2 uses the tanh form).
// With z = 2*sqrt(2/pi)*(x + 0.044715 x^3), 0.5*(1 + tanh(z/2)) = sigmoid(z), so
// gelu(x) = x * s and gelu'(x) = s + x * s * (1 - s) * dz/dx, s = sigmoid(z);
// sigmoid is evaluated with the hardware exp2 and reciprocal.
__device__ __forceinline__ float gelu_sigmoid(float x) {
  const float k2 = 2.f * 0.7978845608028654f * 1.4426950408889634f;  // 2*sqrt(2/pi)*log2(e)
  const float z2 = k2 * x * (1.f + 0.044715f * x * x);               // z * log2(e)
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z2));
}
__device__ __forceinline__ float gelu_tanh(float x) { return x * gelu_sigmoid(x); }
// gelu'(x) from the same sigmoid s = gelu_sigmoid(x)
__device__ __forceinline__ float gelu_tanh_grad_s(float x, float s) {
  const float k = 2.f * 0.7978845608028654f;
  return s + x * s * (1.f - s) * k * (1.f + 3.f * 0.044715f * x * x);
}

// Blocks are dispatched round-robin over the 8 XCDs (each with its own L2).
// Renumber so each XCD gets one contiguous range of logical block ids, which
// keeps neighbouring tiles (sharing operand panels) in the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  if (nblocks % 8 != 0) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

// The same for any block count n = 8q + r: XCDs 0..r-1 take q + 1 logical
// ids each, the others q (dispatched id bid goes to XCD bid % 8 as its
// (bid / 8)-th block).
__device__ __forceinline__ int xcd_remap_any(int bid, int nblocks) {
  const int q = nblocks / 8, r = nblocks % 8, x = bid % 8;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + bid / 8;
}
