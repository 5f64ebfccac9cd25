// Device helpers shared by the gfx950 kernels of the hybrid GQA attention path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spark {

// Head layout of the model: 16 query heads over 4 KV heads of dimension 256, sliding
// window 512 (Spark-X2.6-4B-Base hybrid attention explainer, eliteato.com/news/34565,
// sections "配套效率设计" and "滑动窗口 512").
constexpr int kQHeads = 16;
constexpr int kKvHeads = 4;
constexpr int kGroup = kQHeads / kKvHeads;
constexpr int kHeadDim = 256;
constexpr int kWindow = 512;

constexpr int kSliding = 0;
constexpr int kFull = 1;

// Per layer type: RoPE base and rotated width (explainer page, parameter table of
// section "全局注意力 5M 基频 RoPE": theta 1e4 over all dims on sliding layers, theta 5e6
// over the first quarter of the head on full layers).
template <int LT> struct LayerTraits;
template <> struct LayerTraits<kSliding> {
  static constexpr double kTheta = 10000.0;
  static constexpr int kRot = 256;
  static constexpr bool kWindowed = true;
};
template <> struct LayerTraits<kFull> {
  static constexpr double kTheta = 5000000.0;
  static constexpr int kRot = 64;
  static constexpr bool kWindowed = false;
};

// Softmax runs in the log2 domain: score * (1/16) * log2(e), then exp2.
constexpr float kScoreScaleLog2 = 0.0625f * 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two floats to a packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_global16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Operand layout: lane l holds A[l % 32][8 * (l / 32) + j] and B[8 * (l / 32) + j][l % 32]
// for j = 0..7; result element v of lane l is D[8 * (v / 4) + 4 * (l / 32) + v % 4][l % 32].
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l holds A[l % 16][8 * (l / 16) + j] and B[8 * (l / 16) + j][l % 16]; result
// element v of lane l is D[4 * (l / 16) + v][l % 16].
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Inverse frequency of rotary pair m in revolutions per position:
// theta^(-2m/r) / (2 pi), in fp64.
__device__ __forceinline__ double rope_inv_rev(int m, int rot, double log2_theta) {
  return exp2(-(2.0 * m / rot) * log2_theta) * 0.15915494309189535;
}

// The same inverse frequencies as a table evaluated at compile time, for kernels that
// should not spend a barrier and an fp64 exp2 per workgroup on them: natural log by the
// atanh series after reducing to [1, 2), exp2 by the Taylor series of e^y after splitting
// off the integer part.  Relative error below 3e-15 (the fp64 rounding of log2 theta,
// scaled by the exponent), i.e. under 1e-9 revolution of angle at position 2^20.
namespace cx {
constexpr double kLn2 = 0.69314718055994530942;
constexpr double ln(double x) {
  int k = 0;
  while (x >= 2.0) { x *= 0.5; ++k; }
  while (x < 1.0) { x *= 2.0; --k; }
  const double z = (x - 1.0) / (x + 1.0), z2 = z * z;
  double term = z, sum = 0.0;
  for (int i = 0; i < 60; ++i) { sum += term / (2 * i + 1); term *= z2; }
  return 2.0 * sum + k * kLn2;
}
constexpr double exp2(double x) {
  int n = 0;
  while (x > 0.5) { x -= 1.0; ++n; }
  while (x < -0.5) { x += 1.0; --n; }
  const double y = x * kLn2;
  double term = 1.0, sum = 1.0;
  for (int i = 1; i < 30; ++i) { term *= y / i; sum += term; }
  for (; n > 0; --n) sum *= 2.0;
  for (; n < 0; ++n) sum *= 0.5;
  return sum;
}
}  // namespace cx

template <int LT>
struct RopeTable {
  double inv_rev[LayerTraits<LT>::kRot / 2];   // theta^(-2m/r) / (2 pi), revolutions per position
};
template <int LT>
constexpr RopeTable<LT> make_rope_table() {
  using T = LayerTraits<LT>;
  RopeTable<LT> t{};
  const double log2_theta = cx::ln(T::kTheta) / cx::kLn2;
  for (int m = 0; m < T::kRot / 2; ++m) t.inv_rev[m] = cx::exp2(-(2.0 * m / T::kRot) * log2_theta) * 0.15915494309189535;
  return t;
}
constexpr RopeTable<kSliding> kRopeSliding = make_rope_table<kSliding>();
// theta^(-2 d / r) of the sliding layer for a pair offset d = 8 k, k = 0..3.
constexpr double rope_step8(int k) {
  return cx::exp2(-(2.0 * 8 * k / LayerTraits<kSliding>::kRot) * (cx::ln(LayerTraits<kSliding>::kTheta) / cx::kLn2));
}
constexpr double kRopeStep8[4] = {1.0, rope_step8(1), rope_step8(2), rope_step8(3)};

// cos and sin of the rotary angle of position p for a pair whose inverse frequency is
// inv_rev revolutions per position.  The angle is reduced to [0, 1) revolution in fp64
// (exact to ~1e-10 rev for p < 2^20) before the hardware sin/cos, whose argument is in
// revolutions.
__device__ __forceinline__ void rope_cos_sin(double p, double inv_rev, float& c, float& s) {
  double a = p * inv_rev;
  a -= floor(a);
  const float f = (float)a;
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

// Rotate the 8 pairs (x1[j], x2[j]) held as two 16-byte bf16 chunks, in place, at
// position p; inv(j) gives pair j's inverse frequency in revolutions per position.
template <class Inv>
__device__ __forceinline__ void rope_rotate_pairs(u32x4& x1, u32x4& x2, double p, Inv inv) {
  u32x4 y1, y2;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float c0, s0, c1, s1;
    rope_cos_sin(p, inv(2 * w), c0, s0);
    rope_cos_sin(p, inv(2 * w + 1), c1, s1);
    const float a0 = bf16_lo(x1[w]), a1 = bf16_hi(x1[w]);
    const float b0 = bf16_lo(x2[w]), b1 = bf16_hi(x2[w]);
    y1[w] = pack_bf16x2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
    y2[w] = pack_bf16x2(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
    // One pair of rotations at a time: overlapping all eight sin/cos evaluations (with
    // their fp64 angle reductions) costs registers the callers cannot spare.
    __builtin_amdgcn_sched_barrier(0);
  }
  x1 = y1;
  x2 = y2;
}

// The same with inverse frequencies inv[m0 + j] (a table in LDS).
__device__ __forceinline__ void rope_rotate_chunks(u32x4& x1, u32x4& x2, double p,
                                                   const double* inv, int m0) {
  rope_rotate_pairs(x1, x2, p, [&](int j) { return inv[m0 + j]; });
}

__device__ __forceinline__ float sigmoidf_fast(float g) {
  return 1.0f / (1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

}  // namespace spark
