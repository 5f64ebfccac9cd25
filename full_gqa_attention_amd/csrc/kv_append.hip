// KV-cache append on gfx950: rotate each new key at its position and store it, with its
// value, in the layer's cache: slot = position on full layers (contiguous cache, 4 KB per
// token per layer: F16 vs Q4 comparison page, hotelren.com/news/5475707, section 一),
// slot = position mod 512 on sliding layers (a ring holding exactly the window,
// Sharp-Spark-X2.5-4B-GGUF guide, mpbf.cn/news/67460, section 三).
// Sixteen threads own one (token, KV head) row: each loads a rotary pair of 16-byte
// chunks, so the row is read and written as 512 contiguous bytes.
#include "spark_device.hpp"
#include "spark_launch.hpp"

namespace spark {
namespace {

constexpr int kThreads = 256;              // 4 tokens x 4 KV heads x 16 threads
constexpr int kTokensPerBlock = 4;

template <int LT>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  using T = LayerTraits<LT>;
  __shared__ double s_inv[T::kRot / 2];
  const int tid = threadIdx.x;
  if (tid < T::kRot / 2) s_inv[tid] = rope_inv_rev(tid, T::kRot, log2(T::kTheta));
  __syncthreads();

  const int b = blockIdx.y;
  const int t = blockIdx.x * kTokensPerBlock + (tid >> 6);
  const int g = (tid >> 4) & 3;
  const int c = tid & 15;
  if (t >= a.n_new) return;
  if (LT == kSliding && t < a.n_new - kWindow) return;   // overwritten later in the ring
  const int p = a.pos[b] + t;
  if (p < 0) return;
  const int slot = (LT == kFull) ? p : (p & (kWindow - 1));
  if (slot >= a.cache_cap) return;                        // never write past the cache

  int off_a, off_b;
  bool rot;
  if (LT == kSliding) {
    off_a = 8 * c; off_b = 128 + 8 * c; rot = true;
  } else if (c < 4) {
    off_a = 8 * c; off_b = 32 + 8 * c; rot = true;
  } else {
    off_a = 64 + 16 * (c - 4); off_b = off_a + 8; rot = false;
  }
  const size_t src = (((size_t)b * a.n_new + t) * kKvHeads + g) * kHeadDim;
  const size_t dst = (((size_t)b * a.cache_cap + slot) * kKvHeads + g) * kHeadDim;
  u32x4 k0 = ld_global16(a.k + src + off_a);
  u32x4 k1 = ld_global16(a.k + src + off_b);
  if (rot) rope_rotate_chunks(k0, k1, (double)p, s_inv, off_a);
  st_global16(a.cache_k + dst + off_a, k0);
  st_global16(a.cache_k + dst + off_b, k1);
  st_global16(a.cache_v + dst + 8 * c, ld_global16(a.v + src + 8 * c));
  st_global16(a.cache_v + dst + 128 + 8 * c, ld_global16(a.v + src + 128 + 8 * c));
}

// 8-bit append: the row's rotated key (fp32, never rounded to bf16) and its value are
// stored as q8_0 blocks of 32 along head_dim (Sharp-Spark-X2.5-4B-GGUF guide, section 四:
// the q8_0 KV cache, 36 -> 19 KB per token).  Per block, in fp32: d = max|x| / 127 and
// code = round(x * (1/d)), half away from zero (0 when d = 0); d is stored as fp16
// (nearest even).  Thirty-two threads own one (token, KV head) row, eight values each, so
// a block is four neighbouring lanes.
constexpr int kQ8RowsPerBlock = kThreads / 32;   // 2 tokens x 4 KV heads

__device__ __forceinline__ void quantize8(const float (&x)[8], int8_t* codes, uint16_t* scales, int c) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  const float d = m / 127.0f;                        // IEEE division, as the reference
  const float inv = d > 0.0f ? 1.0f / d : 0.0f;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = (int)roundf(x[j] * inv);           // half away from zero, |q| <= 127
    w[j >> 2] |= (uint32_t)(q & 0xff) << (8 * (j & 3));
  }
  *reinterpret_cast<u32x2*>(codes + 8 * c) = u32x2{w[0], w[1]};
  if ((c & 3) == 0) scales[c >> 2] = __builtin_bit_cast(uint16_t, (_Float16)d);
}

template <int LT>
__global__ __launch_bounds__(kThreads) void append_q8_kernel(AppendQ8Args a) {
  using T = LayerTraits<LT>;
  __shared__ double s_inv[T::kRot / 2];
  const int tid = threadIdx.x;
  if (tid < T::kRot / 2) s_inv[tid] = rope_inv_rev(tid, T::kRot, log2(T::kTheta));
  __syncthreads();

  const int b = blockIdx.y;
  const int t = blockIdx.x * (kQ8RowsPerBlock / kKvHeads) + (tid >> 7);
  const int g = (tid >> 5) & 3;
  const int c = tid & 31;                            // 8-value chunk of the row
  // Every lane of a row stays to the end (the block maximum is a four-lane shuffle);
  // rows that write nothing are whole 32-lane groups, so skipping them is uniform per row.
  bool live = t < a.n_new && !(LT == kSliding && t < a.n_new - kWindow);
  const int p = live ? a.pos[b] + t : 0;
  live = live && p >= 0;
  const int slot = (LT == kFull) ? p : (p & (kWindow - 1));
  live = live && slot < a.cache_cap;
  if (!live) return;

  const size_t src = (((size_t)b * a.n_new + t) * kKvHeads + g) * kHeadDim;
  const size_t row = ((size_t)b * a.cache_cap + slot) * kKvHeads + g;
  float x[8];
  // Key: rotate-half pairs (m, m + r/2) for m < r/2; this lane computes its own half.
  {
    const u32x4 own = ld_global16(a.k + src + 8 * c);
    const int half_chunks = T::kRot / 16;            // chunks in the first half of the slice
    const bool rot = 8 * c < T::kRot;
    if (rot) {
      const bool first = c < half_chunks;
      const u32x4 other = ld_global16(a.k + src + 8 * (first ? c + half_chunks : c - half_chunks));
      const int m0 = 8 * (first ? c : c - half_chunks);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float c0, s0, c1, s1;
        rope_cos_sin((double)p, s_inv[m0 + 2 * w], c0, s0);
        rope_cos_sin((double)p, s_inv[m0 + 2 * w + 1], c1, s1);
        const float x1a = first ? bf16_lo(own[w]) : bf16_lo(other[w]);
        const float x1b = first ? bf16_hi(own[w]) : bf16_hi(other[w]);
        const float x2a = first ? bf16_lo(other[w]) : bf16_lo(own[w]);
        const float x2b = first ? bf16_hi(other[w]) : bf16_hi(own[w]);
        x[2 * w] = first ? x1a * c0 - x2a * s0 : x2a * c0 + x1a * s0;
        x[2 * w + 1] = first ? x1b * c1 - x2b * s1 : x2b * c1 + x1b * s1;
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        x[2 * w] = bf16_lo(own[w]);
        x[2 * w + 1] = bf16_hi(own[w]);
      }
    }
  }
  quantize8(x, a.k_codes + row * kHeadDim, a.k_scales + row * 8, c);
  {
    const u32x4 vv = ld_global16(a.v + src + 8 * c);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = bf16_lo(vv[w]);
      x[2 * w + 1] = bf16_hi(vv[w]);
    }
  }
  quantize8(x, a.v_codes + row * kHeadDim, a.v_scales + row * 8, c);
}

}  // namespace

hipError_t launch_append_q8(int layer_type, const AppendQ8Args& a, hipStream_t stream) {
  constexpr int kTok = kQ8RowsPerBlock / kKvHeads;
  const dim3 grid((a.n_new + kTok - 1) / kTok, a.batch);
  if (layer_type == kSliding)
    hipLaunchKernelGGL(append_q8_kernel<kSliding>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(append_q8_kernel<kFull>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_append(int layer_type, const AppendArgs& a, hipStream_t stream) {
  const dim3 grid((a.n_new + kTokensPerBlock - 1) / kTokensPerBlock, a.batch);
  if (layer_type == kSliding)
    hipLaunchKernelGGL(append_kernel<kSliding>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<kFull>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spark
