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

}  // namespace

hipError_t launch_append(int layer_type, const AppendArgs& a, hipStream_t stream) {
  const dim3 grid((a.n_new + kTokensPerBlock - 1) / kTokensPerBlock, a.batch);
  if (layer_type == kSliding)
    hipLaunchKernelGGL(append_kernel<kSliding>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<kFull>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spark
