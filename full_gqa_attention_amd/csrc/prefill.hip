// Flash-attention prefill for the hybrid sliding/full GQA layer on gfx950.
//
// One workgroup = 8 waves = one KV head g of one sequence and a block of 64 query
// positions; wave w computes query head 4g + w/2 for 32 of those positions, so every K/V
// tile staged in LDS serves 4 query heads x 64 positions = 256 query rows (GQA sharing).
//
// Per tile of 32 keys (double-buffered in LDS, one barrier per tile):
//   * K rows are loaded, rotated (RoPE with the layer type's theta and width) in fp32,
//     rounded to bf16 and stored row-major; V rows are stored transposed so both MFMA
//     operands come from 16-byte LDS reads;
//   * S^T = K * Q^T on v_mfma_f32_32x32x16_bf16 (Q, rotated once, stays in registers),
//     so each lane owns one query row and its softmax statistics need no broadcast;
//   * online softmax in fp32 / log2 domain; the running maximum is only moved when a new
//     score exceeds it by more than 8 (so P <= 2^8), which makes the O rescale rare;
//   * O^T += V^T * P^T on the same MFMA, accumulators in fp32.
// Tiles wholly outside a wave's visible band are skipped; sliding layers only visit the
// 512-key band (Spark-X2.6-4B-Base hybrid attention explainer, eliteato.com/news/34565,
// section "滑动窗口 512": a token sees at most the last 512 tokens; full layers see every
// earlier token, section "36 层混合注意力排布").
// Epilogue: O / l * sigmoid(gate) (F16 vs Q4 comparison page, hotelren.com/news/5475707,
// section 三: one sigmoid gate per head), stored as bf16.  The workgroup that owns a
// key tile's positions also writes the rotated keys and values into the KV cache.
#include "spark_device.hpp"
#include "spark_launch.hpp"

namespace spark {
namespace {

constexpr int kBM = 64;           // query positions per workgroup
constexpr int kBN = 32;           // keys per tile
constexpr int kThreads = 512;     // 8 waves
constexpr int kKsStride = 264;    // bf16 per K row in LDS (256 + 8: conflict-free reads)
constexpr int kVtStride = 40;     // bf16 per transposed V row (32 keys + 8)
constexpr int kKsTile = kBN * kKsStride;
constexpr int kVtTile = kHeadDim * kVtStride;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

// Position of key `key` (0..31) of a tile inside a transposed V row: keys
// 16t + 8a + 4h + b are stored at 16t + 8h + 4a + b, which is the order in which the
// P^T operand of lane half h lists them (see the S^T result layout).
__device__ __forceinline__ int vt_slot(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

struct KvStage {
  u32x4 k[2];
  u32x4 v[2];
};

template <int LT>
__device__ __forceinline__ void k_chunk_offsets(int c, int& off_a, int& off_b, bool& rot) {
  if (LT == kSliding) {          // pairs (d, d + 128): thread c owns d in [8c, 8c + 8)
    off_a = 8 * c;
    off_b = 128 + 8 * c;
    rot = true;
  } else if (c < 4) {            // pairs (d, d + 32) for d < 32
    off_a = 8 * c;
    off_b = 32 + 8 * c;
    rot = true;
  } else {                       // dims 64..255 are not rotated
    off_a = 64 + 16 * (c - 4);
    off_b = off_a + 8;
    rot = false;
  }
}

template <int LT>
__device__ __forceinline__ void load_tile(const PrefillArgs& a, int b, int g, int k0, int tid,
                                          KvStage& st) {
  const int S = a.seq_len;
  {  // K: thread -> (key = tid / 16, chunk pair c = tid % 16)
    const int key = tid >> 4, c = tid & 15;
    int off_a, off_b;
    bool rot;
    k_chunk_offsets<LT>(c, off_a, off_b, rot);
    const int p = k0 + key;
    if (p < S) {
      const uint16_t* row = a.k + (((size_t)b * S + p) * kKvHeads + g) * kHeadDim;
      st.k[0] = ld_global16(row + off_a);
      st.k[1] = ld_global16(row + off_b);
    } else {
      st.k[0] = u32x4{0, 0, 0, 0};
      st.k[1] = u32x4{0, 0, 0, 0};
    }
  }
  {  // V: thread -> (key = tid % 32, dims [8dc, 8dc+8) and [128+8dc, 128+8dc+8))
    const int key = tid & 31, dc = tid >> 5;
    const int p = k0 + key;
    if (p < S) {
      const uint16_t* row = a.v + (((size_t)b * S + p) * kKvHeads + g) * kHeadDim;
      st.v[0] = ld_global16(row + 8 * dc);
      st.v[1] = ld_global16(row + 128 + 8 * dc);
    } else {
      st.v[0] = u32x4{0, 0, 0, 0};
      st.v[1] = u32x4{0, 0, 0, 0};
    }
  }
}

// Rotate the staged keys, write K and V^T into LDS, and (for tiles of this workgroup's
// own positions) into the KV cache.
template <int LT>
__device__ __forceinline__ void store_tile(const PrefillArgs& a, int b, int g, int k0, int q0,
                                           int tid, KvStage& st, uint16_t* ks, uint16_t* vt,
                                           const double* inv) {
  const int S = a.seq_len;
  const int cap = a.cache_cap;
  const bool own = a.cache_k != nullptr && k0 >= q0;
  {
    const int key = tid >> 4, c = tid & 15;
    int off_a, off_b;
    bool rot;
    k_chunk_offsets<LT>(c, off_a, off_b, rot);
    const int p = k0 + key;
    if (rot) rope_rotate_chunks(st.k[0], st.k[1], (double)p, inv, off_a);
    *reinterpret_cast<u32x4*>(ks + key * kKsStride + off_a) = st.k[0];
    *reinterpret_cast<u32x4*>(ks + key * kKsStride + off_b) = st.k[1];
    if (own && p < S && (LT == kFull || p >= S - kWindow)) {
      const int slot = (LT == kFull) ? p : (p & (kWindow - 1));
      uint16_t* dst = a.cache_k + (((size_t)b * cap + slot) * kKvHeads + g) * kHeadDim;
      st_global16(dst + off_a, st.k[0]);
      st_global16(dst + off_b, st.k[1]);
    }
  }
  {
    const int key = tid & 31, dc = tid >> 5;
    const int col = vt_slot(key);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int d0 = 128 * half + 8 * dc;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = st.v[half][w];
        vt[(d0 + 2 * w) * kVtStride + col] = (uint16_t)(x & 0xffffu);
        vt[(d0 + 2 * w + 1) * kVtStride + col] = (uint16_t)(x >> 16);
      }
    }
    const int p = k0 + key;
    if (own && p < S && (LT == kFull || p >= S - kWindow)) {
      const int slot = (LT == kFull) ? p : (p & (kWindow - 1));
      uint16_t* dst = a.cache_v + (((size_t)b * cap + slot) * kKvHeads + g) * kHeadDim;
      st_global16(dst + 8 * dc, st.v[0]);
      st_global16(dst + 128 + 8 * dc, st.v[1]);
    }
  }
}

template <int LT>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
  using T = LayerTraits<LT>;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2 * kKsTile];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2 * kVtTile];
  __shared__ double s_inv[T::kRot / 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int S = a.seq_len;
  const int units = a.batch * kKvHeads;

  // Block order: full layers take the longest (latest) query blocks first.
  const int id = blockIdx.x;
  const int bg = id % units;
  const int ord = id / units;
  const int qb = (LT == kFull) ? (a.nqb - 1 - ord) : ord;
  const int b = bg / kKvHeads;
  const int g = bg % kKvHeads;
  const int q0 = qb * kBM;

  if (tid < T::kRot / 2) s_inv[tid] = rope_inv_rev(tid, T::kRot, log2(T::kTheta));
  __syncthreads();

  // ---- Q fragments: lane holds row r32 of its 32-row slab, dims 16s + 8*half + j.
  const int hq = g * kGroup + (wave >> 1);
  const int r0 = q0 + 32 * (wave & 1);
  const int row = r0 + r32;
  bf16x8 qf[16];
  {
    u32x4 raw[16];
    if (row < S) {
      const uint16_t* qrow = a.q + (((size_t)b * S + row) * kQHeads + hq) * kHeadDim;
#pragma unroll
      for (int s = 0; s < 16; ++s) raw[s] = ld_global16(qrow + 16 * s + 8 * half);
    } else {
#pragma unroll
      for (int s = 0; s < 16; ++s) raw[s] = u32x4{0, 0, 0, 0};
    }
    const double p = (double)row;
    if (LT == kSliding) {        // chunk s pairs with chunk s + 8 (d + 128)
#pragma unroll
      for (int s = 0; s < 8; ++s) rope_rotate_chunks(raw[s], raw[s + 8], p, s_inv, 16 * s + 8 * half);
    } else {                     // chunk s (s < 2) pairs with chunk s + 2 (d + 32)
#pragma unroll
      for (int s = 0; s < 2; ++s) rope_rotate_chunks(raw[s], raw[s + 2], p, s_inv, 16 * s + 8 * half);
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = as_bf16x8(raw[s]);
  }

  // ---- key tiles this workgroup visits
  const int hi_key = min(q0 + kBM - 1, S - 1);
  const int lo_key = T::kWindowed ? max(0, q0 - (kWindow - 1)) : 0;
  const int kt_lo = lo_key / kBN;
  const int kt_hi = hi_key / kBN;

  f32x16 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x16{0};
  float m_run = -1e30f;
  float l_part = 0.0f;

  KvStage st;
  load_tile<LT>(a, b, g, kt_lo * kBN, tid, st);
  store_tile<LT>(a, b, g, kt_lo * kBN, q0, tid, st, s_k, s_vt, s_inv);
  __syncthreads();

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int buf = (kt - kt_lo) & 1;
    const int k0 = kt * kBN;
    const bool more = kt < kt_hi;
    if (more) load_tile<LT>(a, b, g, k0 + kBN, tid, st);

    const uint16_t* ks = s_k + buf * kKsTile;
    const uint16_t* vt = s_vt + buf * kVtTile;
    // Wave-uniform visibility of this tile for rows r0..r0+31.
    const bool any = (k0 <= r0 + 31) && (!T::kWindowed || k0 + kBN - 1 >= r0 - (kWindow - 1));
    if (any) {
      f32x16 sacc = f32x16{0};
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + r32 * kKsStride + 16 * s + 8 * half));
        sacc = mfma_32x32x16(ka, qf[s], sacc);
      }
      float t[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) t[v] = sacc[v] * kScoreScaleLog2;
      const bool edge = (k0 + kBN - 1 > r0) || (T::kWindowed && k0 < r0 + 31 - (kWindow - 1));
      if (edge) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + 8 * (v >> 2) + 4 * half + (v & 3);
          const bool vis = key <= row && (!T::kWindowed || key > row - kWindow);
          t[v] = vis ? t[v] : -INFINITY;
        }
      }
      float mt = t[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mt = fmaxf(mt, t[v]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      if (__any(mt > m_run + kRescaleThreshold)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] *= alpha;
        m_run = m_new;
      }
      bf16x8 pf[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 pk;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float p0 = __builtin_amdgcn_exp2f(t[8 * tt + 2 * w] - m_run);
          const float p1 = __builtin_amdgcn_exp2f(t[8 * tt + 2 * w + 1] - m_run);
          pk[w] = pack_bf16x2(p0, p1);
          l_part += bf16_lo(pk[w]) + bf16_hi(pk[w]);
        }
        pf[tt] = as_bf16x8(pk);
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4*>(
              vt + (32 * db + r32) * kVtStride + 16 * tt + 8 * half));
          o[db] = mfma_32x32x16(va, pf[tt], o[db]);
        }
      }
    }

    if (more) store_tile<LT>(a, b, g, k0 + kBN, q0, tid, st, s_k + (buf ^ 1) * kKsTile,
                             s_vt + (buf ^ 1) * kVtTile, s_inv);
    __syncthreads();
  }

  // ---- epilogue: O / l * sigmoid(gate), bf16
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (row < S) {
    const float gl = bf16_to_f32(a.gate[((size_t)b * S + row) * kQHeads + hq]);
    const float scale = sigmoidf_fast(gl) / l_tot;
    uint16_t* orow = a.out + (((size_t)b * S + row) * kQHeads + hq) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        u32x2 w;
        w[0] = pack_bf16x2(o[db][4 * qd] * scale, o[db][4 * qd + 1] * scale);
        w[1] = pack_bf16x2(o[db][4 * qd + 2] * scale, o[db][4 * qd + 3] * scale);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * qd + 4 * half) = w;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(int layer_type, const PrefillArgs& a, hipStream_t stream) {
  const int blocks = a.nqb * a.batch * kKvHeads;
  if (layer_type == kSliding)
    hipLaunchKernelGGL(prefill_kernel<kSliding>, dim3(blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_kernel<kFull>, dim3(blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

int prefill_block_rows() { return kBM; }

}  // namespace spark
