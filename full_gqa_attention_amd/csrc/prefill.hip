// Flash-attention prefill for the hybrid sliding/full GQA layer on gfx950.
//
// Two launches.  First a streaming pass applies RoPE to K once per position (into the
// caller's workspace) and writes the rotated keys and the values into the KV cache when
// one is given.  Then the attention kernel:
//
// One workgroup = 8 waves (two per SIMD) = one KV head g of one sequence and a block of
// 64 query positions; wave w computes query head 4g + w/2 for 32 of the positions.  Every
// K/V tile in LDS thus serves 4 query heads x 64 positions (GQA sharing).  Two waves per
// SIMD let one wave's MFMAs run while the other waits on LDS reads or transcendentals:
// measured on gfx950, each LDS read or exp interleaved into a single wave's MFMA stream
// costs that stream about 11-17 cycles.
//
// K/V tiles of 32 keys stream through a 3-stage LDS ring filled by direct global->LDS
// loads (no register staging), issued two tiles ahead:
//   * K tile (rotated dims from the workspace; on full layers the dims RoPE leaves alone
//     straight from K), chunk-major (16-byte chunk c of key j at slot 32c + j): the MFMA A
//     operand of S^T = K Q^T is one conflict-free 16-byte read.  Without a prefix the K and
//     V fragment reads are pinned ahead of their MFMAs (K four, V two).
//   * V tile, row-major with the chunk index XOR-swizzled by 4 * (row % 4): the A operand
//     of O^T += V^T P^T (V transposed) comes from two ds_read_b64_tr_b16 per MFMA, which
//     transpose 16-bit elements across each group of 16 lanes.
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16; each lane owns one
//     query row per block, so softmax statistics need no broadcast.  Q is rotated and
//     pre-scaled by log2(e)/16 once; the softmax runs in exp2 form in fp32; the running
//     maximum moves only when a score exceeds it by more than 8 (P <= 2^8), so the O
//     rescale is rare (full layers start the QK MFMAs from minus that maximum); row sums
//     come from v_dot2_f32_bf16 on the rounded P.
// Sliding layers visit only the 512-key band (Spark-X2.6-4B-Base hybrid attention
// explainer, eliteato.com/news/34565, section "滑动窗口 512"); full layers every earlier
// key (section "36 层混合注意力排布").  Epilogue: O / l * sigmoid(gate) (F16 vs Q4
// comparison page, hotelren.com/news/5475707, section 三), stored as bf16.
#include "spark_device.hpp"
#include "spark_launch.hpp"

#include <type_traits>

namespace spark {
namespace {

constexpr int kBM = 64;            // query positions per workgroup
constexpr int kBN = 32;            // keys per tile
constexpr int kWaves = 8;                          // waves per workgroup
constexpr int kRowBlocks = 8 / kWaves;            // 32-row blocks per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kTileBytes = kBN * kHeadDim * 2;   // 16 KB per K or V tile
constexpr float kRescaleThreshold = 8.0f;        // log2 units
constexpr int kKAhead = 4;                        // full layers: K fragments read ahead
// Instruction classes of __builtin_amdgcn_sched_group_barrier's mask.
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
constexpr float kQScale = 0.0625f * 1.4426950408889634f;   // 1/sqrt(256) * log2(e)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Direct global -> LDS load of 16 bytes per lane into the 1 KB block at lds_block (lane l
// fills bytes 16l .. 16l+15).  Written as inline asm so that the compiler does not track
// it: given the builtin, it cannot tell which ring stage a load fills and waits for every
// load in flight before the first LDS read of some steps.  Every wait for these loads is
// therefore explicit (wait_vmcnt before the barrier that publishes a tile).  The asm sets
// M0, which nothing else in these kernels uses.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 in the clobber list: see above
__device__ __forceinline__ void dma16(const void* src, void* lds_block) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_block;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds) : "memory", "m0");
}
// The same load from a wave-uniform 64-bit base (SGPRs) plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, void* lds_block) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_block;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// vmcnt <= N, other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Maximum of a lane's 16 scores, in code the compiler sees: the scores come straight from
// an MFMA, and the compiler inserts the wait states a VALU read of an MFMA result needs
// only before instructions it can see (an inline-asm v_max3_f32 chain here read the
// accumulator while the MFMA was still writing it, on the path that skips the masking).
__device__ __forceinline__ float max16(const f32x16& x) {
  float a = __builtin_fmaxf(__builtin_fmaxf(x[0], x[1]), x[2]);
  float b = __builtin_fmaxf(__builtin_fmaxf(x[3], x[4]), x[5]);
  float c = __builtin_fmaxf(__builtin_fmaxf(x[6], x[7]), x[8]);
  float d = __builtin_fmaxf(__builtin_fmaxf(x[9], x[10]), x[11]);
  float e = __builtin_fmaxf(__builtin_fmaxf(x[12], x[13]), x[14]);
  a = __builtin_fmaxf(__builtin_fmaxf(a, b), c);
  d = __builtin_fmaxf(__builtin_fmaxf(d, e), x[15]);
  return __builtin_fmaxf(a, d);
}

// The same with the NaN-propagating maximum, which gfx950 has as a three-input instruction
// that needs no canonicalising of its inputs (the IEEE maximum above gets a v_max_f32 x, x
// for the first two).
__device__ __forceinline__ float maximum16(const f32x16& x) {
  auto mx = [](float p, float q) { return __builtin_elementwise_maximum(p, q); };
  float a = mx(mx(x[0], x[1]), x[2]);
  float b = mx(mx(x[3], x[4]), x[5]);
  float c = mx(mx(x[6], x[7]), x[8]);
  float d = mx(mx(x[9], x[10]), x[11]);
  float e = mx(mx(x[12], x[13]), x[14]);
  a = mx(mx(a, b), c);
  d = mx(mx(d, e), x[15]);
  return mx(a, d);
}

// max(x, x of lane l ^ 32): v_permlane32_swap hands every lane the values of lanes l % 32
// and 32 + l % 32, i.e. its own and its partner's.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Workgroup barrier that only waits for this wave's LDS operations.  __syncthreads()
// would also wait for every outstanding global load, including the tile prefetched two
// steps ahead; the loads a step depends on are waited for explicitly instead.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

constexpr int kKLoads = 16 / kWaves;              // K-tile load instructions per wave
constexpr int kVLoads = 16 / kWaves;              // V-tile load instructions per wave

// The K tile layout of the short-sequence kernels (prefill_split_kernel): 16 blocks of
// 1 KB, block 8 ch + jb holding keys 4 jb .. 4 jb + 3, its 16-byte slot 16 r + t key
// 4 jb + r, chunk 16 ch + (t ^ (key & 15)).  One load instruction then fills a block from
// four contiguous 256-byte half rows, where the chunk-major layout of prefill_kernel reads
// 32 rows x 32 bytes per instruction, twice the cache lines (measured: the short kernels'
// tile loads took a sixth of their time; the long band of prefill_kernel hides them); the
// XOR spreads the 32 keys of one chunk over all banks for the MFMA operand reads.
// Byte offset, from the tile's first row, that lane reads for block n (rows past lim, the
// tile's last readable row, read that row instead).
__device__ __forceinline__ uint32_t kswz_src(int n, int lane, int lim) {
  const int r = lane >> 4, t = lane & 15;
  const int j = 4 * (n & 7) + r;
  const int c = 16 * (n >> 3) + (t ^ (j & 15));
  return (uint32_t)(min(j, lim) * 2048 + 16 * c);
}
// Byte offset in the tile of key r32's chunk c (c = 2 s + half: the MFMA A operand of step s).
__device__ __forceinline__ int kswz_read(int c, int r32) {
  return 8192 * (c >> 4) + 1024 * (r32 >> 2) + 256 * (r32 & 3) + 16 * ((c & 15) ^ (r32 & 15));
}

// Global rows of key position p (p < P + n) of (sequence b, KV head g): the cached prefix
// for p < P (slot p, or ring slot p mod 512 on a sliding layer), else the chunk's keys as
// rotated by the RoPE pass and its values.
template <int LT>
__device__ __forceinline__ size_t prefix_row(const PrefillArgs& a, int b, int g, int p) {
  const int slot = LT == kFull ? p : (p & (kWindow - 1));
  return (((size_t)b * a.cache_cap + slot) * kKvHeads + g) * kHeadDim;
}
// Token rows of sequence b: first row and length.  Uniform batches are b * S and S;
// varlen batches read cu_seqlens, clamped so that a malformed table can only shorten a
// sequence, never move an access outside the T rows or beyond the largest length.
struct SeqSpan {
  size_t row0;
  int len;
};
__device__ __forceinline__ SeqSpan seq_span(const PrefillArgs& a, int b) {
  if (a.cu_seqlens == nullptr) return {(size_t)b * a.seq_len, a.seq_len};
  const int T = a.total_tokens;
  const int lo = min(max(a.cu_seqlens[b], 0), T);
  const int hi = min(max(a.cu_seqlens[b + 1], lo), min(T, lo + a.seq_len));
  return {(size_t)lo, hi - lo};
}

__device__ __forceinline__ size_t chunk_row(const SeqSpan& sp, int g, int p, int P) {
  return ((sp.row0 + (p - P)) * kKvHeads + g) * kHeadDim;
}

// Load instruction i of tile (keys k0 .. k0+31, absolute positions) of (sequence b, KV
// head g).  Instruction n of K brings chunks 2n, 2n+1 of all 32 keys; instruction n of V
// rows 2n, 2n+1 with chunk positions swizzled by 4 * (row % 4).  Rows past the chunk's
// end load its last key (masked later).  PFX = false: no prefix (start_pos == 0), every
// key comes from the chunk.
//
// Without a prefix, the load takes a wave-uniform base (key k0, plus this wave's part) and
// a per-lane 32-bit offset that depends on the lane alone (and on the clamp of the last
// tile): measured 2-6% faster than 64-bit per-lane addresses, which also held registers
// the MFMA operand reads could use.  With a prefix, a tile wholly inside the prefix or
// wholly inside the chunk picks its source once and only a tile across start_pos selects
// per lane; there the scalar-base form was 2-5% slower (both forms in one kernel).
template <int LT, bool PFX, bool KSWZ = false>
__device__ __forceinline__ void issue_one(const PrefillArgs& a, int b, const SeqSpan& sp, int g, int k0,
                                          int wave, int lane, uint8_t* ks, uint8_t* vs, int i) {
  static_assert(!(KSWZ && PFX), "the swizzled K layout is for calls without a prefix");
  const int P = PFX ? a.start_pos : 0;
  const int kend = P + sp.len;
  const bool in_chunk = !PFX || k0 >= P, in_prefix = k0 + kBN <= P;   // wave-uniform
  if (!PFX) {
    static_assert(kKLoads == 2 && kVLoads == 2, "offsets below assume 8 waves");
    const int h = lane >> 5, l31 = lane & 31;
    const int lim = kend - 1 - k0;                  // last readable row of the tile
    const size_t base = (((sp.row0 + k0) * kKvHeads + g) * kHeadDim) * 2;   // bytes
    if (i < kKLoads) {
      if constexpr (KSWZ) {
        const int n = kKLoads * wave + i;
        dma16_s((const uint8_t*)a.k_rot + base, kswz_src(n, lane, lim), ks + n * 1024);
      } else {
        // Wave w loads dims 32w .. 32w + 31 of the tile's keys: rotated ones from the
        // workspace, the rest (full layers: dims >= 64, which RoPE leaves as they are)
        // straight from K, so that the RoPE pass writes only the rotated dims.
        constexpr int kRot = LayerTraits<LT>::kRot;
        const bool rotated = kRot == kHeadDim || wave < kRot / 32;   // wave-uniform
        const uint8_t* src = (const uint8_t*)(rotated ? a.k_rot : a.k) + base + 64 * wave;
        dma16_s(src, (uint32_t)(min(l31, lim) * 2048 + 16 * h + 32 * i), ks + (kKLoads * wave + i) * 1024);
      }
    } else {
      const int j = i - kKLoads;
      const uint8_t* src = (const uint8_t*)a.v + base;
      const int r = 2 * j + h;                       // row within this wave's four
      dma16_s(src, (uint32_t)(min(4 * wave + r, lim) * 2048 + 16 * (l31 ^ (4 * r))), vs + (kVLoads * wave + j) * 1024);
    }
    return;
  }
  if (i < kKLoads) {
    const int pk = min(k0 + (lane & 31), kend - 1);
    const int n = kKLoads * wave + i;
    const int off = 8 * (2 * n + (lane >> 5));
    const bool from_cache = !in_chunk && (in_prefix || pk < P);
    const uint16_t* base = from_cache ? a.cache_k : a.k_rot;
    const size_t row = from_cache ? prefix_row<LT>(a, b, g, pk) : chunk_row(sp, g, pk, P);
    dma16(base + (row + off), ks + n * 1024);
  } else {
    const int n = kVLoads * wave + (i - kKLoads);
    const int r = 2 * n + (lane >> 5);
    const int off = 8 * ((lane & 31) ^ (4 * (r & 3)));
    const int p = min(k0 + r, kend - 1);
    const bool from_cache = !in_chunk && (in_prefix || p < P);
    const uint16_t* base = from_cache ? a.cache_v : a.v;
    const size_t row = from_cache ? prefix_row<LT>(a, b, g, p) : chunk_row(sp, g, p, P);
    dma16(base + (row + off), vs + n * 1024);
  }
}
template <int LT, bool PFX>
__device__ __forceinline__ void issue_tile(const PrefillArgs& a, int b, const SeqSpan& sp, int g, int k0,
                                           int wave, int lane, uint8_t* ks, uint8_t* vs) {
#pragma unroll
  for (int i = 0; i < kKLoads + kVLoads; ++i) issue_one<LT, PFX>(a, b, sp, g, k0, wave, lane, ks, vs, i);
}

// RoPE of the chunk's K, once per position p = P + t: k_rot = R_p(k) (rotate-half form:
// pair (m, m + r/2) is rotated by angle p * theta^(-2m/r) for m < r/2; dims >= r are
// copied), and, when a cache is given, the rotated keys and the values into their cache
// slots (full layer: slot p; sliding layer: slot p mod 512 for the last 512 positions,
// here only when there is no cached prefix -- otherwise those slots still hold keys the
// chunk's first queries read, and the ring is written after the attention) --
// Spark-X2.6-4B-Base hybrid attention explainer, eliteato.com/news/34565, sections
// "全局注意力 5M 基频 RoPE" and "滑动窗口 512".  One thread per 16-byte chunk of a K row: a
// rotary chunk also reads its partner chunk (dims + or - r/2) and computes its own half of
// the pair.  Full layers without a prefix read dims >= r straight from K in the attention,
// so the pass writes only the rotated chunks of k_rot; with ROT_ONLY (no cache either) it
// has one thread per rotated chunk only.
template <int LT, bool ROT_ONLY = false>
__global__ __launch_bounds__(256) void prefill_rope_kernel(PrefillArgs a) {
  using T = LayerTraits<LT>;
  static_assert(!ROT_ONLY || LT == kFull, "sliding layers rotate every dim");
  constexpr int kHalf = T::kRot / 16;                // chunks in the first half of the rotary span
  constexpr int kRowChunks = ROT_ONLY ? 2 * kHalf : 32;   // threads per K row
  __shared__ double s_inv[T::kRot / 2];
  if (threadIdx.x < T::kRot / 2) s_inv[threadIdx.x] = rope_inv_rev(threadIdx.x, T::kRot, log2(T::kTheta));
  __syncthreads();
  // The attention launch that follows claims its work from this counter (varlen).
  if (a.sched != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.sched = 0;
  // Grid: x = tokens of a sequence (two per workgroup), y = sequence.
  const int b = blockIdx.y;
  const SeqSpan sp = seq_span(a, b);
  const int idx = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const int t = idx / (kKvHeads * kRowChunks);       // token within the sequence
  const int g = (idx / kRowChunks) % kKvHeads;
  const int c = idx % kRowChunks;
  if (t >= sp.len) return;
  const size_t row = (sp.row0 + t) * kKvHeads + g;
  const int p = a.start_pos + t;
  const uint16_t* krow = a.k + row * kHeadDim;
  const u32x4 x = ld_global16(krow + 8 * c);
  u32x4 y = x;
  if (c < 2 * kHalf) {
    const bool first = c < kHalf;
    const u32x4 xp = ld_global16(krow + 8 * (first ? c + kHalf : c - kHalf));
    const int m0 = 8 * (first ? c : c - kHalf);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float c0, s0, c1, s1;
      rope_cos_sin((double)p, s_inv[m0 + 2 * w], c0, s0);
      rope_cos_sin((double)p, s_inv[m0 + 2 * w + 1], c1, s1);
      const float a0 = bf16_lo(x[w]), a1 = bf16_hi(x[w]);
      const float b0 = bf16_lo(xp[w]), b1 = bf16_hi(xp[w]);
      y[w] = first ? pack_bf16x2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1)
                   : pack_bf16x2(a0 * c0 + b0 * s0, a1 * c1 + b1 * s1);
    }
  }
  if (LT == kSliding || a.start_pos > 0 || c < 2 * kHalf) st_global16(a.k_rot + row * kHeadDim + 8 * c, y);
  if (a.cache_k != nullptr && (LT == kFull || (a.start_pos == 0 && t >= sp.len - kWindow))) {
    const int slot = LT == kFull ? p : (p & (kWindow - 1));
    const size_t dst = (((size_t)b * a.cache_cap + slot) * kKvHeads + g) * kHeadDim + 8 * c;
    st_global16(a.cache_k + dst, y);
    st_global16(a.cache_v + dst, ld_global16(a.v + row * kHeadDim + 8 * c));
  }
}

// Sliding layer after a chunk that continues a prefix: the chunk's last 512 positions
// into their ring slots (p mod 512), once the attention has read the prefix's keys there.
// One thread per 16-byte chunk of those rows' K and V.
__global__ __launch_bounds__(256) void prefill_ring_kernel(PrefillArgs a) {
  const int n = a.seq_len;
  const int t0 = n > kWindow ? n - kWindow : 0;       // first chunk row kept
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t per_seq = (size_t)(n - t0) * kKvHeads * 32;
  if (idx >= (size_t)a.batch * per_seq) return;
  const int b = (int)(idx / per_seq);
  const size_t r = idx % per_seq;
  const int t = t0 + (int)(r / (kKvHeads * 32));
  const int g = (int)((r / 32) % kKvHeads);
  const int c = (int)(r % 32);
  const int slot = (a.start_pos + t) & (kWindow - 1);
  const size_t src = (((size_t)b * n + t) * kKvHeads + g) * kHeadDim + 8 * c;
  const size_t dst = (((size_t)b * a.cache_cap + slot) * kKvHeads + g) * kHeadDim + 8 * c;
  st_global16(a.cache_k + dst, ld_global16(a.k_rot + src));
  st_global16(a.cache_v + dst, ld_global16(a.v + src));
}

// Workgroup -> (sequence, KV head, query block).  Workgroups are dealt round-robin to the
// 8 XCDs; when the (sequence, KV head) units divide evenly over them, each XCD gets the
// query blocks of one unit (so its L2 serves one K/V stream), alternating blocks between
// the XCDs sharing a unit.  Full layers run the longest (latest) blocks first.
template <int LT>
__device__ __forceinline__ void block_coords(int id, int batch, int nqb, int& b, int& g, int& qb) {
  const int units = batch * kKvHeads;
  int unit, qidx;
  if (8 % units == 0 && nqb % (8 / units) == 0) {
    const int r = 8 / units;
    const int x = id & 7, j = id >> 3;
    unit = x / r;
    // Full layers deal each run of r blocks in alternating directions (snake order), so
    // that the XCDs sharing a unit get equal work (blocks of a full layer differ in size).
    qidx = r * j + (LT == kFull && (j & 1) ? r - 1 - x % r : x % r);
  } else {
    unit = id % units;
    qidx = id / units;
  }
  b = unit / kKvHeads;
  g = unit % kKvHeads;
  qb = (LT == kFull) ? (nqb - 1 - qidx) : qidx;
}

// Rotate (RoPE at position p) and scale the Q row slice this lane holds, into MFMA
// B-operand fragments: fragment s holds dims 16s + 8*half + j.
template <int LT>
__device__ __forceinline__ void load_q(const PrefillArgs& a, const SeqSpan& sp, int hq, int row, int pos0,
                                       int half, const double* inv, bf16x8* qf) {
  using T = LayerTraits<LT>;
  u32x4 raw[16];
  if (row < sp.len) {
    const uint16_t* qrow = a.q + ((sp.row0 + row) * kQHeads + hq) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 16; ++s) raw[s] = ld_global16(qrow + 16 * s + 8 * half);
  } else {
#pragma unroll
    for (int s = 0; s < 16; ++s) raw[s] = u32x4{0, 0, 0, 0};
  }
  const double p = (double)(pos0 + row);   // the row's position
  constexpr int kPairChunks = T::kRot / 32;         // fragment s pairs with s + kPairChunks
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s < kPairChunks) {
      u32x4 y1, y2;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float c0, s0, c1, s1;
        const int m = 16 * s + 8 * half + 2 * w;
        rope_cos_sin(p, inv[m], c0, s0);
        rope_cos_sin(p, inv[m + 1], c1, s1);
        const float a0 = bf16_lo(raw[s][w]), a1 = bf16_hi(raw[s][w]);
        const float b0 = bf16_lo(raw[s + kPairChunks][w]), b1 = bf16_hi(raw[s + kPairChunks][w]);
        y1[w] = pack_bf16x2((a0 * c0 - b0 * s0) * kQScale, (a1 * c1 - b1 * s1) * kQScale);
        y2[w] = pack_bf16x2((b0 * c0 + a0 * s0) * kQScale, (b1 * c1 + a1 * s1) * kQScale);
      }
      qf[s] = as_bf16x8(y1);
      qf[s + kPairChunks] = as_bf16x8(y2);
    } else if (s >= 2 * kPairChunks) {
      u32x4 y;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        y[w] = pack_bf16x2(bf16_lo(raw[s][w]) * kQScale, bf16_hi(raw[s][w]) * kQScale);
      qf[s] = as_bf16x8(y);
    }
  }
}

// Rotate and scale one rotary pair of Q fragments, the arithmetic of load_q's pair step:
// x1 holds dims m0 .. m0 + 7, x2 the dims r/2 further on, at position p.
__device__ __forceinline__ void rotate_q_pair(const u32x4& x1, const u32x4& x2, double p, const double* inv,
                                              int m0, bf16x8& q1, bf16x8& q2) {
  u32x4 y1, y2;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float c0, s0, c1, s1;
    const int m = m0 + 2 * w;
    rope_cos_sin(p, inv[m], c0, s0);
    rope_cos_sin(p, inv[m + 1], c1, s1);
    const float a0 = bf16_lo(x1[w]), a1 = bf16_hi(x1[w]);
    const float b0 = bf16_lo(x2[w]), b1 = bf16_hi(x2[w]);
    y1[w] = pack_bf16x2((a0 * c0 - b0 * s0) * kQScale, (a1 * c1 - b1 * s1) * kQScale);
    y2[w] = pack_bf16x2((b0 * c0 + a0 * s0) * kQScale, (b1 * c1 + a1 * s1) * kQScale);
  }
  q1 = as_bf16x8(y1);
  q2 = as_bf16x8(y2);
}

template <int LT, bool PFX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void prefill_kernel(PrefillArgs a) {
  using T = LayerTraits<LT>;
  // The ring: [stage][K, V]; the loop below is unrolled by the stage count.
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[3][2][kTileBytes];
  uint8_t* const s_k0 = &s_ring[0][0][0];
  uint8_t* const s_v0 = &s_ring[0][1][0];
  uint8_t* const s_k1 = &s_ring[1][0][0];
  uint8_t* const s_v1 = &s_ring[1][1][0];
  uint8_t* const s_k2 = &s_ring[2][0][0];
  uint8_t* const s_v2 = &s_ring[2][1][0];
  __shared__ double s_inv[T::kRot / 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: wave-uniform branches
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int P = PFX ? a.start_pos : 0;      // position of chunk row 0

  int b, g, qb;
  if (PFX || a.sched == nullptr) {        // prefix calls are never varlen
    block_coords<LT>(blockIdx.x, a.batch, a.nqb, b, g, qb);
  } else {
    // Variable lengths: workgroups go to the XCDs round-robin by id, so a fixed mapping would
    // give some XCDs more work than others.  Instead each workgroup claims the next item of
    // one queue, in the order the fixed mapping would use (latest blocks first on full
    // layers), skipping blocks past the end of their sequence; the grid has one workgroup
    // per item, so every item is claimed once.
    __shared__ int s_item;
    if (tid == 0) {
      const int units = a.batch * kKvHeads, items = units * a.nqb;
      int item = -1;
      for (;;) {
        const int k = atomicAdd(a.sched, 1);
        if (k >= items) break;
        const int qx = k / units, qbk = (LT == kFull) ? (a.nqb - 1 - qx) : qx;
        if (qbk * kBM < seq_span(a, (k % units) / kKvHeads).len) { item = k; break; }
      }
      s_item = item;
    }
    __syncthreads();
    const int item = s_item;
    if (item < 0) return;                   // the queue ran out (whole workgroup)
    const int units = a.batch * kKvHeads;
    b = (item % units) / kKvHeads;
    g = item % kKvHeads;
    const int qx = item / units;
    qb = (LT == kFull) ? (a.nqb - 1 - qx) : qx;
  }
  const int q0 = qb * kBM;
  const SeqSpan sp = seq_span(a, b);
  const int S = sp.len;                     // chunk rows of this sequence
  if (q0 >= S) return;                      // a shorter sequence (whole workgroup)
  const int hq = g * kGroup + (kRowBlocks == 2 ? wave : wave >> 1);
  const int rb0 = kRowBlocks == 2 ? 0 : (wave & 1);      // first 32-row block of this wave

  const int hi_key = P + min(q0 + kBM - 1, S - 1);                 // absolute key positions
  const int lo_key = T::kWindowed ? max(0, P + q0 - (kWindow - 1)) : 0;
  const int kt_lo = lo_key / kBN;
  const int kt_hi = hi_key / kBN;

  // Start streaming the first two tiles before anything else.
  issue_tile<LT, PFX>(a, b, sp, g, kt_lo * kBN, wave, lane, s_k0, s_v0);
  if (kt_lo + 1 <= kt_hi) issue_tile<LT, PFX>(a, b, sp, g, (kt_lo + 1) * kBN, wave, lane, s_k1, s_v1);

  if (tid < T::kRot / 2) s_inv[tid] = rope_inv_rev(tid, T::kRot, log2(T::kTheta));
  barrier_lds();

  // Q fragments of both 32-row blocks: lane holds row r32 of each.
  bf16x8 qf[kRowBlocks][16];
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) load_q<LT>(a, sp, hq, q0 + 32 * (rb0 + rb) + r32, P, half, s_inv, qf[rb]);

  // First tiles: wait for this lane's loads (of both), publish.
  wait_vmcnt<0>();
  barrier_lds();

  // Running maximum c of each row.  Full layers without a prefix start their QK MFMAs from
  // -c, so that the common step exponentiates the MFMA results directly (the subtractions
  // leave the path from the QK MFMAs to the PV MFMAs), and rescale when a score beats c by
  // more than kRescaleThreshold.  The other forms keep c = -1e30 until their first key and
  // subtract c from the scores: the same change measured 2.7% slower on sliding layers, and
  // the prefix form, whose per-tile source choice needs registers of its own, would spill.
  constexpr bool kRel = !T::kWindowed && !PFX;
  // Forms without a prefix read K and V fragments ahead in a pinned order (below).
  constexpr bool kPin = !PFX;
  f32x16 o[kRowBlocks][8];
  float c_run[kRowBlocks], l_part[kRowBlocks];
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[rb][i] = f32x16{0};
    c_run[rb] = kRel ? 0.0f : -1e30f;
    l_part[rb] = 0.0f;
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Per-lane byte offsets of the transposed V reads: lane l = 16 grp + 4 vr + vc provides
  // row 4*(grp/2) + vr (+8 for the second read of a fragment) and dims
  // 32 db + 16 (grp & 1) + 4 vc of the tile; chunk positions are swizzled by 4 * vr.
  const int grp = lane >> 4, vr = (lane >> 2) & 3, vc = lane & 3;
  const int v_lane_off = (4 * (grp >> 1) + vr) * 512 + 16 * (2 * (grp & 1) + (vc >> 1)) + 8 * (vc & 1);

  // One pipeline step on tile kt held in stage ST: start loading tile kt+2 into stage
  // ST+2, compute tile kt, then finish tile kt+1 (stage ST+1) and publish it.
  auto step = [&](auto stage_tag, int kt) {
    constexpr int ST = decltype(stage_tag)::value;
    uint8_t* const ks = ST == 0 ? s_k0 : ST == 1 ? s_k1 : s_k2;
    uint8_t* const vs = ST == 0 ? s_v0 : ST == 1 ? s_v1 : s_v2;
    uint8_t* const ks1 = ST == 0 ? s_k1 : ST == 1 ? s_k2 : s_k0;
    uint8_t* const vs1 = ST == 0 ? s_v1 : ST == 1 ? s_v2 : s_v0;
    uint8_t* const ks2 = ST == 0 ? s_k2 : ST == 1 ? s_k0 : s_k1;
    uint8_t* const vs2 = ST == 0 ? s_v2 : ST == 1 ? s_v0 : s_v1;
    const int k0 = kt * kBN;
    const bool two_ahead = kt + 2 <= kt_hi;
    // Steps 1 and 2 issue tile kt+2 one load every four QK MFMAs (issuing a tile's loads
    // back to back stalls every wave of the CU on the texture unit's queue); without a
    // prefix unconditionally: past the last tile they reload it into the idle stage, unused.
    // A conditional load among the MFMAs ends a scheduling region every four MFMAs (1.2-1.9%
    // slower on full layers; on sliding layers it measured 0-1% faster until the fragment
    // reads were pinned, which needs one region).  Step 0 issues its prefetch after its
    // MFMAs, which measured slightly faster than interleaving there.

    // Which row blocks see any key of this tile (wave-uniform).
    bool any[kRowBlocks], edge[kRowBlocks], any_rb = false;
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
      const int r0 = P + q0 + 32 * (rb0 + rb);   // position of the block's first row
      any[rb] = (k0 <= r0 + 31) && (!T::kWindowed || k0 + kBN - 1 >= r0 - (kWindow - 1));
      edge[rb] = (k0 + kBN - 1 > r0) || (T::kWindowed && k0 < r0 + 31 - (kWindow - 1));
      any_rb = any_rb || any[rb];
    }
    if (any_rb) {
      f32x16 sacc[kRowBlocks];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) sacc[rb] = kRel ? -c_run[rb] : 0.0f;
      if constexpr (kPin) {
        // K fragments read kKAhead MFMAs ahead, in an order pinned by scheduling groups: left
        // to itself the scheduler sinks each read to just before its MFMA, two at a time.
        // The tile loads go in unconditionally (sliding layers too): a branch here would end
        // the scheduling region every four MFMAs; past the last tile they reload it into
        // the idle stage, unused, and are waited for before the epilogue.
        auto kfrag = [&](int s) {
          return as_bf16x8(*reinterpret_cast<const u32x4*>(ks + (32 * (2 * s + half) + r32) * 16));
        };
        bf16x8 kb[kKAhead];
#pragma unroll
        for (int j = 0; j < kKAhead; ++j) kb[j] = kfrag(j);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const bf16x8 ka = kb[s % kKAhead];
          if (s + kKAhead < 16) kb[s % kKAhead] = kfrag(s + kKAhead);
#pragma unroll
          for (int rb = 0; rb < kRowBlocks; ++rb) sacc[rb] = mfma_32x32x16(ka, qf[rb][s], sacc[rb]);
          if (ST != 0 && (s & 3) == 1)
            issue_one<LT, PFX>(a, b, sp, g, min(kt + 2, kt_hi) * kBN, wave, lane, ks2, vs2, s >> 2);
        }
#pragma unroll
        for (int j = 0; j < kKAhead; ++j) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          if (s + kKAhead < 16) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + (32 * (2 * s + half) + r32) * 16));
#pragma unroll
          for (int rb = 0; rb < kRowBlocks; ++rb) sacc[rb] = mfma_32x32x16(ka, qf[rb][s], sacc[rb]);
          if (ST != 0 && (LT == kFull || two_ahead) && (s & 3) == 1)
            issue_one<LT, PFX>(a, b, sp, g, LT == kFull ? min(kt + 2, kt_hi) * kBN : k0 + 2 * kBN, wave, lane, ks2,
                               vs2, s >> 2);
        }
      }
      bf16x8 pf[kRowBlocks][2];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) {
        const int row = q0 + 32 * (rb0 + rb) + r32;
        const int rpos = P + row;                 // this lane's query position
        if (edge[rb]) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k0 + 8 * (v >> 2) + 4 * half + (v & 3);
            const bool vis = key <= rpos && (!T::kWindowed || key > rpos - kWindow);
            sacc[rb][v] = vis ? sacc[rb][v] : -INFINITY;
          }
        }
        float l_pair[kRowBlocks][2] = {};   // two independent row-sum chains
        if constexpr (!kRel) {
          const float mt = max_halves(max16(sacc[rb]));
          if (__any(mt > c_run[rb] + kRescaleThreshold)) {
            const float m_new = fmaxf(c_run[rb], mt);
            const float alpha = __builtin_amdgcn_exp2f(c_run[rb] - m_new);
            l_part[rb] *= alpha;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[rb][i] *= alpha;
            c_run[rb] = m_new;
          }
        } else if (const float mt = maximum16(sacc[rb]); kt == kt_lo || __any(mt > kRescaleThreshold)) {
          // The decision needs only this lane's half of the row (its partner lane is in the
          // same wave); the row's maximum is formed when the wave rescales.  The first tile
          // holds key 0, which every row sees: it sets the maximum (c = 0 before it).
          const float m_old = kt == kt_lo ? -1e30f : c_run[rb];
          const float m_new = fmaxf(m_old, max_halves(mt) + c_run[rb]);
          const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);
          l_part[rb] *= alpha;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[rb][i] *= alpha;
          const float d = m_new - c_run[rb];      // scores relative to the new maximum
#pragma unroll
          for (int v = 0; v < 16; ++v) sacc[rb][v] -= d;
          c_run[rb] = m_new;
        }
        const float off = kRel ? 0.0f : c_run[rb];   // x - 0.0f folds to x
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          u32x4 pk;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            // The pair is built as bf16x2 and then stored into pk, not read back out of
            // pk: hipcc (ROCm 7.2) folds a bf16x2 bit-cast of pk[w] to pk[0] for every w.
            const bf16x2 p2 = {(__bf16)__builtin_amdgcn_exp2f(sacc[rb][8 * tt + 2 * w] - off),
                               (__bf16)__builtin_amdgcn_exp2f(sacc[rb][8 * tt + 2 * w + 1] - off)};
            l_pair[rb][w & 1] = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l_pair[rb][w & 1], false);
            pk[w] = __builtin_bit_cast(uint32_t, p2);
          }
          pf[rb][tt] = as_bf16x8(pk);
        }
        l_part[rb] += l_pair[rb][0] + l_pair[rb][1];
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int off = v_lane_off + 16 * tt * 512 + 64 * (db ^ vr);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + off));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + off + 8 * 512));
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int rb = 0; rb < kRowBlocks; ++rb) o[rb][db] = mfma_32x32x16(va, pf[rb][tt], o[rb][db]);
        }
      }
      if constexpr (kPin) {
        // V fragments (two transposing reads each) read two MFMAs ahead, pinned likewise.
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
          if (i + 2 < 16) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
        }
      }
    }
    // Step 0 issues its prefetch after the MFMAs; the others issue it one instruction every
    // four QK MFMAs, or here when this wave's rows see no key of the tile.
    if (two_ahead && (ST == 0 || !any_rb)) issue_tile<LT, PFX>(a, b, sp, g, k0 + 2 * kBN, wave, lane, ks2, vs2);
    if (kt + 1 <= kt_hi) {
      // This lane's loads of tile kt+1 were issued one step ago; tile kt+2's may still be
      // in flight.  Every lane waits for its own loads before the barrier: other waves
      // read them.
      if (two_ahead) wait_vmcnt<kKLoads + kVLoads>(); else wait_vmcnt<0>();
    }
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);   // keep the unrolled steps apart (register pressure)
  };

  for (int kt = kt_lo;;) {
    step(std::integral_constant<int, 0>{}, kt);
    if (++kt > kt_hi) break;
    step(std::integral_constant<int, 1>{}, kt);
    if (++kt > kt_hi) break;
    step(std::integral_constant<int, 2>{}, kt);
    if (++kt > kt_hi) break;
  }
  // The last step's reloads may still be in flight: done before the epilogue (which stages
  // through the ring on sliding layers) and before the workgroup ends.
  if constexpr (!T::kWindowed || kPin) wait_vmcnt<0>();

  // ---- epilogue: O / l * sigmoid(gate), bf16
  if constexpr (T::kWindowed) {
    static_assert(kRowBlocks == 1, "one 32-row block per wave");
    // Sliding layers: each wave stages its 32 rows through its own 8.25 KB of the (now
    // idle) ring, half the dims at a time, so that the stores write whole 256-byte row
    // segments: a workgroup's short band leaves no time for scattered 16-byte pieces to
    // merge into whole lines in L2 (written bytes dropped from 1.55x to 1x the output).
    // Row pitch 264 bytes keeps the 8-byte writes of the 32 rows on distinct banks.  The
    // stores are non-temporal: measured 3% faster at S = 32768 (on full layers, whose
    // epilogue is a small share of the call, they were 2% slower at S = 8192 and are not used).
    const int row = q0 + 32 * rb0 + r32;
    const float l_tot = l_part[0] + __shfl_xor(l_part[0], 32);
    const float gl = row < S ? bf16_to_f32(a.gate[(sp.row0 + row) * kQHeads + hq]) : 0.0f;
    const float scale = sigmoidf_fast(gl) / l_tot;
    constexpr int kPitch = 264;
    uint8_t* const stage = &s_ring[0][0][0] + wave * (32 * kPitch);   // 8 x 8448 B of 96 KB
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) {
        const int db = 4 * r + d4;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          u32x2 w;
          w[0] = pack_bf16x2(o[0][db][4 * qd] * scale, o[0][db][4 * qd + 1] * scale);
          w[1] = pack_bf16x2(o[0][db][4 * qd + 2] * scale, o[0][db][4 * qd + 3] * scale);
          *reinterpret_cast<u32x2*>(stage + r32 * kPitch + (32 * d4 + 8 * qd + 4 * half) * 2) = w;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));   // lgkmcnt(0): own writes
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rr = 4 * i + (lane >> 4), c = lane & 15;   // row rr, 16-byte piece c
        const u32x4 x = *reinterpret_cast<const u32x4*>(stage + rr * kPitch + c * 16);
        const int grow = q0 + 32 * rb0 + rr;
        if (grow < S)
          __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(a.out + ((sp.row0 + grow) * kQHeads + hq) * kHeadDim +
                                                               128 * r + 8 * c));
      }
      __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));   // reads done before reuse
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    // Full layers: lanes l and l + 32 hold the two 4-dim halves of each 8-dim run of row
    // l % 32; one v_permlane32_swap per dword gives lane l the whole even run and lane l + 32
    // the whole odd run of each pair, so every store writes 16 contiguous bytes (half as
    // many row-scattered store instructions as 8-byte pieces would need).
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
      const int row = q0 + 32 * (rb0 + rb) + r32;
      const float l_tot = l_part[rb] + __shfl_xor(l_part[rb], 32);
      const bool ok = row < S;                 // the same for lanes l and l + 32
      const float gl = ok ? bf16_to_f32(a.gate[(sp.row0 + row) * kQHeads + hq]) : 0.0f;
      const float scale = sigmoidf_fast(gl) / l_tot;
      uint16_t* orow = a.out + ((sp.row0 + (ok ? row : 0)) * kQHeads + hq) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // Elements 8m .. 8m + 3 are run qd = 2m, 8m + 4 .. 8m + 7 run 2m + 1.
          const f32x16& ov = o[rb][db];
          const uint32_t e0 = pack_bf16x2(ov[8 * m] * scale, ov[8 * m + 1] * scale);
          const uint32_t e1 = pack_bf16x2(ov[8 * m + 2] * scale, ov[8 * m + 3] * scale);
          const uint32_t d0 = pack_bf16x2(ov[8 * m + 4] * scale, ov[8 * m + 5] * scale);
          const uint32_t d1 = pack_bf16x2(ov[8 * m + 6] * scale, ov[8 * m + 7] * scale);
          // Lanes < 32 keep e and receive e of lane + 32; lanes >= 32 receive d of lane - 32
          // and keep d: each then holds dims 8 (2m + half) .. + 7 in order.
          const auto s0 = __builtin_amdgcn_permlane32_swap(e0, d0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(e1, d1, false, false);
          if (ok)
            *reinterpret_cast<u32x4*>(orow + 32 * db + 8 * (2 * m + half)) = u32x4{s0[0], s1[0], s0[1], s1[1]};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Sliding layers of short sequences, whose 64-row query blocks cannot fill the chip (at
// S = 1024: 16 blocks x 4 KV heads = 64 workgroups for 256 CUs, each walking up to 18
// dependent tiles).  Here a workgroup takes 32 query positions of one (sequence, KV head)
// and its waves are HPW query heads times the two halves of the key band: wave w computes
// head w % HPW of its share over the tiles of half w / HPW, so the dependent chain is at
// most 9 tiles.  HPW = 4 (8 waves, the whole group) gives twice as many workgroups as the
// 64-row kernel; HPW = 2 (4 waves, one per SIMD, each K/V tile loaded by two workgroups)
// four times as many, for grids that would otherwise leave CUs idle.  Each half streams
// its tiles through its own two-stage ring (prefetch one tile ahead; the ring's 128 KB
// allow one workgroup per CU); at the end the second half's (max, sum, O) go through LDS
// to the wave of the same head in the first half, which merges them with log-sum-exp
// weights and runs the usual gated epilogue.

constexpr int kSplitRows = 32;                       // query positions per workgroup
// Whether the workgroups take 2 query heads each (twice as many workgroups of 4 waves)
// rather than 4, given the 4-head grid: both run one workgroup per CU, a round of 2-head
// workgroups in about 0.6 of the time of a round of 4-head ones (measured at S = 512 ..
// 4032), so the 2-head form wins while it needs at most 1.5 times as many rounds.
constexpr int kCUs = 256;
__host__ inline bool split_two_heads(int wgs4) {
  const int rounds4 = (wgs4 + kCUs - 1) / kCUs, rounds2 = (2 * wgs4 + kCUs - 1) / kCUs;
  return 2 * rounds2 <= 3 * rounds4;
}
// Load instructions per wave and tile when HPW waves share a half's tiles (a tile is 32
// instructions of 1 KB).
template <int HPW>
constexpr int split_loads() { return 32 / HPW; }

// One tile (keys k0 .. k0 + 31, K in ks, V in vs) for the 32 rows starting at position r0,
// lane row r32: S^T = K Q^T, band mask on edge tiles, lazy online softmax, O^T += V^T P^T.
// The same arithmetic as a step of prefill_kernel.  load(j), j = 0 .. NL - 1, issues the
// j-th load instruction of the next tile: spread evenly over the 16 QK MFMAs (back to
// back, a tile's loads stall every wave of the CU on the texture unit's queue), or all at
// once when no row of the block sees this tile.
template <int NL, class Load>
__device__ __forceinline__ void split_tile(const uint8_t* ks, const uint8_t* vs, int k0, int r0, int lane,
                                           const bf16x8 (&qf)[16], f32x16 (&o)[8], float& m_run, float& l_part,
                                           int v_lane_off, Load load) {
  const int half = lane >> 5, r32 = lane & 31;
  const int vr = (lane >> 2) & 3;
  const bool any = (k0 <= r0 + 31) && (k0 + kBN - 1 >= r0 - (kWindow - 1));
  if (!any) {                                        // wave-uniform: no row of the block sees the tile
#pragma unroll
    for (int j = 0; j < NL; ++j) load(j);
    return;
  }
  const bool edge = (k0 + kBN - 1 > r0) || (k0 < r0 + 31 - (kWindow - 1));
  f32x16 sacc = f32x16{0};
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + kswz_read(2 * s + half, r32)));
    sacc = mfma_32x32x16(ka, qf[s], sacc);
    constexpr int kEvery = 16 / NL;
    if (s % kEvery == kEvery - 1) load(s / kEvery);
  }
  const int rpos = r0 + r32;
  if (edge) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = k0 + 8 * (v >> 2) + 4 * half + (v & 3);
      sacc[v] = (key <= rpos && key > rpos - kWindow) ? sacc[v] : -INFINITY;
    }
  }
  const float mt = max_halves(max16(sacc));
  if (__any(mt > m_run + kRescaleThreshold)) {
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_part *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
    m_run = m_new;
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float l_pair[2] = {0.0f, 0.0f};
  bf16x8 pf[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    u32x4 pk;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 p2 = {(__bf16)__builtin_amdgcn_exp2f(sacc[8 * tt + 2 * w] - m_run),
                         (__bf16)__builtin_amdgcn_exp2f(sacc[8 * tt + 2 * w + 1] - m_run)};
      l_pair[w & 1] = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l_pair[w & 1], false);
      pk[w] = __builtin_bit_cast(uint32_t, p2);
    }
    pf[tt] = as_bf16x8(pk);
  }
  l_part += l_pair[0] + l_pair[1];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int off = v_lane_off + 16 * tt * 512 + 64 * (db ^ vr);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + off));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + off + 8 * 512));
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[db] = mfma_32x32x16(va, pf[tt], o[db]);
    }
  }
}

// MFMAs of the one-wave-per-SIMD tile step, in asm so that the register classes are ours:
// the Q fragments (the B operand of S^T = K Q^T, read-only in the loop) in AGPRs, the
// accumulators S^T and O^T, the K, V and P fragments in VGPRs -- which leaves VGPRs for
// fragments read several MFMAs ahead.  Left to itself the compiler puts the accumulators
// in AGPRs, and moves blocks of O between the two register files around every MFMA
// sequence.
//
// The compiler adds no wait states around asm, so the asm carries them: 11 between an
// 8-pass 32x32x16 MFMA (gfx950) and a VALU read of its result (S^T), a few between a VALU
// write and an MFMA read (the P fragments).  Back-to-back accumulation into the same
// registers needs none.
template <bool FIRST, bool LAST>
__device__ __forceinline__ void mfma_qk_asm(f32x16& acc, bf16x8 k, const bf16x8& q) {
  if constexpr (FIRST)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "a"(q));
  else if constexpr (LAST)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 4" : "+v"(acc) : "v"(k), "a"(q));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "a"(q));
}
template <bool AFTER_VALU>
__device__ __forceinline__ void mfma_pv_asm(f32x16& acc, bf16x8 v, bf16x8 p) {
  if constexpr (AFTER_VALU)
    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(v), "v"(p));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(v), "v"(p));
}
// The wait states between the last PV MFMA of the loop and the first VALU read of O after
// it, tied to O so that no read moves above them.
__device__ __forceinline__ void mfma_result_fence(f32x16 (&o)[8]) {
  asm volatile("s_nop 7\n\ts_nop 4"
               : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]), "+v"(o[4]), "+v"(o[5]), "+v"(o[6]), "+v"(o[7]));
}
// 16 fragments of 16 bytes, 1 KB apart in LDS from p, straight into AGPRs (complete when
// the asm ends), so that the Q fragments are born in the register file they stay in.
__device__ __forceinline__ void lds_read16_agpr(const void* p, bf16x8 (&q)[16]) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
  asm volatile("ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:1024\n\t"
               "ds_read_b128 %2, %16 offset:2048\n\tds_read_b128 %3, %16 offset:3072\n\t"
               "ds_read_b128 %4, %16 offset:4096\n\tds_read_b128 %5, %16 offset:5120\n\t"
               "ds_read_b128 %6, %16 offset:6144\n\tds_read_b128 %7, %16 offset:7168\n\t"
               "ds_read_b128 %8, %16 offset:8192\n\tds_read_b128 %9, %16 offset:9216\n\t"
               "ds_read_b128 %10, %16 offset:10240\n\tds_read_b128 %11, %16 offset:11264\n\t"
               "ds_read_b128 %12, %16 offset:12288\n\tds_read_b128 %13, %16 offset:13312\n\t"
               "ds_read_b128 %14, %16 offset:14336\n\tds_read_b128 %15, %16 offset:15360\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=a"(q[0]), "=a"(q[1]), "=a"(q[2]), "=a"(q[3]), "=a"(q[4]), "=a"(q[5]), "=a"(q[6]), "=a"(q[7]),
                 "=a"(q[8]), "=a"(q[9]), "=a"(q[10]), "=a"(q[11]), "=a"(q[12]), "=a"(q[13]), "=a"(q[14]),
                 "=a"(q[15])
               : "v"(a)
               : "memory");
}

// split_tile for workgroups of one wave per SIMD (HPW = 2), where no other wave hides a
// wave's own LDS latency: fragments are read several MFMAs ahead of their use (the
// register file of a lone wave holds them), so no MFMA waits on a read issued just
// before it.  The next tile's 16 loads go one after each QK MFMA, unconditionally (the
// caller gives a harmless tile when there is none): a branch among the MFMAs would end the
// scheduling region, and with it the early reads.
template <class Load>
__device__ __forceinline__ void split_tile_deep(const uint8_t* ks, const uint8_t* vs, int k0, int r0, int lane,
                                                const bf16x8 (&qf)[16], f32x16 (&o)[8], float& m_run,
                                                float& l_part, int v_lane_off, Load load) {
  const int half = lane >> 5, r32 = lane & 31;
  const int vr = (lane >> 2) & 3;
  const bool any = (k0 <= r0 + 31) && (k0 + kBN - 1 >= r0 - (kWindow - 1));
  if (!any) {                                        // wave-uniform: no row of the block sees the tile
#pragma unroll
    for (int j = 0; j < 16; ++j) load(j);
    return;
  }
  const bool edge = (k0 + kBN - 1 > r0) || (k0 < r0 + 31 - (kWindow - 1));
  auto read_k = [&](int s) { return as_bf16x8(*reinterpret_cast<const u32x4*>(ks + kswz_read(2 * s + half, r32))); };
  auto read_v = [&](int tt, int db) {
    const int off = v_lane_off + 16 * tt * 512 + 64 * (db ^ vr);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + off + 8 * 512));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // K fragments eight ahead of their MFMA, V fragments of the first 16 keys during the
  // softmax and of the second 16 during the first half of the PV MFMAs.
  bf16x8 ka[16];
#pragma unroll
  for (int s = 0; s < 8; ++s) ka[s] = read_k(s);
  f32x16 sacc;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s == 0)
      mfma_qk_asm<true, false>(sacc, ka[s], qf[s]);
    else if (s == 15)
      mfma_qk_asm<false, true>(sacc, ka[s], qf[s]);
    else
      mfma_qk_asm<false, false>(sacc, ka[s], qf[s]);
    if (s + 8 < 16) ka[s + 8] = read_k(s + 8);
    load(s);
  }
  bf16x8 va[2][8];
#pragma unroll
  for (int db = 0; db < 8; ++db) va[0][db] = read_v(0, db);
  const int rpos = r0 + r32;
  if (edge) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = k0 + 8 * (v >> 2) + 4 * half + (v & 3);
      sacc[v] = (key <= rpos && key > rpos - kWindow) ? sacc[v] : -INFINITY;
    }
  }
  const float mt = max_halves(max16(sacc));
  if (__any(mt > m_run + kRescaleThreshold)) {
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_part *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
    m_run = m_new;
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float l_pair[2] = {0.0f, 0.0f};
  bf16x8 pf[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    u32x4 pk;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 p2 = {(__bf16)__builtin_amdgcn_exp2f(sacc[8 * tt + 2 * w] - m_run),
                         (__bf16)__builtin_amdgcn_exp2f(sacc[8 * tt + 2 * w + 1] - m_run)};
      l_pair[w & 1] = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l_pair[w & 1], false);
      pk[w] = __builtin_bit_cast(uint32_t, p2);
    }
    pf[tt] = as_bf16x8(pk);
  }
  l_part += l_pair[0] + l_pair[1];
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    if (db == 0)
      mfma_pv_asm<true>(o[db], va[0][db], pf[0]);
    else
      mfma_pv_asm<false>(o[db], va[0][db], pf[0]);
    va[1][db] = read_v(1, db);
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    if (db == 0)
      mfma_pv_asm<true>(o[db], va[1][db], pf[1]);
    else
      mfma_pv_asm<false>(o[db], va[1][db], pf[1]);
  }
}

template <int HPW>
__global__ __launch_bounds__(128 * HPW) __attribute__((amdgpu_waves_per_eu(HPW / 2, HPW / 2)))
void prefill_split_kernel(PrefillArgs a) {
  using T = LayerTraits<kSliding>;
  static_assert(HPW == 2 || HPW == 4, "query heads per workgroup");
  constexpr int kParts = kGroup / HPW;              // workgroups per (block, KV head)
  constexpr int kNL = split_loads<HPW>();
  // [band half][stage][K, V]: 128 KB; after the loop it holds the second half's O.
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[2][2][2][kTileBytes];
  __shared__ double s_inv[T::kRot / 2];
  __shared__ float s_ml[kGroup][2][2][64];          // [head][half][max, row sums][lane]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = wave / HPW, hw = wave % HPW;      // band half, head within the workgroup
  const int half = lane >> 5, r32 = lane & 31;
  const int units = a.batch * kKvHeads * kParts;
  const int u = blockIdx.x % units;
  const int part = u % kParts, g = (u / kParts) % kKvHeads, b = u / (kParts * kKvHeads);
  const int q0 = (blockIdx.x / units) * kSplitRows;
  const SeqSpan sp = seq_span(a, b);
  const int S = sp.len;
  if (q0 >= S) return;                              // whole workgroup
  const int hq = g * kGroup + part * HPW + hw;

  const int hi_key = min(q0 + kSplitRows - 1, S - 1);
  const int lo_key = max(0, q0 - (kWindow - 1));
  const int kt_lo = lo_key / kBN, n = hi_key / kBN - kt_lo + 1;
  const int n0 = (n + 1) / 2;                       // tiles of the first half (the second: n - n0)
  const int my_lo = bh ? kt_lo + n0 : kt_lo, my_n = bh ? n - n0 : n0;
  uint8_t* const ring = &s_ring[bh][0][0][0];
  // Load j of a tile of this half: the HPW waves of the half each issue the loads of
  // 8 / HPW of prefill_kernel's waves (virtual waves (8 / HPW) hw + j / 4).
  auto issue_j = [&](int kt, int stage, int j) {
    uint8_t* ks = ring + stage * 2 * kTileBytes;
    issue_one<kSliding, false, true>(a, b, sp, g, kt * kBN, (8 / HPW) * hw + (j >> 2), lane, ks, ks + kTileBytes, j & 3);
  };
  if (my_n > 0) {
#pragma unroll
    for (int j = 0; j < kNL; ++j) issue_j(my_lo, 0, j);
  }
  bf16x8 qf[16];
  uint16_t gate_raw = 0;                            // HPW = 2: loaded here, used by the epilogue
  if constexpr (HPW == 2) {
    // The two waves of a head (the band halves) each load and rotate half of its Q
    // fragments, the rotary pairs (s, s + 8) for s in [4 bh, 4 bh + 4) (sliding layers
    // rotate all 256 dims), into LDS -- the first half's second ring stage, idle until the
    // first step issues its loads -- and both read all 16 back, into AGPRs.  The loads go
    // out before the frequency table is computed, which hides part of their latency.
    static_assert(T::kRot == kHeadDim, "every Q fragment is in a rotary pair");
    // Rows past the sequence's end read its last row (their outputs are never stored):
    // loads under a branch would be waited for at the branch's end.
    const int row = q0 + r32, rowc = min(row, S - 1);
    const uint16_t* qrow = a.q + ((sp.row0 + rowc) * kQHeads + hq) * kHeadDim;
    u32x4 qr[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qr[j] = ld_global16(qrow + 16 * (4 * bh + j) + 8 * half);
      qr[4 + j] = ld_global16(qrow + 16 * (4 * bh + j + 8) + 8 * half);
    }
    gate_raw = a.gate[(sp.row0 + rowc) * kQHeads + hq];
    if (tid < T::kRot / 2) s_inv[tid] = rope_inv_rev(tid, T::kRot, log2(T::kTheta));
    barrier_lds();
    uint8_t* const qs = &s_ring[0][1][0][0] + hw * kTileBytes;   // [fragment][lane] x 16 B per head
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sf = 4 * bh + j;
      bf16x8 y1, y2;
      rotate_q_pair(qr[j], qr[4 + j], (double)row, s_inv, 16 * sf + 8 * half, y1, y2);
      *reinterpret_cast<bf16x8*>(qs + (sf * 64 + lane) * 16) = y1;
      *reinterpret_cast<bf16x8*>(qs + ((sf + 8) * 64 + lane) * 16) = y2;
    }
    barrier_lds();
    lds_read16_agpr(qs + lane * 16, qf);
  } else {
    if (tid < T::kRot / 2) s_inv[tid] = rope_inv_rev(tid, T::kRot, log2(T::kTheta));
    barrier_lds();
    load_q<kSliding>(a, sp, hq, q0 + r32, 0, half, s_inv, qf);
  }
  wait_vmcnt<0>();
  barrier_lds();

  f32x16 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x16{0};
  float m_run = -1e30f, l_part = 0.0f;
  const int grp = lane >> 4, vr = (lane >> 2) & 3, vc = lane & 3;
  const int v_lane_off = (4 * (grp >> 1) + vr) * 512 + 16 * (2 * (grp & 1) + (vc >> 1)) + 8 * (vc & 1);

  // Both halves step together (one barrier per step); the second half has n - n0 <= n0
  // tiles and idles in its last step when n is odd.
  for (int i = 0; i < n0; ++i) {
    const int st = i & 1;
    if (i < my_n) {
      // The next tile goes into the stage read in step i - 1 (every wave passed the barrier
      // after it).  The last step loads its own tile there again, unused: a conditional
      // load would put branches among the QK MFMAs.
      const int kt_next = min(my_lo + i + 1, my_lo + my_n - 1);
      const uint8_t* ks = ring + st * 2 * kTileBytes;
      auto ld = [&](int j) { issue_j(kt_next, st ^ 1, j); };
      if constexpr (HPW == 2)
        split_tile_deep(ks, ks + kTileBytes, (my_lo + i) * kBN, q0, lane, qf, o, m_run, l_part, v_lane_off, ld);
      else
        split_tile<kNL>(ks, ks + kTileBytes, (my_lo + i) * kBN, q0, lane, qf, o, m_run, l_part, v_lane_off, ld);
      wait_vmcnt<0>();                              // this lane's loads (also before the merge reuses the rings)
    }
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (HPW == 2) mfma_result_fence(o);
  // The halves split the rest: the first stores dims 0 .. 127 (blocks 0 .. 3 of O), the
  // second dims 128 .. 255.  Each hands the other its (max, row sums) and the four blocks
  // the other stores, through LDS (the rings are idle now; 16 bytes per lane,
  // lane-linear), merges the four it keeps with the partner's by log-sum-exp weights and
  // runs the gated epilogue on them.
  f32x4* const s_o = reinterpret_cast<f32x4*>(&s_ring[0][0][0][0]);   // [half][HPW][16][64] x 16 B
  auto exchange = [&](auto keep_tag) {
    constexpr int kKeep = decltype(keep_tag)::value, kGive = 4 - kKeep;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        s_o[((bh * HPW + hw) * 16 + 4 * i + qd) * 64 + lane] =
            f32x4{o[kGive + i][4 * qd], o[kGive + i][4 * qd + 1], o[kGive + i][4 * qd + 2], o[kGive + i][4 * qd + 3]};
    s_ml[hw][bh][0][lane] = m_run;
    s_ml[hw][bh][1][lane] = l_part;
    barrier_lds();
    const float m1 = s_ml[hw][1 - bh][0][lane], l1 = s_ml[hw][1 - bh][1][lane];
    const float mm = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
    l_part = l_part * a0 + l1 * a1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const f32x4 x = s_o[(((1 - bh) * HPW + hw) * 16 + 4 * i + qd) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[kKeep + i][4 * qd + e] = o[kKeep + i][4 * qd + e] * a0 + x[e] * a1;
      }
    barrier_lds();                                  // merge reads done before the staging writes
  };
  // Epilogue: O / l * sigmoid(gate) for this half's 128 dims, staged through LDS (pitch 264
  // bytes) so that the stores write whole 256-byte row runs (non-temporal, as in the
  // 64-row kernel's sliding epilogue: 2% faster here).
  auto epilogue = [&](auto keep_tag) {
    constexpr int kKeep = decltype(keep_tag)::value;
    const int row = q0 + r32;
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    const float gl = HPW == 2 ? bf16_to_f32(gate_raw)
                              : row < S ? bf16_to_f32(a.gate[(sp.row0 + row) * kQHeads + hq]) : 0.0f;
    const float scale = sigmoidf_fast(gl) / l_tot;
    constexpr int kPitch = 264;
    uint8_t* const stage = &s_ring[0][0][0][0] + (bh * HPW + hw) * (32 * kPitch);
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        u32x2 w;
        w[0] = pack_bf16x2(o[kKeep + d4][4 * qd] * scale, o[kKeep + d4][4 * qd + 1] * scale);
        w[1] = pack_bf16x2(o[kKeep + d4][4 * qd + 2] * scale, o[kKeep + d4][4 * qd + 3] * scale);
        *reinterpret_cast<u32x2*>(stage + r32 * kPitch + (32 * d4 + 8 * qd + 4 * half) * 2) = w;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));   // lgkmcnt(0): own writes
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = 4 * i + (lane >> 4), c = lane & 15;
      const u32x4 x = *reinterpret_cast<const u32x4*>(stage + rr * kPitch + c * 16);
      const int grow = q0 + rr;
      if (grow < S)
        __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(a.out + ((sp.row0 + grow) * kQHeads + hq) * kHeadDim +
                                                             32 * kKeep + 8 * c));
    }
  };
  if (bh == 0) {
    exchange(std::integral_constant<int, 0>{});
    epilogue(std::integral_constant<int, 0>{});
  } else {
    exchange(std::integral_constant<int, 4>{});
    epilogue(std::integral_constant<int, 4>{});
  }
}

}  // namespace

hipError_t launch_prefill(int layer_type, const PrefillArgs& a, hipStream_t stream) {
  const int blocks = a.nqb * a.batch * kKvHeads;
  const dim3 rope_grid((unsigned)(((size_t)a.seq_len * kKvHeads * 32 + 255) / 256), (unsigned)a.batch);
  if (layer_type == kSliding) {
    hipLaunchKernelGGL(prefill_rope_kernel<kSliding>, rope_grid, dim3(256), 0, stream, a);
    // Too few 64-row blocks to fill the chip's 256 CUs: 32-row blocks with the key band
    // split over two wave groups (batches without a cached prefix, uniform lengths).
    if (a.start_pos == 0 && a.cu_seqlens == nullptr && blocks < kCUs) {
      const int nqb32 = (a.seq_len + kSplitRows - 1) / kSplitRows;
      const int wgs = nqb32 * a.batch * kKvHeads;   // workgroups of the whole-group form
      if (split_two_heads(wgs))
        hipLaunchKernelGGL(prefill_split_kernel<2>, dim3(2 * wgs), dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL(prefill_split_kernel<4>, dim3(wgs), dim3(512), 0, stream, a);
      return hipGetLastError();
    }
    if (a.start_pos > 0)
      hipLaunchKernelGGL((prefill_kernel<kSliding, true>), dim3(blocks), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<kSliding, false>), dim3(blocks), dim3(kThreads), 0, stream, a);
    if (a.start_pos > 0 && a.cache_k != nullptr) {
      const int kept = a.seq_len < kWindow ? a.seq_len : kWindow;
      const size_t n = (size_t)a.batch * kept * kKvHeads * 32;
      hipLaunchKernelGGL(prefill_ring_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
    }
  } else {
    if (a.start_pos == 0 && a.cache_k == nullptr) {
      constexpr int kRotChunks = LayerTraits<kFull>::kRot / 8;     // rotated 16-byte chunks per row
      const dim3 grid((unsigned)(((size_t)a.seq_len * kKvHeads * kRotChunks + 255) / 256), (unsigned)a.batch);
      hipLaunchKernelGGL((prefill_rope_kernel<kFull, true>), grid, dim3(256), 0, stream, a);
    } else {
      hipLaunchKernelGGL(prefill_rope_kernel<kFull>, rope_grid, dim3(256), 0, stream, a);
    }
    if (a.start_pos > 0)
      hipLaunchKernelGGL((prefill_kernel<kFull, true>), dim3(blocks), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<kFull, false>), dim3(blocks), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

size_t prefill_workspace_bytes(int batch, int seq_len) {
  return (size_t)batch * seq_len * kKvHeads * kHeadDim * sizeof(uint16_t);   // [T, 4, 256] bf16
}

int prefill_block_rows() { return kBM; }

}  // namespace spark
