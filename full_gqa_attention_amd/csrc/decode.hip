// Split-KV GQA decode for the hybrid sliding/full layer on gfx950.
//
// Decode is bound by streaming the KV cache from HBM (F16 vs Q4 comparison page,
// hotelren.com/news/5475707, section 二: each generated token re-reads its state), so
// every cache byte is read exactly once and the whole batch's reads are spread evenly
// over the workgroups:
//   * partition: sequence b owns c_b = ceil(n_b / 32) chunks of 32 visible keys; the chunks
//     of all sequences are numbered back to back and partition w of P takes chunks
//     [floor(wC/P), floor((w+1)C/P)).  Every workgroup computes the prefix sums of the c_b
//     itself (a scan over the batch in LDS) and finds its first sequence, so the plan costs
//     no launch and no host sync, and uneven context lengths still give every workgroup
//     the same amount of traffic.  Workgroup 0 also records, for the merge, the range of
//     partitions that touch each sequence.
//   * split: workgroup w walks its chunks; each run of chunks inside one sequence is a
//     segment with its own online softmax, written as a partial result (max, sum,
//     unnormalised O per query head) to slot w + b, which is unique because both w and b
//     only grow along the partition.  The workgroup has one wave per KV head, and that
//     wave scores the 4 query heads sharing the head against each key row it loads (GQA,
//     Spark-X2.6-4B-Base explainer, eliteato.com/news/34565, section "配套效率设计"):
//       - S = Q K^T on v_mfma_f32_16x16x32_bf16 (rows = the 4 query heads, padded to 16),
//         K rows loaded straight into the B operand (64 contiguous bytes per key per load);
//       - online softmax in fp32 / log2 domain across the 16 lanes that hold the scores;
//       - O += P V on the VALU in fp32: V rows are loaded fully coalesced (two 512-byte
//         rows per instruction), each lane owns 8 dims of one key parity, P from LDS.
//   * merge: per (sequence, query head), the partials of the partitions that touched the
//     sequence are combined with log-sum-exp weights and the sigmoid head gate is applied.
// Sliding layers read the 512-slot ring; full layers the contiguous cache.
//
// The 8-bit cache (q8_0 blocks of 32 along head_dim, Sharp-Spark-X2.5-4B-GGUF guide,
// section 四) runs the same kernels with Q8 = true: each 32-dim MFMA step of S = Q K^T is
// exactly one quantisation block, so the K codes enter the MFMA as bf16 integers (exact,
// |code| <= 127) and the step's result is scaled by that key's block scale in fp32; V
// codes are read back as code * scale on the VALU.
#include "spark_device.hpp"
#include "spark_launch.hpp"

namespace spark {
namespace {

constexpr int kThreads = 256;   // 4 waves = 4 KV heads
constexpr int kChunk = 32;      // keys per inner iteration and per partition unit
constexpr int kSlot = kKvHeads * kHeadDim;   // bf16 per cache slot
// LDS pitch of a staged 8-bit K row: 256 code bytes + 16, so that the 8-byte fragment reads
// of 16 keys x two 8-byte column groups (half a wave) fall on 64 distinct banks.
constexpr int kK8Pitch = 272;

template <int LT>
__device__ __forceinline__ int visible_keys(int L, int cap) {
  const int n = LT == kFull ? L : min(L, kWindow);
  return max(0, min(n, cap));   // never read past the cache; L < 1 sees nothing
}

template <int LT>
__device__ __forceinline__ int chunks_of(int L, int cap) {
  return (visible_keys<LT>(L, cap) + kChunk - 1) / kChunk;
}

// First chunk of partition w: floor(w C / P).
__device__ __forceinline__ int part_lo(int w, int C, int P) {
  return (int)(((long long)w * C) / P);
}

// Partition holding chunk x: the largest w with floor(w C / P) <= x.
__device__ __forceinline__ int part_of(int x, int C, int P) {
  return (int)((((long long)(x + 1) * P) + C - 1) / C) - 1;
}

__device__ __forceinline__ float half_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Eight int8 codes (two dwords) as eight exact bf16 values.
__device__ __forceinline__ bf16x8 codes_to_bf16(u32x2 x) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t d = x[w >> 1] >> (16 * (w & 1));
    r[w] = pack_bf16x2((float)(int8_t)(d & 0xff), (float)(int8_t)((d >> 8) & 0xff));
  }
  return as_bf16x8(r);
}

// Online-softmax attention of the 4 query heads of KV head g of sequence b over keys
// [ks, ke) of its cache; writes the partial result to slot `slot`.
template <int LT, bool Q8>
__device__ __forceinline__ void attend_segment(const DecodeArgs& a, int b, int L, int ks, int ke,
                                               int slot, int g, int lane, const double* s_inv,
                                               float (*s_p)[kChunk][4], float (*s_alpha)[4],
                                               uint8_t* s_k8) {
  // Q as the A operand: lane l holds head l % 16 (only 0..3 are real), dims 32s + 8(l/16) + j.
  const int hrow = lane & 15;
  const int kq = lane >> 4;
  bf16x8 qa[8];
  {
    u32x4 raw[8];
    if (hrow < kGroup) {
      const uint16_t* qrow = a.q + ((size_t)b * kQHeads + g * kGroup + hrow) * kHeadDim;
#pragma unroll
      for (int s = 0; s < 8; ++s) raw[s] = ld_global16(qrow + 32 * s + 8 * kq);
      const double p = (double)(L - 1);
      if (LT == kSliding) {        // chunk s pairs with chunk s + 4 (d + 128)
#pragma unroll
        for (int s = 0; s < 4; ++s) rope_rotate_chunks(raw[s], raw[s + 4], p, s_inv, 32 * s + 8 * kq);
      } else {                     // chunk 0 (d < 32) pairs with chunk 1 (d + 32)
        rope_rotate_chunks(raw[0], raw[1], p, s_inv, 8 * kq);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) raw[s] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) qa[s] = as_bf16x8(raw[s]);
  }

  const size_t seq_base = (size_t)b * a.cache_cap * kSlot + (size_t)g * kHeadDim;
  const uint16_t* kbase = a.cache_k + seq_base;
  const uint16_t* vbase = a.cache_v + seq_base;
  // PV: bf16 -- lane owns 8 dims of the keys of one parity (two 512-byte rows per load);
  // 8-bit -- lane owns 16 dims (half a quantisation block) of the keys c0 + 4i + l / 16
  // (four 256-byte code rows per 16-byte load, one scale per key).
  constexpr int kVDims = Q8 ? 16 : 8;
  constexpr int kVStep = kVDims / 4;                    // keys per load instruction
  constexpr int kVKeys = kChunk / kVStep;               // keys per lane and chunk
  const int vpar = Q8 ? lane >> 4 : lane >> 5;          // key residue this lane accumulates
  const int vdim = kVDims * (Q8 ? lane & 15 : lane & 31);   // first of the dims this lane owns

  float m_run[4], l_run[4], acc[4][kVDims];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    m_run[h] = -1e30f;
    l_run[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < kVDims; ++e) acc[h][e] = 0.0f;
  }

  // 8-bit cache: codes at the same element offsets (one byte each); scales [slot][4][8].
  const int8_t* kbase8 = a.k_codes + seq_base;
  const int8_t* vbase8 = a.v_codes + seq_base;
  const size_t sc_base = ((size_t)b * a.cache_cap * kKvHeads + g) * 8;
  const uint16_t* kscale = a.k_scales + sc_base;
  const uint16_t* vscale = a.v_scales + sc_base;

  for (int c0 = ks; c0 < ke; c0 += kChunk) {
    u32x4 kr[2][8];
    u32x2 kr8[2][8];
    u32x4 ksc[2];
    if constexpr (Q8) {
      // The chunk's K codes through LDS: eight 16-byte loads per lane (key 4i + l / 16,
      // bytes 16 (l % 16) ..), then the 8-byte MFMA fragments read back.  A row past the
      // segment reads its first key: finite, and masked below, so nothing needs zeroing.
      u32x4 kg[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = c0 + 4 * i + (lane >> 4);
        const uint32_t row = (uint32_t)(key < ke ? key : ks);
        kg[i] = *reinterpret_cast<const u32x4*>(kbase8 + (row * kSlot + 16 * (lane & 15)));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(s_k8 + (4 * i + (lane >> 4)) * kK8Pitch + 16 * (lane & 15)) = kg[i];
      // Other lanes of this wave read these rows next, and the next chunk overwrites them
      // after this one's reads.  The rows belong to this wave alone, and LDS executes one
      // wave's operations in issue order, so a write is in LDS before any later read of the
      // wave and a read has its data before any later write; the wave barrier only keeps the
      // compiler from moving the accesses across it.
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < 8; ++s)
          kr8[kb][s] = *reinterpret_cast<const u32x2*>(s_k8 + (16 * kb + hrow) * kK8Pitch + 32 * s + 8 * kq);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = c0 + 16 * kb + hrow;
      const bool ok = key < ke;
      const size_t row = (size_t)(ok ? key : ks);
      if constexpr (Q8) {
        // Scales straight from global memory; the codes come from the LDS stage below.
        ksc[kb] = ld_global16(kscale + (uint32_t)row * (kKvHeads * 8));
      } else {
        const uint16_t* src = kbase + row * kSlot + 8 * kq;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const u32x4 x = ld_global16(src + 32 * s);
          kr[kb][s] = ok ? x : u32x4{0, 0, 0, 0};
        }
      }
    }
    u32x4 vr[kVKeys];
    float vsc[kVKeys];
#pragma unroll
    for (int i = 0; i < kVKeys; ++i) {
      const int key = c0 + kVStep * i + vpar;
      const bool ok = key < ke;
      const size_t row = (size_t)(ok ? key : ks);
      if constexpr (Q8) {
        // As for K: a row past the segment gets P = 0, so its finite values add nothing.
        vr[i] = *reinterpret_cast<const u32x4*>(vbase8 + ((uint32_t)row * kSlot + vdim));
        vsc[i] = half_to_f32(vscale[(uint32_t)row * (kKvHeads * 8) + (vdim >> 5)]);
      } else {
        const u32x4 x = ld_global16(vbase + row * kSlot + vdim);
        vr[i] = ok ? x : u32x4{0, 0, 0, 0};
      }
    }

    // Scores: lanes 0..15 hold heads 0..3 (element v) for key c0 + 16kb + lane.
    float t[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 sc = f32x4{0, 0, 0, 0};
      if constexpr (Q8) {
        // Step s is block s of the key row; lanes 0..15 hold key hrow, whose scales
        // ksc[kb] holds (eight fp16).
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const f32x4 part = mfma_16x16x32(qa[s], codes_to_bf16(kr8[kb][s]), f32x4{0, 0, 0, 0});
          const float d = half_to_f32(ksc[kb][s >> 1] >> (16 * (s & 1)));
          sc += d * part;
        }
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) sc = mfma_16x16x32(qa[s], as_bf16x8(kr[kb][s]), sc);
      }
      const bool ok = c0 + 16 * kb + hrow < ke;
#pragma unroll
      for (int v = 0; v < 4; ++v) t[kb][v] = ok ? sc[v] * kScoreScaleLog2 : -INFINITY;
    }
    float alpha[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float mx = fmaxf(t[0][v], t[1][v]);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_new = fmaxf(m_run[v], mx);
      alpha[v] = __builtin_amdgcn_exp2f(m_run[v] - m_new);
      const float p0 = __builtin_amdgcn_exp2f(t[0][v] - m_new);
      const float p1 = __builtin_amdgcn_exp2f(t[1][v] - m_new);
      t[0][v] = p0;
      t[1][v] = p1;
      float ps = p0 + p1;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ps += __shfl_xor(ps, off);
      l_run[v] = l_run[v] * alpha[v] + ps;
      m_run[v] = m_new;
    }
    if (lane < 16) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        *reinterpret_cast<f32x4*>(&s_p[g][16 * kb + lane][0]) =
            f32x4{t[kb][0], t[kb][1], t[kb][2], t[kb][3]};
      if (lane == 0) *reinterpret_cast<f32x4*>(&s_alpha[g][0]) = f32x4{alpha[0], alpha[1], alpha[2], alpha[3]};
    }
    __builtin_amdgcn_wave_barrier();
    const f32x4 al = *reinterpret_cast<const f32x4*>(&s_alpha[g][0]);
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int e = 0; e < kVDims; ++e) acc[h][e] *= al[h];
#pragma unroll
    for (int i = 0; i < kVKeys; ++i) {
      f32x4 pp = *reinterpret_cast<const f32x4*>(&s_p[g][kVStep * i + vpar][0]);
      float x[kVDims];
      if constexpr (Q8) {
        pp *= vsc[i];                          // value = code * scale: fold the scale into P
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = (float)(int8_t)((vr[i][e >> 2] >> (8 * (e & 3))) & 0xff);
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          x[2 * w] = bf16_lo(vr[i][w]);
          x[2 * w + 1] = bf16_hi(vr[i][w]);
        }
      }
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int e = 0; e < kVDims; ++e) acc[h][e] += pp[h] * x[e];
    }
    __builtin_amdgcn_wave_barrier();
  }

  // Merge the lanes that hold the same dims of other keys, then write this segment's
  // partial results.
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < kVDims; ++e) {
      if constexpr (Q8) acc[h][e] += __shfl_xor(acc[h][e], 16);
      acc[h][e] += __shfl_xor(acc[h][e], 32);
    }

  const size_t head0 = (size_t)slot * kQHeads + g * kGroup;
  if (lane < 256 / kVDims) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float* dst = a.ws_o + (head0 + h) * kHeadDim + vdim;
#pragma unroll
      for (int e = 0; e < kVDims; e += 4)
        *reinterpret_cast<f32x4*>(dst + e) = f32x4{acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]};
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      a.ws_ml[(head0 + h) * 2] = m_run[h];
      a.ws_ml[(head0 + h) * 2 + 1] = l_run[h];
    }
  }
}

template <int LT, bool Q8>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  using T = LayerTraits<LT>;
  __shared__ double s_inv[T::kRot / 2];
  __shared__ __attribute__((aligned(16))) float s_p[kKvHeads][kChunk][4];
  __shared__ __attribute__((aligned(16))) float s_alpha[kKvHeads][4];
  // 8-bit cache: each wave's chunk of K codes, 32 rows at a 272-byte pitch.
  __shared__ __attribute__((aligned(16))) uint8_t s_k8[Q8 ? kKvHeads : 1][Q8 ? kChunk * kK8Pitch : 16];

  __shared__ int s_scan[kThreads];

  // Chunk counts of the batch: thread t owns sequences [t per, t per + per); inclusive
  // prefix sums over the threads.
  const int tid = threadIdx.x;
  const int per = (a.batch + kThreads - 1) / kThreads;
  const int b0 = min(tid * per, a.batch);
  const int b1 = min(b0 + per, a.batch);
  int own = 0;
  for (int b = b0; b < b1; ++b) own += chunks_of<LT>(a.seq_lens[b], a.cache_cap);
  s_scan[tid] = own;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  const int C = s_scan[kThreads - 1];
  const int P = min(a.nparts, C);            // so that no partition is empty
  const int w = blockIdx.x;
  if (w == 0) {
    // Partitions touching each sequence: those holding its first and its last chunk, and
    // all between (read by the merge).
    int run = s_scan[tid] - own;
    for (int b = b0; b < b1; ++b) {
      const int c = chunks_of<LT>(a.seq_lens[b], a.cache_cap);
      a.ws_range[b] = c > 0 ? int2{part_of(run, C, P), part_of(run + c - 1, C, P)} : int2{0, -1};
      run += c;
    }
  }
  if (w >= P) return;                        // uniform over the workgroup
  const int lo = part_lo(w, C, P);
  const int hi = part_lo(w + 1, C, P);

  const int lane = tid & 63;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < T::kRot / 2) s_inv[tid] = rope_inv_rev(tid, T::kRot, log2(T::kTheta));
  __syncthreads();

  // The thread owning chunk lo is the first whose inclusive prefix exceeds lo; walk its
  // sequences from there.  Each sequence with chunks in [lo, hi) is one segment.
  int t0 = 0, t1 = kThreads - 1;
  while (t0 < t1) {
    const int mid = (t0 + t1) >> 1;
    if (s_scan[mid] > lo) t1 = mid; else t0 = mid + 1;
  }
  int b = min(t0 * per, a.batch);
  int cb = t0 > 0 ? s_scan[t0 - 1] : 0;      // chunks before sequence b
  for (;;) {
    const int L = a.seq_lens[b];
    const int n = visible_keys<LT>(L, a.cache_cap);
    const int cn = cb + (n + kChunk - 1) / kChunk;
    if (cn > lo && cn > cb) {
      const int ks = (max(lo, cb) - cb) * kChunk;
      const int ke = min((min(hi, cn) - cb) * kChunk, n);
      attend_segment<LT, Q8>(a, b, L, ks, ke, w + b, g, lane, s_inv, s_p, s_alpha, &s_k8[Q8 ? g : 0][0]);
    }
    if (cn >= hi || b + 1 >= a.batch) break;
    ++b;
    cb = cn;
  }
}

// One wave per (sequence, query head); lane l owns dims 4l..4l+3.  The partials are
// merged in one online pass: running max, rescaled sum and rescaled output.
constexpr int kReduceWaves = 4;

__global__ __launch_bounds__(64 * kReduceWaves) void decode_reduce_kernel(DecodeArgs a) {
  __shared__ float s_ml[kReduceWaves][2];
  __shared__ f32x4 s_o[kReduceWaves][64];
  const int b = blockIdx.x / kQHeads;
  const int h = blockIdx.x % kQHeads;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int2 r = a.ws_range[b];
  // Wave v merges partitions r.x + v, r.x + v + 4, ... (lane: dims 4 lane .. 4 lane + 3).
  float m = -1e30f, l = 0.0f;
  f32x4 o = f32x4{0, 0, 0, 0};
#pragma unroll 4
  for (int w = r.x + wave; w <= r.y; w += kReduceWaves) {
    const size_t hs = (size_t)(w + b) * kQHeads + h;
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + hs * 2);
    const f32x4 ow = *reinterpret_cast<const f32x4*>(a.ws_o + hs * kHeadDim + 4 * lane);
    const float mn = fmaxf(m, ml.x);
    const float sa = __builtin_amdgcn_exp2f(m - mn);
    const float sb = __builtin_amdgcn_exp2f(ml.x - mn);
    l = l * sa + ml.y * sb;
    o = o * sa + ow * sb;
    m = mn;
  }
  if (lane == 0) { s_ml[wave][0] = m; s_ml[wave][1] = l; }
  s_o[wave][lane] = o;
  __syncthreads();
  if (wave != 0) return;
  float mt = s_ml[0][0];
#pragma unroll
  for (int v = 1; v < kReduceWaves; ++v) mt = fmaxf(mt, s_ml[v][0]);
  float lt = 0.0f;
  f32x4 ot = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int v = 0; v < kReduceWaves; ++v) {
    const float sv = __builtin_amdgcn_exp2f(s_ml[v][0] - mt);
    lt += s_ml[v][1] * sv;
    ot += s_o[v][lane] * sv;
  }
  // No visible key (r empty): l = 0 and o = 0, written as zeros.
  const float gl = bf16_to_f32(a.gate[(size_t)b * kQHeads + h]);
  const float sc = lt > 0.0f ? sigmoidf_fast(gl) / lt : 0.0f;
  uint16_t* dst = a.out + ((size_t)b * kQHeads + h) * kHeadDim + 4 * lane;
  *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(ot[0] * sc, ot[1] * sc), pack_bf16x2(ot[2] * sc, ot[3] * sc)};
}

// ---------------------------------------------------------------------------------------
// Sliding layers in one launch.  A sequence sees at most 512 keys, the valid ring slots
// [0, n) with n = min(L, 512) (softmax does not depend on their order), i.e. at most 16
// chunks of 32.  Workgroup (b, g) has 8 waves; wave w takes chunks w and w + 8, scoring
// the 4 query heads of KV head g against their keys with an online softmax.  The 8 states
// meet in LDS, where the workgroup merges them with log-sum-exp weights and applies the
// gate: one pass over the ring, no partial results in HBM and no merge launch.  A wave
// issues its first chunk's K and V loads before anything else and the second chunk's as
// soon as the first one's registers are consumed (K after the scores, V after the PV
// sums), so the CU streams its 512 KB share of the ring with about one chunk per wave in
// flight.
constexpr int kRingWaves = 8;
constexpr int kRingChunks = kWindow / kChunk / kRingWaves;   // 2 per wave
constexpr int kRingVKeys = kChunk / 2;                        // V loads per lane and chunk

// K of keys [ks, ke): lane l takes key ks + 16 kb + l % 16, dims 32 s + 8 (l / 16) .. + 7
// (the MFMA B operand).  Keys past ke read slot ks (finite, masked by the caller).
__device__ __forceinline__ void ring_load_k(const DecodeArgs& a, size_t seq_base, int ks, int ke, int lane,
                                            u32x4 (&kr)[2][8]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = ks + 16 * kb + (lane & 15);
    const uint16_t* src = a.cache_k + seq_base + (uint32_t)(key < ke ? key : ks) * kSlot + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 8; ++s) kr[kb][s] = ld_global16(src + 32 * s);
  }
}

// V of keys [ks, ke): lane l takes dims 8 (l % 32) .. + 7 of the keys of parity l / 32
// (two 512-byte rows per load instruction).
__device__ __forceinline__ void ring_load_v(const DecodeArgs& a, size_t seq_base, int ks, int ke, int lane,
                                            u32x4 (&vr)[kRingVKeys]) {
#pragma unroll
  for (int i = 0; i < kRingVKeys; ++i) {
    const int key = ks + 2 * i + (lane >> 5);
    vr[i] = ld_global16(a.cache_v + seq_base + (uint32_t)(key < ke ? key : ks) * kSlot + 8 * (lane & 31));
  }
}

__global__ __launch_bounds__(64 * kRingWaves) void decode_ring_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float s_o[kRingWaves][kGroup][kHeadDim];   // 32 KB
  __shared__ __attribute__((aligned(16))) float s_p[kRingWaves][kChunk][4];
  __shared__ float s_ml[kRingWaves][kGroup][2];
  const int b = blockIdx.x / kKvHeads;
  const int g = blockIdx.x % kKvHeads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = a.seq_lens[b];
  const int n = max(0, min(min(L, kWindow), a.cache_cap));
  const int hrow = lane & 15, kq = lane >> 4;
  const int vpar = lane >> 5, vdim = 8 * (lane & 31);
  const size_t seq_base = (size_t)b * a.cache_cap * kSlot + (size_t)g * kHeadDim;

  // The gate logits of the two outputs this thread finishes (heads tid / 256 and + 2 of the
  // group), Q of the 4 heads of KV head g (lanes 0..15: head l % 16, the first 4 real) and
  // this wave's first chunk: all loads issued together.
  const uint16_t g0 = a.gate[(size_t)b * kQHeads + g * kGroup + (tid >> 8)];
  const uint16_t g1 = a.gate[(size_t)b * kQHeads + g * kGroup + (tid >> 8) + 2];
  u32x4 raw[8];
  u32x4 kr[2][8];
  u32x4 vr[kRingVKeys];
  const int ks0 = kChunk * w;
  if (ks0 < n) {
    if (hrow < kGroup) {
      const uint16_t* qrow = a.q + ((size_t)b * kQHeads + g * kGroup + hrow) * kHeadDim;
#pragma unroll
      for (int s = 0; s < 8; ++s) raw[s] = ld_global16(qrow + 32 * s + 8 * kq);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) raw[s] = u32x4{0, 0, 0, 0};
    }
    ring_load_k(a, seq_base, ks0, min(ks0 + kChunk, n), lane, kr);
    ring_load_v(a, seq_base, ks0, min(ks0 + kChunk, n), lane, vr);
  }

  float m_run[4], l_run[4], acc[4][8];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    m_run[h] = -1e30f;
    l_run[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  }
  if (ks0 < n) {
    // Q rotated at position L - 1 (frequencies from the compile-time table) while the K and
    // V loads are in flight.
    bf16x8 qa[8];
    if (hrow < kGroup) {
      // Pair 32 s + 8 kq + j: the table entry of 32 s + j (a constant) times theta^(-16 kq / r).
      const double f = kq == 0 ? kRopeStep8[0] : kq == 1 ? kRopeStep8[1] : kq == 2 ? kRopeStep8[2] : kRopeStep8[3];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        rope_rotate_pairs(raw[s], raw[s + 4], (double)(L - 1),
                          [&](int j) { return kRopeSliding.inv_rev[32 * s + j] * f; });
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) qa[s] = as_bf16x8(raw[s]);
    // One chunk [ks, ke) on the K and V now in registers; after_scores() runs once the K
    // registers are consumed, after_pv() once the V registers are.
    auto chunk = [&](int ks, int ke, auto after_scores, auto after_pv) {
      // Scores: lanes 0..15 hold heads 0..3 (element v) for key ks + 16 kb + lane.
      float t[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x4 sc = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < 8; ++s) sc = mfma_16x16x32(qa[s], as_bf16x8(kr[kb][s]), sc);
        const bool ok = ks + 16 * kb + hrow < ke;
#pragma unroll
        for (int v = 0; v < 4; ++v) t[kb][v] = ok ? sc[v] * kScoreScaleLog2 : -INFINITY;
      }
      after_scores();
      float alpha[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float mx = fmaxf(t[0][v], t[1][v]);
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        const float m_new = fmaxf(m_run[v], mx);
        alpha[v] = __builtin_amdgcn_exp2f(m_run[v] - m_new);
        const float p0 = __builtin_amdgcn_exp2f(t[0][v] - m_new);
        const float p1 = __builtin_amdgcn_exp2f(t[1][v] - m_new);
        t[0][v] = p0;
        t[1][v] = p1;
        float ps = p0 + p1;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) ps += __shfl_xor(ps, off);
        l_run[v] = l_run[v] * alpha[v] + ps;
        m_run[v] = m_new;
        // Lanes 16..63 reduced the padding rows of the MFMA, not these heads: every lane
        // rescales its value sums by lane 0's factor.
        alpha[v] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[v]), 0));
      }
      // P through this wave's own LDS rows to the lanes that own the value dims.  One wave
      // issues its LDS operations in order, so the wave barriers (which only keep the
      // compiler from moving the accesses across them) suffice between its writes and reads.
      if (lane < 16) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          *reinterpret_cast<f32x4*>(&s_p[w][16 * kb + lane][0]) = f32x4{t[kb][0], t[kb][1], t[kb][2], t[kb][3]};
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha[h];
#pragma unroll
      for (int i = 0; i < kRingVKeys; ++i) {
        const f32x4 pp = *reinterpret_cast<const f32x4*>(&s_p[w][2 * i + vpar][0]);
        float x[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x[2 * q] = bf16_lo(vr[i][q]);
          x[2 * q + 1] = bf16_hi(vr[i][q]);
        }
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] += pp[h] * x[e];
      }
      __builtin_amdgcn_wave_barrier();
      after_pv();
    };
    static_assert(kRingChunks == 2, "two chunks per wave");
    // The second chunk's loads are unconditional (no register of the first chunk has to
    // survive them): when it lies past n its rows are clamped into the 512-slot ring and
    // never used.
    const int ks1 = ks0 + kChunk * kRingWaves;
    const int ke1 = max(min(ks1 + kChunk, n), ks1);
    chunk(ks0, min(ks0 + kChunk, n),
          [&] {
            __builtin_amdgcn_sched_barrier(0);   // not hoisted above the scores (registers)
            ring_load_k(a, seq_base, ks1, ke1, lane, kr);
          },
          [&] {
            __builtin_amdgcn_sched_barrier(0);   // not hoisted above the PV sums (registers)
            ring_load_v(a, seq_base, ks1, ke1, lane, vr);
          });
    if (ks1 < n) chunk(ks1, ke1, [] {}, [] {});
    // Lanes holding the same dims of the other key parity.
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], 32);
  }
  // Every wave's state into LDS (a wave without keys: m = -1e30, l = 0, O = 0).
  if (lane < 32) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int e = 0; e < 8; e += 4)
        *reinterpret_cast<f32x4*>(&s_o[w][h][vdim + e]) = f32x4{acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]};
  }
  if (lane < 4) {
    s_ml[w][lane][0] = m_run[lane];
    s_ml[w][lane][1] = l_run[lane];
  }
  __syncthreads();
  // Thread t merges head h = idx / 256 of the group, dim d = idx % 256, idx = t and t + 512.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = tid + 64 * kRingWaves * j;
    const int h = idx >> 8, d = idx & 255;
    float M = -1e30f;
#pragma unroll
    for (int v = 0; v < kRingWaves; ++v) M = fmaxf(M, s_ml[v][h][0]);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int v = 0; v < kRingWaves; ++v) {
      const float sv = __builtin_amdgcn_exp2f(s_ml[v][h][0] - M);
      lsum += s_ml[v][h][1] * sv;
      o += s_o[v][h][d] * sv;
    }
    const int hq = g * kGroup + h;
    const float gl = bf16_to_f32(j == 0 ? g0 : g1);
    const float scale = lsum > 0.0f ? sigmoidf_fast(gl) / lsum : 0.0f;   // no visible key: zeros
    a.out[((size_t)b * kQHeads + hq) * kHeadDim + d] = (uint16_t)(pack_bf16x2(o * scale, 0.0f) & 0xffffu);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Partitions chosen automatically (bf16 cache): one per CU of MI355X (256 CUs).  One 4-wave
// workgroup per CU streams faster than two or more: fewer concurrent streams, each reading
// 64 KB of consecutive K (and V) slots per step, keep HBM rows open longer, and each extra
// partition adds a 16 KB partial result to write and merge.  A constant, not a query of the
// current device, so that the workspace size depends on the call's arguments alone.
constexpr int kDefaultParts = 256;

}  // namespace

// Partitions chosen automatically: one per CU for the bf16 cache (above); two per CU for
// the 8-bit cache, whose waves hold half the bytes in flight per load and issue more,
// smaller loads per byte: a second workgroup per CU keeps more bytes in flight while the
// other waits (batch 64, 1K-32K keys: 774 -> 525 us).
DecodePlan plan_decode(int layer_type, int batch, int max_seq_len, int nparts, bool q8) {
  DecodePlan p{};
  const int n = layer_type == kFull ? max_seq_len : (max_seq_len < kWindow ? max_seq_len : kWindow);
  const long long max_chunks = (long long)batch * ((n + kChunk - 1) / kChunk);
  int P = nparts;
  if (P <= 0) {
    const int want = (q8 ? 2 : 1) * kDefaultParts;
    P = (int)(max_chunks < want ? max_chunks : want);
    if (P < 1) P = 1;
  }
  p.nparts = P;
  p.range_offset = 0;
  p.o_offset = align256((size_t)batch * 2 * sizeof(int32_t));
  const size_t slots = (size_t)P + batch;
  p.ml_offset = p.o_offset + align256(slots * kQHeads * kHeadDim * sizeof(float));
  p.total_bytes = p.ml_offset + slots * kQHeads * 2 * sizeof(float);
  return p;
}

// bf16 sliding layers of a batch of at least 16 sequences: the one-launch ring kernel.
// Smaller batches give it too few workgroups (4 per sequence) to hide its three dependent
// memory round trips (Q with the first chunk, the second chunk's K, then its V): at batch 1
// and 4 it took 21 us against 16 us for split + merge, at batch 64 27 us against 32 us.
// Everything else runs split + merge (the 8-bit variant of the ring kernel ran out of
// registers with two chunks per wave: 93 spilled VGPRs).
constexpr int kRingMinBatch = 16;

template <bool Q8>
hipError_t launch_decode_impl(int layer_type, const DecodeArgs& a, hipStream_t stream) {
  if constexpr (!Q8) {
    if (layer_type == kSliding && a.batch >= kRingMinBatch) {
      hipLaunchKernelGGL(decode_ring_kernel, dim3(a.batch * kKvHeads), dim3(64 * kRingWaves), 0, stream, a);
      return hipGetLastError();
    }
  }
  if (layer_type == kSliding)
    hipLaunchKernelGGL((decode_split_kernel<kSliding, Q8>), dim3(a.nparts), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<kFull, Q8>), dim3(a.nparts), dim3(kThreads), 0, stream, a);
  hipLaunchKernelGGL(decode_reduce_kernel, dim3(a.batch * kQHeads), dim3(64 * kReduceWaves), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(int layer_type, const DecodeArgs& a, hipStream_t stream) {
  return launch_decode_impl<false>(layer_type, a, stream);
}

hipError_t launch_decode_q8(int layer_type, const DecodeArgs& a, hipStream_t stream) {
  return launch_decode_impl<true>(layer_type, a, stream);
}

}  // namespace spark
