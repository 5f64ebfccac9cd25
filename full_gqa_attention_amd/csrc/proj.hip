// Upstream projections of the attention layer on gfx950, in W8A8 FP8 (Spark-X2.6-4B-FP8
// walkthrough, nxmr.cn/news/148448, sections 二 and 三): q_k_v_proj with FP8 E4M3 weights
// (one static scale per output channel) and activations quantised to FP8 per token with a
// dynamic scale; g_proj in BF16.  Hidden 2560 -> q 4096, k 1024, v 1024 (section 一).
//
// Two launches:
//   * quant_gate_kernel: 16 tokens per workgroup read their hidden values once, compute the
//     16 gate logits from the bf16 values on v_mfma_f32_16x16x32_bf16 (fp32 accumulation,
//     g_proj), s = max|x| / 448 and the OCP E4M3FN codes of x / s (v_cvt_pk_fp8_f32:
//     nearest even), into the workspace;
//   * qkv_gemm_kernel: C = X_q W_q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (block scales 1),
//     output tiles of 256 tokens x 256 channels on 8 waves, K in stages of 128 bytes
//     through an LDS ring filled by direct global->LDS loads; epilogue C * s_token * s_channel, rounded to bf16,
//     staged through LDS by rows and stored straight into the q, k or v layout the attention
//     path reads.
#include "spark_device.hpp"
#include "spark_launch.hpp"

namespace spark {
namespace {

constexpr int kHidden = 2560;
constexpr int kQkvOut = 6144;
constexpr int kQOut = kQHeads * kHeadDim;      // 4096
constexpr int kKvOut = kKvHeads * kHeadDim;    // 1024
constexpr int kGates = kQHeads;                // 16 gate logits per token
constexpr float kE4M3Max = 448.0f;

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------------------
// Quantisation of the activations and the bf16 gate projection.  A workgroup of 4 waves
// takes 16 tokens; wave w holds the hidden slice [640 w, 640 w + 640) of all 16 in
// registers.  In K step s (32 values) lane l holds the 8 values of token l % 16 at
// 640 w + 32 s + 8 (l / 16): the A operand of v_mfma_f32_16x16x32_bf16, whose B operand is
// the same slice of gate row l % 16 (so the gate weights are read once per 16 tokens).
// The 4 waves' 16 x 16 partial logits and per-token maxima meet in LDS.
constexpr int kQgTokens = 16, kQgWaves = 4;
constexpr int kQgSlice = kHidden / kQgWaves;   // 640
constexpr int kQgSteps = kQgSlice / 32;        // 20
// LDS row of a token's codes: 784 bytes = 3 x 256 + 16, so that the 8-byte writes of 16
// tokens x 2 lanes (half a wave) fall on 64 distinct banks.
constexpr int kQgCodePitch = kQgSlice + 144;

__global__ __launch_bounds__(256) void quant_gate_kernel(ProjArgs a) {
  __shared__ float s_gate[kQgWaves][kQgTokens * kGates];
  __shared__ float s_max[kQgWaves][kQgTokens];
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[kQgWaves][kQgTokens][kQgCodePitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kQgTokens;
  const int tr = lane & 15;
  const int t = min(t0 + tr, a.tokens - 1);    // rows past the end re-read the last row
  const int k0 = wave * kQgSlice + 8 * (lane >> 4);
  const uint16_t* xr = a.x + (size_t)t * kHidden + k0;
  const uint16_t* gr = a.w_gate + (size_t)tr * kHidden + k0;
  u32x4 xv[kQgSteps];
#pragma unroll
  for (int s = 0; s < kQgSteps; ++s) xv[s] = ld_global16(xr + 32 * s);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float m = 0.0f;
#pragma unroll
  for (int s = 0; s < kQgSteps; ++s) {
    const u32x4 g = ld_global16(gr + 32 * s);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv[s]), as_bf16x8(g), acc, 0, 0, 0);
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, fmaxf(fabsf(bf16_lo(xv[s][w])), fabsf(bf16_hi(xv[s][w]))));
  }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if (lane < kQgTokens) s_max[wave][lane] = m;
  // Output element v of lane l is logit (token 4 (l / 16) + v, gate l % 16).
#pragma unroll
  for (int v = 0; v < 4; ++v) s_gate[wave][(4 * (lane >> 4) + v) * kGates + tr] = acc[v];
  __syncthreads();
  {
    const int i = threadIdx.x;                   // (token i / 16, gate i % 16)
    const float g = s_gate[0][i] + s_gate[1][i] + s_gate[2][i] + s_gate[3][i];
    if (t0 + i / kGates < a.tokens) a.gate[(size_t)t0 * kGates + i] = (uint16_t)(pack_bf16x2(g, 0.0f) & 0xffffu);
  }
  // Per-token FP8: s = max|x| / 448, codes E4M3FN(x / s), both quotients IEEE fp32.  Per
  // element, x / s is formed as q0 = x * y with y = 1 / s (one IEEE division per token) and
  // one correction, q = q0 + (x - s q0) y in fused multiply-adds (Markstein), with x's
  // sign: an exhaustive check over every bf16 x and every bf16 maximum
  // (tests/test_quant_quotient.py) finds q equal to the IEEE quotient wherever
  // |x / s| >= 2^-10 when s >= 2^-80, and below 2^-10 both give the zero code of x's sign.
  // Tokens with a smaller scale take the division itself.  (160 IEEE divisions per lane
  // took about half of this kernel's time.)
  const float mt = fmaxf(fmaxf(s_max[0][tr], s_max[1][tr]), fmaxf(s_max[2][tr], s_max[3][tr]));
  const float sc = mt / kE4M3Max;
  // A lane's codes are 8-byte pieces of its token's row, 32 bytes apart: they go to LDS
  // first, and the wave then stores its 16 tokens x 640 bytes in 16-byte pieces that run
  // along the rows (each store instruction writes 1 KB in at most three runs instead of 64
  // pieces of 8 bytes).
  uint8_t* const sc_row = &s_codes[wave][tr][8 * (lane >> 4)];
  auto codes = [&](auto quot) {
#pragma unroll
    for (int s = 0; s < kQgSteps; ++s) {
      uint32_t w[2];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t p0 = xv[s][2 * d], p1 = xv[s][2 * d + 1];
        const float y0 = quot(bf16_lo(p0)), y1 = quot(bf16_hi(p0));
        const float y2 = quot(bf16_lo(p1)), y3 = quot(bf16_hi(p1));
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, pk, true);
        w[d] = (uint32_t)pk;
      }
      *reinterpret_cast<u32x2*>(sc_row + 32 * s) = u32x2{w[0], w[1]};
    }
  };
  if (sc >= 0x1p-80f) {
    const float ry = 1.0f / sc;
    codes([&](float x) {
      const float q0 = __fmul_rn(x, ry);
      // x's sign restored: for x = -0 the sums give +0, where x / s is -0 (code 0x80).
      return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-sc, q0, x), ry, q0), x);
    });
  } else {
    codes([&](float x) { return sc > 0.0f ? x / sc : 0.0f; });
  }
  // This wave's LDS writes are done before its reads (one wave's LDS operations execute in
  // order; the barrier keeps the compiler from moving them).
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  constexpr int kChunks = kQgSlice / 16;         // 40 pieces of 16 bytes per token
#pragma unroll
  for (int i = 0; i < kQgTokens * kChunks / 64; ++i) {
    const int f = 64 * i + lane, tok = f / kChunks, c = f % kChunks;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&s_codes[wave][tok][16 * c]);
    if (t0 + tok < a.tokens) st_global16(a.xq + (size_t)(t0 + tok) * kHidden + wave * kQgSlice + 16 * c, v);
  }
  if (wave == 0 && lane < kQgTokens && t0 + tr < a.tokens) a.xs[t] = sc;
}

// ---------------------------------------------------------------------------------------
// FP8 GEMM.  Workgroup tiles of tokens x channels on WM x WN waves, each wave owning
// BMW x BNW blocks of 32 x 32; K in stages of BK bytes (64 or 128) through a ring of S LDS
// stages, each filled S - 1 stages ahead.  In a stage, operand row r holds its BK / 16
// chunks of 16 bytes at r BK + 16 (c ^ swz(r)) with swz(r) = (r / 2) & 7 (BK = 128) or
// (r / 4) & 3 (BK = 64).  LDS serves a 16-byte read 16 lanes at a time over 64 banks
// (256 bytes): the 16 rows such a group reads (one chunk each) then land on 16 distinct
// 16-byte bank groups, 256 / BK rows per bank row times 16 / (256 / BK) swizzle values.
// (With swz(r) = r & 7 at BK = 128, rows r and r + 8 met in one bank group: the counters
// showed half of all LDS cycles as bank conflicts.)  A direct load fills one kilobyte
// (1024 / BK rows) per instruction: lane l writes bytes 16 l .. 16 l + 15 of the block,
// i.e. row l / (BK / 16) of the block and physical chunk l % (BK / 16), so it fetches
// the logical chunk whose swizzled place that is.

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 in the clobber list: nothing else uses it
// Direct global -> LDS load of 16 bytes per lane from a wave-uniform base plus a per-lane
// 32-bit offset, into the 1 KB block at lds_block (lane l fills bytes 16 l .. 16 l + 15).
// Untracked by the compiler: every wait for it is an explicit vmcnt before a barrier.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, void* lds_block) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_block;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_vmcnt0() {
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));   // vmcnt(0), others untouched
}
// This wave's LDS accesses done (its own staged writes visible to its other lanes).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));   // lgkmcnt(0), others untouched
  __builtin_amdgcn_wave_barrier();
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {                // vmcnt <= N, others untouched
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int BK>
__device__ __forceinline__ int swz(int r) { return BK == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }

// Row r, logical 16-byte chunk c of a stage buffer.
template <int BK>
__device__ __forceinline__ const u32x4* stage_chunk(const uint8_t* buf, int r, int c) {
  return reinterpret_cast<const u32x4*>(buf + r * BK + 16 * (c ^ swz<BK>(r)));
}

template <int WM, int WN, int BMW, int BNW, int S, int BK>
struct GemmShape {
  static_assert(BK == 64 || BK == 128, "stage depth");
  static constexpr int kWaves = WM * WN;
  static constexpr int kBM = 32 * BMW * WM, kBN = 32 * BNW * WN;       // workgroup tile
  static constexpr int kChunks = BK / 16, kBlockRows = 1024 / BK;
  static constexpr int kKSteps = kHidden / BK;                          // stages over K
  static constexpr int kXBlocks = kBM / kBlockRows, kWBlocks = kBN / kBlockRows;  // 1 KB blocks
  static constexpr int kLoads = (kXBlocks + kWBlocks) / kWaves;        // per wave and stage
  static constexpr int kXLoads = kXBlocks / kWaves;                    // loads i < kXLoads are X
  static_assert(kXBlocks % kWaves == 0 && kWBlocks % kWaves == 0, "even load split");
  static_assert(kQkvOut % kBN == 0 && kQOut % kBN == 0 && kKvOut % kBN == 0, "tiles inside q, k or v");
};

// Waves WM x WN; each wave owns (32 BMW) x (32 BNW) outputs as BMW x BNW blocks of 32 x 32.
template <int WM, int WN, int BMW, int BNW, int S, int BK>
__global__ __launch_bounds__(64 * WM * WN) void qkv_gemm_kernel(ProjArgs a) {
  using G = GemmShape<WM, WN, BMW, BNW, S, BK>;
  constexpr int kKSteps = G::kKSteps;
  __shared__ __attribute__((aligned(1024))) uint8_t s_x[S][G::kBM * BK];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w[S][G::kBN * BK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int n_tiles = kQkvOut / G::kBN;
  const int n_tile = blockIdx.x % n_tiles;      // consecutive workgroups share the token rows
  const int m0 = (blockIdx.x / n_tiles) * G::kBM;
  const int n0 = n_tile * G::kBN;
  const int T = a.tokens;

  // Load i of this wave fills X block wave + kWaves i (i < kXLoads), else W block
  // wave + kWaves (i - kXLoads): which operand is known at compile time.  Per-lane byte
  // offsets from the operand's base (token rows past the end read the last row; their
  // results are not stored).
  const int lr = lane / G::kChunks;
  uint32_t off[G::kLoads];
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) {
    const int blk = wave + G::kWaves * (i < G::kXLoads ? i : i - G::kXLoads);
    const int lc = (lane % G::kChunks) ^ swz<BK>(G::kBlockRows * blk + lr);   // stage row of this lane
    off[i] = i < G::kXLoads ? (uint32_t)min(m0 + G::kBlockRows * blk + lr, T - 1) * kHidden + 16 * lc
                            : (uint32_t)(n0 + G::kBlockRows * blk + lr) * kHidden + 16 * lc;
  }
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int blk = wave + G::kWaves * (i < G::kXLoads ? i : i - G::kXLoads);
      if (i < G::kXLoads) dma16_s(a.xq + k0, off[i], &s_x[stage][blk * 1024]);
      else dma16_s(a.w + k0, off[i], &s_w[stage][blk * 1024]);
    }
  };

  const int wm = wave % WM, wn = wave / WM;     // this wave's tile
  const int half = lane >> 5, r32 = lane & 31;
  f32x16 acc[BMW][BNW];
#pragma unroll
  for (int i = 0; i < BMW; ++i)
#pragma unroll
    for (int j = 0; j < BNW; ++j) acc[i][j] = f32x16{};

#pragma unroll
  for (int p = 0; p < S - 1; ++p) issue(p, p * BK);
  if constexpr (S == 2) wait_vmcnt0(); else wait_vmcnt<G::kLoads * (S - 2)>();
  __syncthreads();
  auto compute = [&](int st) {
#pragma unroll
    for (int j = 0; j < BK / 64; ++j) {          // MFMA K-steps of 64 bytes per stage
      // Lane l: row l % 32 of a 32-row block, K bytes 32 (l / 32) .. + 31 of the step:
      // logical chunks 4 j + 2 half and + 1 (A and B take the same K order).
      const int c0 = 4 * j + 2 * half;
      i32x8 xf[BMW], wf[BNW];
#pragma unroll
      for (int b = 0; b < BMW; ++b) {
        const int rx = 32 * (BMW * wm + b) + r32;
        const u32x4 x0 = *stage_chunk<BK>(s_x[st], rx, c0), x1 = *stage_chunk<BK>(s_x[st], rx, c0 + 1);
        xf[b] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
#pragma unroll
      for (int b = 0; b < BNW; ++b) {
        const int rw = 32 * (BNW * wn + b) + r32;
        const u32x4 w0 = *stage_chunk<BK>(s_w[st], rw, c0), w1 = *stage_chunk<BK>(s_w[st], rw, c0 + 1);
        wf[b] = i32x8{(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3], (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
      }
#pragma unroll
      for (int bm = 0; bm < BMW; ++bm)
#pragma unroll
        for (int bn = 0; bn < BNW; ++bn)
          acc[bm][bn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xf[bm], wf[bn], acc[bm][bn],
                                                                        0, 0, 0, 127, 0, 127);
    }
  };
  // Main loop: stage ks + S - 1 is issued, stage ks computed; then stage ks + 1 must have
  // landed while the S - 2 stages issued after it may still be in flight.  The wait sits in
  // the same basic block as the MFMAs and behind a scheduling barrier, so that the MFMAs
  // are issued first (hoisted above them, the wait stalls on the next stage before this
  // one is computed).
  int ks = 0;
  for (; ks + S - 1 < kKSteps; ++ks) {
    issue((ks + S - 1) % S, (ks + S - 1) * BK);
    compute(ks % S);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (S > 2) wait_vmcnt<G::kLoads * (S - 2)>(); else wait_vmcnt0();
    __syncthreads();                             // reads of this stage done, next visible
  }
  // The last S - 1 stages are already issued.
  for (; ks < kKSteps; ++ks) {
    compute(ks % S);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt0();
    __syncthreads();
  }

  // Epilogue: C * s_token * s_channel -> bf16, into q, k or v (each tile lies in one).  A
  // wave's accumulators hold 2-byte pieces of rows spread over 32 lanes; stored as they are
  // they make scattered 2-byte writes.  So each wave stages 16 rows x 128 channels at a time
  // in LDS (the operand stages are free after the loop's last barrier) and stores whole
  // 256-byte row pieces with 16-byte non-temporal writes (the outputs are not read again by
  // this kernel; measured 8% faster for the whole call at 32768 tokens than plain stores).
  uint16_t* dst;
  int ld, col0;
  if (n0 < kQOut) { dst = a.q; ld = kQOut; col0 = n0; }
  else if (n0 < kQOut + kKvOut) { dst = a.k; ld = kKvOut; col0 = n0 - kQOut; }
  else { dst = a.v; ld = kKvOut; col0 = n0 - kQOut - kKvOut; }
  static_assert(BNW == 4, "a wave's tile is 128 channels: 256 bytes per staged row");
  // Row pitch 272 bytes: rows 4 apart (the two half-waves) start 16 banks apart.
  constexpr int kEpPitch = 272;
  static_assert(G::kWaves * 16 * kEpPitch <= S * G::kBM * BK, "staging fits in the X stages");
  typedef uint16_t __attribute__((may_alias)) u16_alias;
  typedef u32x4 __attribute__((may_alias)) u32x4_alias;
  uint8_t* const ep = &s_x[0][0] + wave * (16 * kEpPitch);
  float sw[BNW];
#pragma unroll
  for (int bn = 0; bn < BNW; ++bn) sw[bn] = a.w_scale[n0 + 32 * (BNW * wn + bn) + r32];
#pragma unroll
  for (int bm = 0; bm < BMW; ++bm)
#pragma unroll
    for (int p = 0; p < 2; ++p) {              // rows 16 p .. 16 p + 15 of the 32-row block
      const int r0 = m0 + 32 * (BMW * wm + bm) + 16 * p;
#pragma unroll
      for (int u = 0; u < 8; ++u) {            // accumulator element 8 p + u: local row rl
        const int rl = 8 * (u >> 2) + 4 * half + (u & 3);
        const float xs = a.xs[min(r0 + rl, T - 1)];
#pragma unroll
        for (int bn = 0; bn < BNW; ++bn) {
          const float y = acc[bm][bn][8 * p + u] * xs * sw[bn];
          *reinterpret_cast<u16_alias*>(ep + rl * kEpPitch + 2 * (32 * bn + r32)) =
              (uint16_t)(pack_bf16x2(y, 0.0f) & 0xffffu);
        }
      }
      wait_lgkmcnt0();
#pragma unroll
      for (int i = 0; i < 4; ++i) {            // 16 lanes per row, 4 rows per read
        const int rl = 4 * i + (lane >> 4), cc = lane & 15;
        const u32x4 x = *reinterpret_cast<const u32x4_alias*>(ep + rl * kEpPitch + 16 * cc);
        if (r0 + rl < T)
          __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(dst + (size_t)(r0 + rl) * ld + col0 + 128 * wn + 8 * cc));
      }
      wait_lgkmcnt0();                         // staged rows read before the next are written
    }
}

// 256 x 256 workgroup tiles on 4 x 2 waves of 2 x 4 blocks, two 128-byte stages.
using GemmCfg = GemmShape<4, 2, 2, 4, 2, 128>;
constexpr auto kGemmKernel = qkv_gemm_kernel<4, 2, 2, 4, 2, 128>;

}  // namespace

size_t proj_workspace_bytes(int tokens) {
  const size_t codes = ((size_t)tokens * kHidden + 255) & ~(size_t)255;
  return codes + (size_t)tokens * sizeof(float);
}

hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(quant_gate_kernel, dim3((a.tokens + kQgTokens - 1) / kQgTokens), dim3(256), 0, stream, a);
  const int m_tiles = (a.tokens + GemmCfg::kBM - 1) / GemmCfg::kBM;
  hipLaunchKernelGGL(kGemmKernel, dim3(m_tiles * (kQkvOut / GemmCfg::kBN)),
                     dim3(64 * GemmCfg::kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spark
