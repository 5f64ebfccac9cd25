// Kernel argument blocks and launchers behind the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spark {

struct PrefillArgs {
  const uint16_t* q;      // [T, 16, 256]: T = B * S tokens, or the sum of the lengths (varlen)
  const uint16_t* k;      // [T, 4, 256]
  const uint16_t* v;      // [T, 4, 256]
  uint16_t* k_rot;        // [T, 4, 256] workspace: K after RoPE (full layers without a
                          // prefix: only the rotated dims, the rest is read from k)
  const uint16_t* gate;   // [T, 16]
  uint16_t* out;          // [T, 16, 256]
  uint16_t* cache_k;      // [B, cap, 4, 256] or null
  uint16_t* cache_v;
  const int32_t* cu_seqlens;  // [B + 1] token offsets of the sequences (varlen), or null
  int* sched;             // varlen: work-queue counter in the workspace (zeroed by the RoPE pass)
  int total_tokens;       // T
  int batch;
  int seq_len;            // S, or the largest length (varlen)
  int cache_cap;
  int nqb;                // query blocks per sequence (of the largest)
  int start_pos;          // position of the chunk's first token; > 0: prefix in the cache
};

struct AppendArgs {
  const uint16_t* k;      // [B, n_new, 4, 256]
  const uint16_t* v;
  const int32_t* pos;     // [B]
  uint16_t* cache_k;      // [B, cap, 4, 256]
  uint16_t* cache_v;
  int batch;
  int n_new;
  int cache_cap;
};

// 8-bit cache (q8_0 blocks of 32 along head_dim): codes [B, cap, 4, 256] int8, scales
// [B, cap, 4, 8] fp16, for K and for V.
struct AppendQ8Args {
  const uint16_t* k;      // [B, n_new, 4, 256] bf16
  const uint16_t* v;
  const int32_t* pos;     // [B]
  int8_t* k_codes;
  uint16_t* k_scales;
  int8_t* v_codes;
  uint16_t* v_scales;
  int batch;
  int n_new;
  int cache_cap;
};

struct DecodeArgs {
  const uint16_t* q;      // [B, 16, 256]
  const uint16_t* gate;   // [B, 16]
  const uint16_t* cache_k;  // bf16 cache (decode)
  const uint16_t* cache_v;
  const int8_t* k_codes;    // 8-bit cache (decode_q8)
  const uint16_t* k_scales;
  const int8_t* v_codes;
  const uint16_t* v_scales;
  const int32_t* seq_lens;
  int2* ws_range;         // [B] first and last partition touching each sequence
  float* ws_o;            // [P + B, 16, 256] partial results, slot = partition + sequence
  float* ws_ml;           // [P + B, 16, 2] (max, sum) per partial
  uint16_t* out;          // [B, 16, 256]
  int batch;
  int cache_cap;
  int nparts;             // P
};

// W8A8 FP8 q_k_v_proj and bf16 g_proj of T tokens.
struct ProjArgs {
  const uint16_t* x;        // [T, 2560] bf16 hidden states
  const uint8_t* w;         // [6144, 2560] E4M3FN codes (rows: q 0..4095, k .., v ..)
  const float* w_scale;     // [6144] per output channel
  const uint16_t* w_gate;   // [16, 2560] bf16
  uint8_t* xq;              // [T, 2560] workspace: E4M3FN codes of the activations
  float* xs;                // [T] workspace: per-token scales
  uint16_t* q;              // [T, 16, 256] bf16
  uint16_t* k;              // [T, 4, 256]
  uint16_t* v;              // [T, 4, 256]
  uint16_t* gate;           // [T, 16]
  int tokens;
};

hipError_t launch_prefill(int layer_type, const PrefillArgs& a, hipStream_t stream);
hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t stream);
size_t proj_workspace_bytes(int tokens);
hipError_t launch_append(int layer_type, const AppendArgs& a, hipStream_t stream);
hipError_t launch_decode(int layer_type, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_append_q8(int layer_type, const AppendQ8Args& a, hipStream_t stream);
hipError_t launch_decode_q8(int layer_type, const DecodeArgs& a, hipStream_t stream);

int prefill_block_rows();
size_t prefill_workspace_bytes(int batch, int seq_len);

// Decode planning, shared by the workspace query and the decode call.
// Workspace regions are byte offsets from its start, each 256-byte aligned.
struct DecodePlan {
  int nparts;
  size_t range_offset;
  size_t o_offset;
  size_t ml_offset;
  size_t total_bytes;
};
DecodePlan plan_decode(int layer_type, int batch, int max_seq_len, int nparts, bool q8 = false);

// Static device scratch of spark_attn_decode_noalloc: its size, and its device address on
// the current device (looked up on the first call per device).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch(void** ptr);

}  // namespace spark
