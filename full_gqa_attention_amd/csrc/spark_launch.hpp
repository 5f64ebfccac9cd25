// Kernel argument blocks and launchers behind the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spark {

struct PrefillArgs {
  const uint16_t* q;      // [B, S, 16, 256]
  const uint16_t* k;      // [B, S, 4, 256]
  const uint16_t* v;      // [B, S, 4, 256]
  const uint16_t* gate;   // [B, S, 16]
  uint16_t* out;          // [B, S, 16, 256]
  uint16_t* cache_k;      // [B, cap, 4, 256] or null
  uint16_t* cache_v;
  int batch;
  int seq_len;
  int cache_cap;
  int nqb;                // query blocks per sequence
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

struct DecodeArgs {
  const uint16_t* q;      // [B, 16, 256]
  const uint16_t* gate;   // [B, 16]
  const uint16_t* cache_k;
  const uint16_t* cache_v;
  const int32_t* seq_lens;
  float* ws_o;            // [B, nsplit, 16, 256]
  float* ws_ml;           // [B, nsplit, 16, 2]
  uint16_t* out;          // [B, 16, 256]
  int batch;
  int cache_cap;
  int nsplit;
  int split_keys;
};

hipError_t launch_prefill(int layer_type, const PrefillArgs& a, hipStream_t stream);
hipError_t launch_append(int layer_type, const AppendArgs& a, hipStream_t stream);
hipError_t launch_decode(int layer_type, const DecodeArgs& a, hipStream_t stream);

int prefill_block_rows();

// Decode planning, shared by the workspace query and the decode call.
struct DecodePlan {
  int split_keys;
  int nsplit;
  size_t ws_o_bytes;
  size_t ws_ml_bytes;
  size_t total_bytes;
};
DecodePlan plan_decode(int layer_type, int batch, int max_seq_len, int split_keys);

}  // namespace spark
