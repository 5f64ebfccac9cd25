// extern "C" entry points declared in include/spark_attn.h: host-side argument checks,
// then the launches (prefill two or three, append one, decode two) on the caller's stream.  Every check
// runs before any HIP call, so a rejected call enqueues nothing and touches no device.
#include "spark_attn.h"
#include "spark_device.hpp"
#include "spark_launch.hpp"

namespace {

constexpr int32_t kMaxBatch = 65535;
constexpr int32_t kMaxSeq = 1 << 20;   // native context of the model: 1,048,576 positions
constexpr int32_t kMaxParts = 1 << 20; // decode partitions (workgroups of the attention launch)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }
bool valid_type(int32_t lt) { return lt == SPARK_LAYER_SLIDING || lt == SPARK_LAYER_FULL; }

spark_status check_cache(int32_t lt, const spark_kv_cache* c, int32_t batch) {
  if (!c || !c->k || !c->v) return SPARK_ERR_INVALID_ARG;
  if (!aligned16(c->k) || !aligned16(c->v)) return SPARK_ERR_INVALID_ARG;
  if (c->batch != batch || c->capacity < 1) return SPARK_ERR_INVALID_ARG;
  if (lt == SPARK_LAYER_SLIDING && c->capacity != SPARK_WINDOW) return SPARK_ERR_INVALID_ARG;
  return SPARK_OK;
}

spark_status check_cache_q8(int32_t lt, const spark_kv_cache_q8* c, int32_t batch) {
  if (!c || !c->k || !c->v || !c->k_scale || !c->v_scale) return SPARK_ERR_INVALID_ARG;
  if (!aligned16(c->k) || !aligned16(c->v) || !aligned16(c->k_scale) || !aligned16(c->v_scale))
    return SPARK_ERR_INVALID_ARG;
  if (c->batch != batch || c->capacity < 1) return SPARK_ERR_INVALID_ARG;
  if (lt == SPARK_LAYER_SLIDING && c->capacity != SPARK_WINDOW) return SPARK_ERR_INVALID_ARG;
  return SPARK_OK;
}

spark_status from_hip(hipError_t e) { return e == hipSuccess ? SPARK_OK : SPARK_ERR_HIP; }

// Varlen workspace: the rotated keys, then (256-byte aligned) the work-queue counter.
size_t varlen_queue_offset(int32_t total_tokens) {
  return (spark::prefill_workspace_bytes(1, total_tokens) + 255) & ~(size_t)255;
}

// Checks shared by the decode entry points (everything but the cache and the workspace).
spark_status check_decode_io(int32_t layer_type, int32_t batch, const void* q, const void* gate_logits,
                             const int32_t* seq_lens, int32_t max_seq_len, int32_t num_parts,
                             const void* out) {
  if (!valid_type(layer_type)) return SPARK_ERR_INVALID_ARG;
  if (batch < 1 || batch > kMaxBatch || max_seq_len < 1 || max_seq_len > kMaxSeq) return SPARK_ERR_INVALID_ARG;
  if (num_parts < 0 || num_parts > kMaxParts) return SPARK_ERR_INVALID_ARG;
  if (!q || !gate_logits || !seq_lens || !out) return SPARK_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned2(gate_logits) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return SPARK_ERR_INVALID_ARG;
  return SPARK_OK;
}

// ... and the caller's workspace of spark_attn_decode and spark_attn_decode_q8.
spark_status check_decode(int32_t layer_type, int32_t batch, const void* q, const void* gate_logits,
                          const int32_t* seq_lens, int32_t max_seq_len, int32_t num_parts,
                          const void* workspace, const void* out) {
  const spark_status st = check_decode_io(layer_type, batch, q, gate_logits, seq_lens, max_seq_len, num_parts, out);
  if (st != SPARK_OK) return st;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return SPARK_ERR_INVALID_ARG;
  return SPARK_OK;
}

// Decode arguments after the checks: the workspace regions of the plan.
spark::DecodeArgs decode_args(const spark::DecodePlan& plan, int32_t batch, int32_t cap, const void* q,
                              const void* gate_logits, const int32_t* seq_lens, void* workspace,
                              void* out) {
  char* ws = static_cast<char*>(workspace);
  spark::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.gate = static_cast<const uint16_t*>(gate_logits);
  a.seq_lens = seq_lens;
  a.ws_range = reinterpret_cast<int2*>(ws + plan.range_offset);
  a.ws_o = reinterpret_cast<float*>(ws + plan.o_offset);
  a.ws_ml = reinterpret_cast<float*>(ws + plan.ml_offset);
  a.out = static_cast<uint16_t*>(out);
  a.batch = batch;
  a.cache_cap = cap;
  a.nparts = plan.nparts;
  return a;
}

}  // namespace

extern "C" {

int32_t spark_abi_version(void) { return SPARK_ATTN_ABI_VERSION; }

int32_t spark_layer_type_of(int32_t layer) {
  if (layer < 0 || layer >= SPARK_N_LAYERS) return -1;
  return layer % 4 == 3 ? SPARK_LAYER_FULL : SPARK_LAYER_SLIDING;
}

int32_t spark_layer_params(int32_t layer_type, double* rope_theta, int32_t* rotary_dims, int32_t* window) {
  if (!valid_type(layer_type)) return SPARK_ERR_INVALID_ARG;
  const bool full = layer_type == SPARK_LAYER_FULL;
  if (rope_theta) *rope_theta = full ? spark::LayerTraits<spark::kFull>::kTheta : spark::LayerTraits<spark::kSliding>::kTheta;
  if (rotary_dims) *rotary_dims = full ? spark::LayerTraits<spark::kFull>::kRot : spark::LayerTraits<spark::kSliding>::kRot;
  if (window) *window = full ? 0 : spark::kWindow;
  return SPARK_OK;
}

const char* spark_status_string(int32_t s) {
  switch (s) {
    case SPARK_OK: return "ok";
    case SPARK_ERR_INVALID_ARG: return "invalid argument";
    case SPARK_ERR_UNSUPPORTED: return "unsupported request";
    case SPARK_ERR_WORKSPACE: return "workspace too small";
    case SPARK_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

size_t spark_attn_prefill_workspace_bytes(int32_t layer_type, int32_t batch, int32_t seq_len) {
  if (!valid_type(layer_type) || batch < 1 || batch > kMaxBatch || seq_len < 1 || seq_len > kMaxSeq ||
      (long long)batch * seq_len > 0xfffffffeLL)
    return 0;
  return spark::prefill_workspace_bytes(batch, seq_len);
}

spark_status spark_attn_prefill(int32_t layer_type, int32_t batch, int32_t seq_len,
                                int32_t start_pos, const void* q, const void* k,
                                const void* v, const void* gate_logits,
                                const spark_kv_cache* cache, void* workspace,
                                size_t workspace_bytes, void* out, void* stream) {
  if (!valid_type(layer_type)) return SPARK_ERR_INVALID_ARG;
  if (batch < 1 || batch > kMaxBatch || seq_len < 1 || seq_len > kMaxSeq) return SPARK_ERR_INVALID_ARG;
  // The RoPE pass runs one thread per 16-byte K chunk, 128 per token, 256 per workgroup;
  // the attention grid has ceil(seq_len / 64) * batch * 4 workgroups.
  if ((long long)batch * seq_len > 0xfffffffeLL) return SPARK_ERR_INVALID_ARG;
  if (!q || !k || !v || !gate_logits || !out) return SPARK_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned2(gate_logits))
    return SPARK_ERR_INVALID_ARG;
  if (start_pos < 0 || (long long)start_pos + seq_len > kMaxSeq) return SPARK_ERR_INVALID_ARG;
  if (start_pos > 0 && !cache) return SPARK_ERR_INVALID_ARG;   // the prefix is read from the cache
  if (cache) {
    const spark_status cs = check_cache(layer_type, cache, batch);
    if (cs != SPARK_OK) return cs;
    if (layer_type == SPARK_LAYER_FULL && (long long)cache->capacity < (long long)start_pos + seq_len)
      return SPARK_ERR_INVALID_ARG;
  }
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return SPARK_ERR_INVALID_ARG;
  if (workspace_bytes < spark::prefill_workspace_bytes(batch, seq_len)) return SPARK_ERR_WORKSPACE;
  const int rows = spark::prefill_block_rows();
  const long long nqb = (seq_len + rows - 1) / rows;

  spark::PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_rot = static_cast<uint16_t*>(workspace);
  a.gate = static_cast<const uint16_t*>(gate_logits);
  a.out = static_cast<uint16_t*>(out);
  a.cache_k = cache ? static_cast<uint16_t*>(cache->k) : nullptr;
  a.cache_v = cache ? static_cast<uint16_t*>(cache->v) : nullptr;
  a.cu_seqlens = nullptr;
  a.total_tokens = batch * seq_len;
  a.batch = batch;
  a.seq_len = seq_len;
  a.cache_cap = cache ? cache->capacity : 0;
  a.nqb = (int)nqb;
  a.start_pos = start_pos;
  return from_hip(spark::launch_prefill(layer_type, a, static_cast<hipStream_t>(stream)));
}

size_t spark_attn_prefill_varlen_workspace_bytes(int32_t layer_type, int32_t total_tokens) {
  if (!valid_type(layer_type) || total_tokens < 1) return 0;
  return varlen_queue_offset(total_tokens) + 256;
}

spark_status spark_attn_prefill_varlen(int32_t layer_type, int32_t batch, const int32_t* cu_seqlens,
                                       int32_t total_tokens, int32_t max_seqlen, const void* q,
                                       const void* k, const void* v, const void* gate_logits,
                                       const spark_kv_cache* cache, void* workspace,
                                       size_t workspace_bytes, void* out, void* stream) {
  if (!valid_type(layer_type)) return SPARK_ERR_INVALID_ARG;
  if (batch < 1 || batch > kMaxBatch || max_seqlen < 1 || max_seqlen > kMaxSeq || total_tokens < 1)
    return SPARK_ERR_INVALID_ARG;
  // Grid as for a uniform batch of max_seqlen: ceil(max_seqlen / 64) * batch * 4 workgroups.
  if ((long long)batch * max_seqlen > 0xfffffffeLL) return SPARK_ERR_INVALID_ARG;
  if (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return SPARK_ERR_INVALID_ARG;
  if (!q || !k || !v || !gate_logits || !out) return SPARK_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned2(gate_logits))
    return SPARK_ERR_INVALID_ARG;
  if (cache) {
    const spark_status cs = check_cache(layer_type, cache, batch);
    if (cs != SPARK_OK) return cs;
    if (layer_type == SPARK_LAYER_FULL && cache->capacity < max_seqlen) return SPARK_ERR_INVALID_ARG;
  }
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return SPARK_ERR_INVALID_ARG;
  if (workspace_bytes < varlen_queue_offset(total_tokens) + 256) return SPARK_ERR_WORKSPACE;
  const int rows = spark::prefill_block_rows();

  spark::PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_rot = static_cast<uint16_t*>(workspace);
  a.gate = static_cast<const uint16_t*>(gate_logits);
  a.out = static_cast<uint16_t*>(out);
  a.cache_k = cache ? static_cast<uint16_t*>(cache->k) : nullptr;
  a.cache_v = cache ? static_cast<uint16_t*>(cache->v) : nullptr;
  a.cu_seqlens = cu_seqlens;
  a.sched = reinterpret_cast<int*>(static_cast<char*>(workspace) + varlen_queue_offset(total_tokens));
  a.total_tokens = total_tokens;
  a.batch = batch;
  a.seq_len = max_seqlen;
  a.cache_cap = cache ? cache->capacity : 0;
  a.nqb = (max_seqlen + rows - 1) / rows;
  a.start_pos = 0;
  return from_hip(spark::launch_prefill(layer_type, a, static_cast<hipStream_t>(stream)));
}

size_t spark_qkv_proj_fp8_workspace_bytes(int32_t tokens) {
  if (tokens < 1 || tokens > kMaxSeq) return 0;
  return spark::proj_workspace_bytes(tokens);
}

spark_status spark_qkv_proj_fp8(int32_t tokens, const void* x, const void* w_qkv, const float* w_scale,
                                const void* w_gate, void* q, void* k, void* v, void* gate_logits,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (tokens < 1 || tokens > kMaxSeq) return SPARK_ERR_INVALID_ARG;
  if (!x || !w_qkv || !w_scale || !w_gate || !q || !k || !v || !gate_logits || !workspace)
    return SPARK_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(w_gate) || !aligned16(q) || !aligned16(k) ||
      !aligned16(v) || !aligned2(gate_logits) || (reinterpret_cast<uintptr_t>(w_scale) & 3u) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return SPARK_ERR_INVALID_ARG;
  if (workspace_bytes < spark::proj_workspace_bytes(tokens)) return SPARK_ERR_WORKSPACE;
  spark::ProjArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint8_t*>(w_qkv);
  a.w_scale = w_scale;
  a.w_gate = static_cast<const uint16_t*>(w_gate);
  a.xq = static_cast<uint8_t*>(workspace);
  a.xs = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                  (((size_t)tokens * 2560 + 255) & ~(size_t)255));
  a.q = static_cast<uint16_t*>(q);
  a.k = static_cast<uint16_t*>(k);
  a.v = static_cast<uint16_t*>(v);
  a.gate = static_cast<uint16_t*>(gate_logits);
  a.tokens = tokens;
  return from_hip(spark::launch_qkv_proj(a, static_cast<hipStream_t>(stream)));
}

spark_status spark_kv_append(int32_t layer_type, int32_t batch, int32_t n_new,
                             const void* k, const void* v, const int32_t* pos,
                             const spark_kv_cache* cache, void* stream) {
  if (!valid_type(layer_type)) return SPARK_ERR_INVALID_ARG;
  if (batch < 1 || batch > kMaxBatch || n_new < 1 || n_new > kMaxSeq) return SPARK_ERR_INVALID_ARG;
  if (!k || !v || !pos) return SPARK_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || (reinterpret_cast<uintptr_t>(pos) & 3u)) return SPARK_ERR_INVALID_ARG;
  const spark_status cs = check_cache(layer_type, cache, batch);
  if (cs != SPARK_OK) return cs;

  spark::AppendArgs a{};
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.pos = pos;
  a.cache_k = static_cast<uint16_t*>(cache->k);
  a.cache_v = static_cast<uint16_t*>(cache->v);
  a.batch = batch;
  a.n_new = n_new;
  a.cache_cap = cache->capacity;
  return from_hip(spark::launch_append(layer_type, a, static_cast<hipStream_t>(stream)));
}

size_t spark_attn_decode_workspace_bytes(int32_t layer_type, int32_t batch, int32_t max_seq_len,
                                         int32_t num_parts) {
  if (!valid_type(layer_type) || batch < 1 || batch > kMaxBatch || max_seq_len < 1 ||
      max_seq_len > kMaxSeq || num_parts < 0 || num_parts > kMaxParts)
    return 0;
  return spark::plan_decode(layer_type, batch, max_seq_len, num_parts).total_bytes;
}

spark_status spark_attn_decode(int32_t layer_type, int32_t batch, const void* q,
                               const void* gate_logits, const spark_kv_cache* cache,
                               const int32_t* seq_lens, int32_t max_seq_len,
                               int32_t num_parts, void* workspace,
                               size_t workspace_bytes, void* out, void* stream) {
  spark_status st = check_decode(layer_type, batch, q, gate_logits, seq_lens, max_seq_len, num_parts,
                                 workspace, out);
  if (st != SPARK_OK) return st;
  st = check_cache(layer_type, cache, batch);
  if (st != SPARK_OK) return st;
  if (layer_type == SPARK_LAYER_FULL && max_seq_len > cache->capacity) return SPARK_ERR_INVALID_ARG;
  // Planned on max_seq_len (not the capacity), exactly as the workspace query plans it.
  const spark::DecodePlan plan = spark::plan_decode(layer_type, batch, max_seq_len, num_parts);
  if (workspace_bytes < plan.total_bytes) return SPARK_ERR_WORKSPACE;
  spark::DecodeArgs a = decode_args(plan, batch, cache->capacity, q, gate_logits, seq_lens, workspace, out);
  a.cache_k = static_cast<const uint16_t*>(cache->k);
  a.cache_v = static_cast<const uint16_t*>(cache->v);
  return from_hip(spark::launch_decode(layer_type, a, static_cast<hipStream_t>(stream)));
}

spark_status spark_attn_decode_noalloc(int32_t layer_type, int32_t batch, const void* q,
                                       const void* gate_logits, const spark_kv_cache* cache,
                                       const int32_t* seq_lens, int32_t max_seq_len,
                                       int32_t num_parts, void* out, void* stream) {
  spark_status st = check_decode_io(layer_type, batch, q, gate_logits, seq_lens, max_seq_len, num_parts, out);
  if (st != SPARK_OK) return st;
  st = check_cache(layer_type, cache, batch);
  if (st != SPARK_OK) return st;
  if (layer_type == SPARK_LAYER_FULL && max_seq_len > cache->capacity) return SPARK_ERR_INVALID_ARG;
  const spark::DecodePlan plan = spark::plan_decode(layer_type, batch, max_seq_len, num_parts);
  if (plan.total_bytes > spark::kStaticScratchBytes) return SPARK_ERR_WORKSPACE;
  void* ws = nullptr;
  if (spark::static_scratch(&ws) != hipSuccess) return SPARK_ERR_HIP;
  spark::DecodeArgs a = decode_args(plan, batch, cache->capacity, q, gate_logits, seq_lens, ws, out);
  a.cache_k = static_cast<const uint16_t*>(cache->k);
  a.cache_v = static_cast<const uint16_t*>(cache->v);
  return from_hip(spark::launch_decode(layer_type, a, static_cast<hipStream_t>(stream)));
}

spark_status spark_kv_append_q8(int32_t layer_type, int32_t batch, int32_t n_new,
                                const void* k, const void* v, const int32_t* pos,
                                const spark_kv_cache_q8* cache, void* stream) {
  if (!valid_type(layer_type)) return SPARK_ERR_INVALID_ARG;
  if (batch < 1 || batch > kMaxBatch || n_new < 1 || n_new > kMaxSeq) return SPARK_ERR_INVALID_ARG;
  if (!k || !v || !pos) return SPARK_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || (reinterpret_cast<uintptr_t>(pos) & 3u)) return SPARK_ERR_INVALID_ARG;
  const spark_status cs = check_cache_q8(layer_type, cache, batch);
  if (cs != SPARK_OK) return cs;

  spark::AppendQ8Args a{};
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.pos = pos;
  a.k_codes = static_cast<int8_t*>(cache->k);
  a.k_scales = static_cast<uint16_t*>(cache->k_scale);
  a.v_codes = static_cast<int8_t*>(cache->v);
  a.v_scales = static_cast<uint16_t*>(cache->v_scale);
  a.batch = batch;
  a.n_new = n_new;
  a.cache_cap = cache->capacity;
  return from_hip(spark::launch_append_q8(layer_type, a, static_cast<hipStream_t>(stream)));
}

size_t spark_attn_decode_q8_workspace_bytes(int32_t layer_type, int32_t batch, int32_t max_seq_len,
                                            int32_t num_parts) {
  if (!valid_type(layer_type) || batch < 1 || batch > kMaxBatch || max_seq_len < 1 ||
      max_seq_len > kMaxSeq || num_parts < 0 || num_parts > kMaxParts)
    return 0;
  return spark::plan_decode(layer_type, batch, max_seq_len, num_parts, true).total_bytes;
}

spark_status spark_attn_decode_q8(int32_t layer_type, int32_t batch, const void* q,
                                  const void* gate_logits, const spark_kv_cache_q8* cache,
                                  const int32_t* seq_lens, int32_t max_seq_len,
                                  int32_t num_parts, void* workspace,
                                  size_t workspace_bytes, void* out, void* stream) {
  spark_status st = check_decode(layer_type, batch, q, gate_logits, seq_lens, max_seq_len, num_parts,
                                 workspace, out);
  if (st != SPARK_OK) return st;
  st = check_cache_q8(layer_type, cache, batch);
  if (st != SPARK_OK) return st;
  if (layer_type == SPARK_LAYER_FULL && max_seq_len > cache->capacity) return SPARK_ERR_INVALID_ARG;
  const spark::DecodePlan plan = spark::plan_decode(layer_type, batch, max_seq_len, num_parts, true);
  if (workspace_bytes < plan.total_bytes) return SPARK_ERR_WORKSPACE;
  spark::DecodeArgs a = decode_args(plan, batch, cache->capacity, q, gate_logits, seq_lens, workspace, out);
  a.k_codes = static_cast<const int8_t*>(cache->k);
  a.k_scales = static_cast<const uint16_t*>(cache->k_scale);
  a.v_codes = static_cast<const int8_t*>(cache->v);
  a.v_scales = static_cast<const uint16_t*>(cache->v_scale);
  return from_hip(spark::launch_decode_q8(layer_type, a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
