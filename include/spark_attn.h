/*
 * spark_attn.h -- C ABI of the hybrid sliding/full GQA attention path on AMD Instinct
 * MI355X (gfx950).
 *
 * The model (Spark-X2.5/X2.6-4B family) stacks 36 attention layers: three sliding-window
 * layers, then one full-attention layer, nine times over, so the last layer is full
 * (Spark-X2.6-4B-Base hybrid attention explainer, eliteato.com/news/34565, section
 * "36 层混合注意力排布").  Every layer has 16 query heads over 4 KV heads of dimension 256
 * (same page, section "配套效率设计"; Spark-X2.6-4B-FP8 walkthrough, nxmr.cn/news/148448,
 * section 一, config table).
 *
 *   layer type | RoPE theta | rotated dims      | keys visible to query i
 *   -----------+------------+-------------------+-------------------------
 *   SLIDING    | 1e4        | all 256           | i-512 < j <= i
 *   FULL       | 5e6        | first 64 (of 256) | j <= i
 *
 * (explainer page, sections "滑动窗口 512" and "全局注意力 5M 基频 RoPE" with its
 * parameter table).  RoPE pairs element m with element m + r/2 of the rotated slice of
 * width r, angle p * theta^(-2m/r).  Scores are scaled by 1/16 = 1/sqrt(256), the
 * softmax runs in fp32 (Spark X2.5-4B F16 vs Q4 comparison, hotelren.com/news/5475707,
 * section 三) and each head's output is multiplied by sigmoid(gate logit) of that head
 * and token (same section; explainer page, section "配套效率设计").  Query head h reads
 * KV head h / 4.
 *
 * Conventions of every call
 *  - All tensors are bf16, row-major, innermost dimension contiguous, in device memory
 *    the caller owns (allocated e.g. through PyTorch).  The library allocates nothing and
 *    keeps no state between calls; calls on disjoint buffers may run concurrently.
 *  - Every pointer to a bf16 tensor must be 16-byte aligned.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and outputs are
 *    valid once that stream has reached the work.  Nothing synchronises the host.
 *  - Host-side argument checks run before anything is enqueued; on failure nothing is
 *    enqueued and the status says why.  Values that live in device memory (`pos`,
 *    `seq_lens`) cannot be checked: out-of-range values are undefined behaviour.
 *  - SPARK_ERR_HIP reports a failed launch (hipGetLastError after the launch).
 */
#ifndef SPARK_ATTN_H
#define SPARK_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARK_ATTN_ABI_VERSION 8

enum { SPARK_Q_HEADS = 16, SPARK_KV_HEADS = 4, SPARK_HEAD_DIM = 256, SPARK_WINDOW = 512,
       SPARK_N_LAYERS = 36 };

typedef enum spark_layer_type {
  SPARK_LAYER_SLIDING = 0,
  SPARK_LAYER_FULL = 1
} spark_layer_type;

typedef enum spark_status {
  SPARK_OK = 0,
  SPARK_ERR_INVALID_ARG = 1, /* null pointer, bad enum, size out of range, misaligned */
  SPARK_ERR_UNSUPPORTED = 2, /* a valid request this build does not implement        */
  SPARK_ERR_WORKSPACE = 3,   /* workspace smaller than required                      */
  SPARK_ERR_HIP = 4          /* the HIP runtime reported a launch failure            */
} spark_status;

/*
 * Type of 0-based layer `layer` of the 36-layer stack: three sliding-window layers, then one
 * full-attention layer, nine times over, so the last layer (35) is full (Spark-X2.6-4B-Base
 * hybrid attention explainer, eliteato.com/news/34565, section "36 层混合注意力排布";
 * Spark-X2.6-4B config.json guide, lqnn.cn/news/248463, section "混合注意力").
 * Returns SPARK_LAYER_FULL when layer mod 4 == 3, SPARK_LAYER_SLIDING for the other layers
 * of 0..35, and -1 for a layer outside 0..35.  Pure function of its argument.
 */
int32_t spark_layer_type_of(int32_t layer);

/*
 * RoPE base, rotated width and window of a layer type (explainer page, parameter table of
 * section "全局注意力 5M 基频 RoPE", and section "滑动窗口 512"): SLIDING 1e4, 256 dims,
 * window 512; FULL 5e6, the first 64 dims (partial_rotary_factor 0.25), no window
 * (*window = 0).  Any output pointer may be NULL.  SPARK_ERR_INVALID_ARG for an unknown
 * type, with nothing written.
 */
int32_t spark_layer_params(int32_t layer_type, double* rope_theta, int32_t* rotary_dims,
                           int32_t* window);

/*
 * KV cache of one layer, for `batch` sequences.  The keys are stored after RoPE, the
 * values as given, both bf16 [batch, capacity, 4, 256].
 *  - FULL layer: contiguous; position p of a sequence lives in slot p (p < capacity).
 *    4 KB per token per layer (F16 vs Q4 comparison page, section 一).
 *  - SLIDING layer: a ring of capacity == 512 slots; position p lives in slot p mod 512,
 *    so a new token replaces exactly the key that just left the window, and the layer's
 *    footprint stays 2 MiB per sequence whatever the context (Sharp-Spark-X2.5-4B-GGUF
 *    guide, mpbf.cn/news/67460, section 三).
 */
typedef struct spark_kv_cache {
  void* k;
  void* v;
  int32_t batch;
  int32_t capacity;
} spark_kv_cache;

/*
 * Bytes of device workspace spark_attn_prefill needs: the rotated keys,
 * bf16 [batch, seq_len, 4, 256].  Returns 0 for sizes spark_attn_prefill would reject.
 */
size_t spark_attn_prefill_workspace_bytes(int32_t layer_type, int32_t batch, int32_t seq_len);

/*
 * Prefill of one layer (Spark-X2.6-4B-Base hybrid attention explainer, eliteato.com/news/34565:
 * masks per layer type in section "36 层混合注意力排布", the 512-token band in "滑动窗口 512",
 * RoPE per type in "全局注意力 5M 基频 RoPE", GQA and the head gate in "配套效率设计"; fp32
 * softmax and the sigmoid gate: Spark X2.5-4B F16 vs Q4 comparison, hotelren.com/news/5475707,
 * section 三).
 *
 * Attention of a chunk of `seq_len` new tokens per sequence, one layer, over
 * the chunk itself and, when start_pos > 0, over the start_pos earlier tokens already
 * in the cache (chunked prefill).  Token t of a sequence sits at position start_pos + t
 * and sees the keys at positions <= start_pos + t (SLIDING: the last 512 of them).
 *   q            bf16 [batch, seq_len, 16, 256], before RoPE
 *   k, v         bf16 [batch, seq_len, 4, 256], k before RoPE
 *   gate_logits  bf16 [batch, seq_len, 16]
 *   cache        optional when start_pos == 0 (NULL = none), required otherwise.  Read:
 *                positions 0..start_pos-1 (FULL, slot p) or max(0, start_pos-512) ..
 *                start_pos-1 (SLIDING, slot p mod 512), as spark_kv_append or an earlier
 *                prefill left them.  Written: the chunk's rotated keys and values at
 *                positions start_pos .. start_pos+seq_len-1 (SLIDING: only the last 512
 *                of them, in their ring slots).  cache->batch must equal batch; FULL
 *                needs capacity >= start_pos + seq_len.
 *   workspace    device scratch of at least spark_attn_prefill_workspace_bytes(...)
 *                bytes, 256-byte aligned, used only during the call (calls sharing one
 *                workspace must be ordered on a stream); SPARK_ERR_WORKSPACE if smaller
 *   out          bf16 [batch, seq_len, 16, 256] (written)
 *   start_pos    position of the chunk's first token, 0 <= start_pos, start_pos +
 *                seq_len <= 2^20; every sequence of the batch starts at it.
 * 1 <= seq_len <= 2^20, 1 <= batch <= 65535, batch * seq_len < 2^32.  Launches: RoPE of
 * K into the workspace (and the cache writes), then the attention with the sigmoid head
 * gate; a SLIDING chunk with start_pos > 0 writes its ring slots in a third launch, after
 * the attention has read the prefix from them.
 */
spark_status spark_attn_prefill(int32_t layer_type, int32_t batch, int32_t seq_len,
                                int32_t start_pos, const void* q, const void* k,
                                const void* v, const void* gate_logits,
                                const spark_kv_cache* cache, void* workspace,
                                size_t workspace_bytes, void* out, void* stream);

/*
 * Bytes of device workspace spark_qkv_proj_fp8 needs: the activations' FP8 codes
 * [tokens, 2560] (padded to 256 bytes), then their per-token scales fp32 [tokens].
 */
size_t spark_qkv_proj_fp8_workspace_bytes(int32_t tokens);

/*
 * The projections that feed the attention, for `tokens` hidden states (Spark-X2.6-4B-FP8
 * walkthrough, nxmr.cn/news/148448, sections 二 and 三): q_k_v_proj in W8A8 FP8 and g_proj
 * in BF16, hidden 2560 (section 一).
 *   x            bf16 [tokens, 2560]
 *   w_qkv        OCP FP8 E4M3FN codes [6144, 2560]: output channels 0..4095 are q (head h
 *                at 256h..256h+255), 4096..5119 k, 5120..6143 v
 *   w_scale      fp32 [6144]: one scale per output channel (quantised offline)
 *   w_gate       bf16 [16, 2560]
 *   q, k, v      bf16 [tokens, 16, 256], [tokens, 4, 256], [tokens, 4, 256] (written):
 *                the layouts spark_attn_prefill takes, before RoPE
 *   gate_logits  bf16 [tokens, 16] (written)
 *   workspace    >= spark_qkv_proj_fp8_workspace_bytes(tokens), 256-byte aligned
 * Per token: s = max|x| / 448 and codes E4M3FN(x / s), nearest even (fp32 divisions);
 * y = s * w_scale[n] * sum_k code_x * code_w (fp32 accumulation), rounded to bf16; gate =
 * x w_gate^T from the bf16 values, fp32 accumulation.  1 <= tokens <= 2^20; x, w_qkv,
 * w_gate, q, k, v 16-byte aligned.  Two launches: quantisation with the gate projection,
 * then the FP8 GEMM on MFMA.
 */
spark_status spark_qkv_proj_fp8(int32_t tokens, const void* x, const void* w_qkv, const float* w_scale,
                                const void* w_gate, void* q, void* k, void* v, void* gate_logits,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace spark_attn_prefill_varlen needs: bf16 [total_tokens, 4, 256],
 * then (256-byte aligned) a 256-byte block holding the work queue of the attention launch. */
size_t spark_attn_prefill_varlen_workspace_bytes(int32_t layer_type, int32_t total_tokens);

/*
 * Prefill of a variable-length batch: the masks, RoPE and gate of spark_attn_prefill (same
 * passages of the hybrid attention explainer), applied to each sequence on its own.
 *
 * Sequences of different lengths are packed one after another
 * (variable-length batch): sequence b owns token rows cu_seqlens[b] .. cu_seqlens[b+1]-1
 * and its token t sits at position t; each sequence attends only to itself.
 *   cu_seqlens   device int32 [batch + 1]: 0 = cu[0] <= cu[1] <= ... <= cu[batch] =
 *                total_tokens, every length <= max_seqlen (zero lengths allowed).  The
 *                host cannot check device contents: a table that breaks these rules gives
 *                unspecified outputs for the rows concerned, but every access stays inside
 *                the buffers (the kernels clamp each sequence to [0, total_tokens) and to
 *                max_seqlen rows).
 *   q, out       bf16 [total_tokens, 16, 256];  k, v  bf16 [total_tokens, 4, 256], k
 *                before RoPE;  gate_logits  bf16 [total_tokens, 16]
 *   cache        optional, as for spark_attn_prefill with start_pos = 0 (row b receives
 *                sequence b's rotated keys and values); FULL needs capacity >= max_seqlen
 *   workspace    >= spark_attn_prefill_varlen_workspace_bytes(layer_type, total_tokens),
 *                256-byte aligned
 * 1 <= batch <= 65535, 1 <= max_seqlen <= 2^20, batch * max_seqlen < 2^32,
 * total_tokens >= 1.  The per-row arithmetic is spark_attn_prefill's: on FULL layers a
 * sequence's outputs are bit for bit those of a batch-1 call on that sequence; a short
 * SLIDING batch-1 call (fewer than 256 blocks of 64 rows x 4 KV heads) splits each key band
 * over two wave groups, so there the two agree up to rounding.  The attention
 * workgroups take their query blocks from a queue in the workspace (latest blocks first on
 * FULL layers), which the RoPE launch resets, so that unequal lengths still spread evenly
 * over the XCDs; calls sharing a workspace must be ordered on a stream.
 */
spark_status spark_attn_prefill_varlen(int32_t layer_type, int32_t batch, const int32_t* cu_seqlens,
                                       int32_t total_tokens, int32_t max_seqlen, const void* q,
                                       const void* k, const void* v, const void* gate_logits,
                                       const spark_kv_cache* cache, void* workspace,
                                       size_t workspace_bytes, void* out, void* stream);

/*
 * KV write (Spark X2.5-4B F16 vs Q4 comparison, hotelren.com/news/5475707, section 一: 4 KB
 * of K and V per token and full layer; Sharp-Spark-X2.5-4B-GGUF guide, mpbf.cn/news/67460,
 * section 三: the sliding layers' cache stays fixed whatever the context, which the
 * 512-slot ring gives; RoPE of the key as in spark_attn_prefill).
 *
 * Append `n_new` tokens per sequence to a layer's cache.
 *   k, v   bf16 [batch, n_new, 4, 256], k before RoPE
 *   pos    device int32 [batch]: position of the first new token of each sequence
 * Token t of sequence b is rotated at position pos[b] + t and stored in slot
 * pos[b] + t (FULL; must be < capacity) or (pos[b] + t) mod 512 (SLIDING; when n_new
 * exceeds 512 only the last 512 tokens are written, as a sequential append would leave
 * them).  The caller tracks lengths: afterwards a sequence holds pos[b] + n_new tokens.
 */
spark_status spark_kv_append(int32_t layer_type, int32_t batch, int32_t n_new,
                             const void* k, const void* v, const int32_t* pos,
                             const spark_kv_cache* cache, void* stream);

/*
 * Bytes of device workspace spark_attn_decode needs for this shape and partition count
 * (num_parts = 0 lets the library choose, exactly as spark_attn_decode will).  The size
 * grows with batch and num_parts only: (num_parts + batch) partial results of 16 x 258
 * floats, plus each sequence's partition range.  Returns 0 for arguments
 * spark_attn_decode would reject.
 */
size_t spark_attn_decode_workspace_bytes(int32_t layer_type, int32_t batch,
                                         int32_t max_seq_len, int32_t num_parts);

/*
 * Decode (Spark X2.5-4B F16 vs Q4 comparison, hotelren.com/news/5475707, section 二: each
 * generated token re-reads the cached state, so decode is bound by memory bandwidth; the
 * visible keys, RoPE of the query and the gate as in spark_attn_prefill).
 *
 * One query token per sequence against the layer's cache.
 *   q            bf16 [batch, 16, 256], before RoPE; it is rotated at position L-1
 *   gate_logits  bf16 [batch, 16]
 *   cache        the layer's cache, already holding the current token
 *   seq_lens     device int32 [batch]: L = tokens in the cache including the current one,
 *                1 <= L <= max_seq_len (a sequence with L < 1 gets a zero output)
 *   max_seq_len  host upper bound of seq_lens; FULL: <= capacity
 *   num_parts    number of workgroups the batch's visible keys are divided among, in
 *                equal runs of 32-key chunks across sequence boundaries (1 .. 2^20), or 0
 *                for the library's choice; the result does not depend on it beyond rounding
 *   workspace    device scratch of at least spark_attn_decode_workspace_bytes(...)
 *                bytes, 256-byte aligned, used only during the call (calls sharing one
 *                workspace must be ordered on a stream)
 *   out          bf16 [batch, 16, 256] (written)
 * FULL layers read positions 0..L-1; SLIDING layers read positions max(0, L-512)..L-1
 * from the ring (attention over a set of keys does not depend on their order).  Two
 * launches: attention with per-(partition, sequence) partial results (each workgroup
 * derives its share of the batch from seq_lens on the device), then a log-sum-exp merge
 * that also applies the gate.
 */
spark_status spark_attn_decode(int32_t layer_type, int32_t batch, const void* q,
                               const void* gate_logits, const spark_kv_cache* cache,
                               const int32_t* seq_lens, int32_t max_seq_len,
                               int32_t num_parts, void* workspace,
                               size_t workspace_bytes, void* out, void* stream);

/*
 * spark_attn_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): no workspace argument.  The
 * partial results live in a static device array of SPARK_DECODE_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that the library holds on every GPU it runs on until the process ends; the call
 * itself allocates and frees nothing.  Its first call on a device, with that device
 * current, looks the array's device address up (hipGetSymbolAddress; a failure returns
 * SPARK_ERR_HIP).  Arguments, limits and results are those of spark_attn_decode; a shape
 * whose spark_attn_decode_workspace_bytes(layer_type, batch, max_seq_len, num_parts)
 * exceeds the array returns SPARK_ERR_WORKSPACE with nothing enqueued (batch 64 with the
 * library's partition count needs about 5 MiB).  Nothing
 * in the array has to start at zero: each call writes every byte it reads before reading
 * it.  All calls on one GPU share the array, which keeps the last call's contents, so
 * calls that may overlap on one GPU (other streams, or other host threads without an
 * order between their streams) race and give undefined results.
 */
#define SPARK_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
spark_status spark_attn_decode_noalloc(int32_t layer_type, int32_t batch, const void* q,
                                       const void* gate_logits, const spark_kv_cache* cache,
                                       const int32_t* seq_lens, int32_t max_seq_len,
                                       int32_t num_parts, void* out, void* stream);

/*
 * 8-bit KV cache of one layer: the q8_0 format the Sharp-Spark-X2.5-4B-GGUF guide
 * (mpbf.cn/news/67460, section 四) enables with --cache-type-k/v q8_0, 36 -> 19 KB per
 * token over the 9 full layers.  Each K or V row of 256 values is 8 blocks of 32; a block
 * stores one scale d = max|x| / 127 (fp16) and 32 int8 codes round(x / d), rounded half
 * away from zero (all 0 when d = 0); the value reads back as code * d.  Decisions are
 * taken in fp32 (d, 1/d and x * (1/d)), and d is rounded to fp16 to nearest even.
 *   k, v               int8 codes [batch, capacity, 4, 256], 16-byte aligned
 *   k_scale, v_scale   fp16 scales [batch, capacity, 4, 8], 16-byte aligned
 * Keys are quantised after RoPE; slots and capacity rules are those of spark_kv_cache.
 * Per token and KV head: 256 + 16 bytes for K and as much for V (bf16: 512 + 512).
 */
typedef struct spark_kv_cache_q8 {
  void* k;
  void* k_scale;
  void* v;
  void* v_scale;
  int32_t batch;
  int32_t capacity;
} spark_kv_cache_q8;

/*
 * spark_kv_append into an 8-bit cache: token t of sequence b is rotated at position
 * pos[b] + t (in fp32, never rounded to bf16), and its key and value are quantised as
 * above into the same slot spark_kv_append would use.  Same arguments, limits and errors
 * as spark_kv_append.
 */
spark_status spark_kv_append_q8(int32_t layer_type, int32_t batch, int32_t n_new,
                                const void* k, const void* v, const int32_t* pos,
                                const spark_kv_cache_q8* cache, void* stream);

/*
 * Bytes of device workspace spark_attn_decode_q8 needs; as
 * spark_attn_decode_workspace_bytes, except that num_parts = 0 plans two partitions per
 * CU (one for the bf16 cache).
 */
size_t spark_attn_decode_q8_workspace_bytes(int32_t layer_type, int32_t batch,
                                            int32_t max_seq_len, int32_t num_parts);

/*
 * spark_attn_decode against an 8-bit cache: keys and values read back as code * scale.
 * Same arguments, limits and errors as spark_attn_decode, with the workspace of
 * spark_attn_decode_q8_workspace_bytes; the two launches stream 272 + 272 bytes per key
 * and KV head instead of 512 + 512.
 */
spark_status spark_attn_decode_q8(int32_t layer_type, int32_t batch, const void* q,
                                  const void* gate_logits, const spark_kv_cache_q8* cache,
                                  const int32_t* seq_lens, int32_t max_seq_len,
                                  int32_t num_parts, void* workspace,
                                  size_t workspace_bytes, void* out, void* stream);

/* Static description of a status code; never NULL. */
const char* spark_status_string(int32_t status);

/* SPARK_ATTN_ABI_VERSION of the built library. */
int32_t spark_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARK_ATTN_H */
