"""CPU fp64 oracle of the hybrid sliding/full GQA attention path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  It shares
no code with the HIP path (``full_gqa_attention_amd``) and imports nothing from it.

What each function computes, and the passage it follows, is stated in its docstring.
Pages cited (titles as given by their addresses):
  [FP8]   Spark-X2.6-4B-FP8 quantisation walkthrough (nxmr.cn/news/148448)
  [F16Q4] Spark X2.5-4B F16 vs Q4 comparison (hotelren.com/news/5475707)
  [CFG]   Spark-X2.6-4B config.json guide (lqnn.cn/news/248463)
  [HYB]   Spark-X2.6-4B-Base hybrid attention explainer (eliteato.com/news/34565)
  [GGUF]  Sharp-Spark-X2.5-4B-GGUF on a 6 GB GPU (mpbf.cn/news/67460)

Modules: ``attention`` (prefill, chunked and varlen prefill, append, decode), ``kvq8``
(the 8-bit q8_0 cache), ``proj`` (the W8A8 FP8 q_k_v_proj and the bf16 g_proj that feed
the path), ``footprint`` (KV byte counts).

Pinning status: every function is pinned by ``tests/test_oracle_*.py`` (closed forms,
invariants, brute force, a library cross-check and the pages' KV-size figures); the
8-bit cache (``kvq8``) by exact closed forms of the q8_0 rule, its error bound, and the
bf16 append and decode it must agree with.  What
no test can pin is numeric agreement with the real model's trained weights: none exist
here, and the RoPE pairing convention (rotate-half) and the partial-rotary frequency
denominator are readings of silent passages (both documented where used).
"""
from .attention import (  # noqa: F401
    FULL,
    HEAD_DIM,
    N_KV_HEADS,
    N_LAYERS,
    N_Q_HEADS,
    SLIDING,
    WINDOW,
    bf16_to_f64,
    decode,
    cache_slot,
    kv_append,
    kv_head_of,
    layer_params,
    layer_type_of,
    layer_types,
    prefill,
    prefill_chunk,
    prefill_varlen,
    rope,
    rope_inv_freq,
    round_to_bf16_bits,
    softmax_scale,
    visibility,
)
from .kvq8 import (  # noqa: F401
    Q8_BLOCK,
    decode_q8,
    kv_append_q8,
    q8_dequantize,
    q8_quantize,
)
from .proj import (  # noqa: F401
    e4m3fn_decode,
    e4m3fn_encode,
    qkv_proj,
    quantize_tokens,
)
from .footprint import (  # noqa: F401
    kv_bytes_full_layer_per_token,
    kv_bytes_model,
    kv_bytes_sliding_layer,
    q8_0_bytes,
)
