/*
 * Random calls of every entry point of spark_attn.h, for a build of the library's host code
 * with AddressSanitizer on a host without a GPU (tests/test_abi_fuzz.py builds and runs
 * it).  Sizes in and out of range, null, misaligned and aligned fake device pointers
 * (never dereferenced by the host), cache descriptors of any shape.  The host-side checks
 * must touch nothing but their arguments; a call that passes them reaches its launch,
 * which fails without a GPU (SPARK_ERR_HIP).  Exit status 1 if a status is out of range
 * or a call reports success.
 */
#include "spark_attn.h"

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

static uint64_t g_state = 0x243F6A8885A308D3ull;

/* splitmix64 */
static uint64_t next_u64(void) {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static int32_t rnd_size(void) {
  static const int32_t v[] = {-3, -1, 0, 1, 2, 3, 7, 16, 31, 32, 33, 511, 512, 513, 4096,
                              65535, 65536, 1 << 20, (1 << 20) + 1, 2147483647, -2147483647 - 1};
  return v[next_u64() % (sizeof v / sizeof v[0])];
}

static void* rnd_ptr(void) {
  static const uintptr_t v[] = {0, 0x100000, 0x100010, 0x100002, 0x100001};
  return (void*)v[next_u64() % (sizeof v / sizeof v[0])];
}

static int32_t rnd_type(void) {
  static const int32_t v[] = {0, 1, 0, 1, 2, -1};
  return v[next_u64() % (sizeof v / sizeof v[0])];
}

static size_t rnd_bytes(void) {
  switch (next_u64() % 4) {
    case 0: return 0;
    case 1: return (size_t)(next_u64() % 4096);
    case 2: return (size_t)1 << 40;
    default: return (size_t)(next_u64() % ((size_t)1 << 34));
  }
}

int main(int argc, char** argv) {
  const long n = argc > 1 ? atol(argv[1]) : 100000;
  long counts[5] = {0, 0, 0, 0, 0};
  long sized = 0;
  for (long i = 0; i < n; ++i) {
    spark_kv_cache c = {rnd_ptr(), rnd_ptr(), rnd_size(), rnd_size()};
    spark_kv_cache_q8 c8 = {rnd_ptr(), rnd_ptr(), rnd_ptr(), rnd_ptr(), rnd_size(), rnd_size()};
    const spark_kv_cache* cp = (next_u64() % 4) ? &c : NULL;
    const spark_kv_cache_q8* cp8 = (next_u64() % 4) ? &c8 : NULL;
    int32_t st = SPARK_ERR_INVALID_ARG;
    switch (next_u64() % 14) {
      case 0:
        st = spark_attn_prefill(rnd_type(), rnd_size(), rnd_size(), rnd_size(), rnd_ptr(), rnd_ptr(), rnd_ptr(),
                                rnd_ptr(), cp, rnd_ptr(), rnd_bytes(), rnd_ptr(), NULL);
        break;
      case 1:
        st = spark_attn_prefill_varlen(rnd_type(), rnd_size(), (const int32_t*)rnd_ptr(), rnd_size(), rnd_size(),
                                       rnd_ptr(), rnd_ptr(), rnd_ptr(), rnd_ptr(), cp, rnd_ptr(), rnd_bytes(),
                                       rnd_ptr(), NULL);
        break;
      case 2:
        st = spark_kv_append(rnd_type(), rnd_size(), rnd_size(), rnd_ptr(), rnd_ptr(), (const int32_t*)rnd_ptr(),
                             cp, NULL);
        break;
      case 3:
        st = spark_attn_decode(rnd_type(), rnd_size(), rnd_ptr(), rnd_ptr(), cp, (const int32_t*)rnd_ptr(),
                               rnd_size(), rnd_size(), rnd_ptr(), rnd_bytes(), rnd_ptr(), NULL);
        break;
      case 4:
        st = spark_attn_decode_noalloc(rnd_type(), rnd_size(), rnd_ptr(), rnd_ptr(), cp, (const int32_t*)rnd_ptr(),
                                       rnd_size(), rnd_size(), rnd_ptr(), NULL);
        break;
      case 5:
        st = spark_kv_append_q8(rnd_type(), rnd_size(), rnd_size(), rnd_ptr(), rnd_ptr(), (const int32_t*)rnd_ptr(),
                                cp8, NULL);
        break;
      case 6:
        st = spark_attn_decode_q8(rnd_type(), rnd_size(), rnd_ptr(), rnd_ptr(), cp8, (const int32_t*)rnd_ptr(),
                                  rnd_size(), rnd_size(), rnd_ptr(), rnd_bytes(), rnd_ptr(), NULL);
        break;
      case 7:
        st = spark_qkv_proj_fp8(rnd_size(), rnd_ptr(), rnd_ptr(), (const float*)rnd_ptr(), rnd_ptr(), rnd_ptr(),
                                rnd_ptr(), rnd_ptr(), rnd_ptr(), rnd_ptr(), rnd_bytes(), NULL);
        break;
      case 8: {
        double th = 0.0;
        int32_t rd = 0, w = 0;
        const int32_t lt = rnd_type();
        st = spark_layer_params(lt, (next_u64() & 1) ? &th : NULL, (next_u64() & 1) ? &rd : NULL,
                                (next_u64() & 1) ? &w : NULL);
        if (st == SPARK_OK) st = SPARK_ERR_HIP;    /* a valid query: counted with the passed checks */
        break;
      }
      case 9: {
        const int32_t t = spark_layer_type_of(rnd_size());
        if (t < -1 || t > 1) { fprintf(stderr, "layer type %d\n", t); return 1; }
        ++sized;
        continue;
      }
      case 10: {
        const char* s = spark_status_string(rnd_size());
        if (s == NULL) { fprintf(stderr, "null status string\n"); return 1; }
        ++sized;
        continue;
      }
      default: {
        volatile size_t z = spark_attn_prefill_workspace_bytes(rnd_type(), rnd_size(), rnd_size()) +
                            spark_attn_prefill_varlen_workspace_bytes(rnd_type(), rnd_size()) +
                            spark_attn_decode_workspace_bytes(rnd_type(), rnd_size(), rnd_size(), rnd_size()) +
                            spark_attn_decode_q8_workspace_bytes(rnd_type(), rnd_size(), rnd_size(), rnd_size()) +
                            spark_qkv_proj_fp8_workspace_bytes(rnd_size());
        (void)z;
        ++sized;
        continue;
      }
    }
    if (st < 0 || st > 4) { fprintf(stderr, "status %d out of range\n", st); return 1; }
    if (st == SPARK_OK) { fprintf(stderr, "a call reported success without a GPU\n"); return 1; }
    ++counts[st];
  }
  printf("calls: %ld; invalid %ld unsupported %ld workspace %ld passed-to-launch %ld; size queries %ld\n", n,
         counts[1], counts[2], counts[3], counts[4], sized);
  return 0;
}
