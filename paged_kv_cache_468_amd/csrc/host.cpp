// Host-only parts of the C ABI: status strings and the KV-size closed form
// ("Module 23: Serving", 23.1: the cache is the product of 2 (keys and
// values), layers, KV heads, head width, context length, batch and bytes per
// value; "Scaling LLM serving", "The KV cache" gives the per-token product).
#include <stdint.h>

#include "pkv.h"

extern "C" const char* pkv_strerror(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported head_dim (64 or 128)";
    case PKV_ENOMEM: return "no free KV block";
    case PKV_EWORKSPACE: return "workspace too small";
    case PKV_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

extern "C" uint64_t pkv_kv_bytes_per_token(int32_t n_layers, int32_t n_kv_heads,
                                           int32_t head_dim, int32_t bytes_per_value) {
  if (n_layers < 0 || n_kv_heads < 0 || head_dim < 0 || bytes_per_value < 0) return 0;
  return 2ull * (uint64_t)n_layers * (uint64_t)n_kv_heads * (uint64_t)head_dim *
         (uint64_t)bytes_per_value;
}

extern "C" uint64_t pkv_kv_cache_bytes(int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                                       int64_t context_len, int64_t batch,
                                       int32_t bytes_per_value) {
  if (context_len < 0 || batch < 0) return 0;
  return pkv_kv_bytes_per_token(n_layers, n_kv_heads, head_dim, bytes_per_value) *
         (uint64_t)context_len * (uint64_t)batch;
}

extern "C" uint64_t pkv_pool_bytes(int32_t num_blocks, int32_t n_kv_heads, int32_t head_dim) {
  if (num_blocks < 0 || n_kv_heads < 0 || head_dim < 0) return 0;
  return (uint64_t)num_blocks * (uint64_t)n_kv_heads * PKV_BLOCK_TOKENS * (uint64_t)head_dim * 2ull;
}
