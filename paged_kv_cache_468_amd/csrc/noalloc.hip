// The decode step for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): pkv_decode_step with the balanced split, its workspace taken
// from a fixed device array that the library holds, one per GPU, instead of
// a caller's buffer. The kernels are pkv_decode_step's own.
//
// The array lives in this file. Host code never passes its name to a kernel
// or a copy: in host code that name is only a stand-in for the symbol. Its
// device address is looked up once per device with hipGetSymbolAddress, on
// the first call made with that device current, and kept; every launch gets
// that address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pkv.h"

namespace {

__device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device
std::mutex g_scratch_mu;

// The current device's copy of the array, looked up on first use.
int current_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PKV_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_decode_step_noalloc(float* out, const void* q, const void* k_new,
                                       const void* v_new, void* k_pool, void* v_pool,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       int32_t num_seqs, int32_t max_blocks_per_seq,
                                       int32_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t head_dim, float scale, int32_t max_context_len,
                                       int32_t* err_flag, void* stream) {
  void* ws = nullptr;
  const int rc = current_scratch(&ws);
  if (rc != PKV_OK) return rc;
  // 0 for arguments pkv_decode_step rejects itself (it reports those)
  const size_t need = pkv_decode_workspace_bytes(num_seqs, n_q_heads, n_kv_heads, head_dim,
                                                 max_context_len, 0);
  if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_EWORKSPACE;
  return pkv_decode_step(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                         num_seqs, max_blocks_per_seq, num_blocks, n_q_heads, n_kv_heads,
                         head_dim, scale, max_context_len, 0, ws, PKV_NOALLOC_SCRATCH_BYTES,
                         err_flag, stream);
}
