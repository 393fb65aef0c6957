// pa_decode_noalloc: pa_decode whose partition results live in a static
// device buffer instead of a caller-provided workspace, for callers that
// cannot allocate (graph capture, serving loops, allocation-free harnesses).
//
// The buffer is the file-scope `scratch` array below.  In host code its name
// is only a host-side stand-in for the symbol: its device address, which
// differs per GPU, comes from hipGetSymbolAddress, looked up once per device
// with that device current and kept in `g_scratch`; only that address is
// ever handed to a kernel.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

static __device__ __align__(256) unsigned char scratch[PA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of the scratch buffer on the current device, or a status.
int current_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
  std::lock_guard<std::mutex> hold(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PA_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, const int32_t* seq_order, int num_seqs,
                                 int num_heads, int num_kv_heads, int head_dim, int block_size,
                                 int num_blocks, int max_context_len, float scale, int dtype,
                                 int cache_dtype, float k_scale, float v_scale, int partition_tokens,
                                 int flags, void* stream) {
  // Host checks first (no HIP call), then the size against the buffer.
  const int st = pa::decode_check(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                  seq_order, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                  num_blocks, max_context_len, dtype, cache_dtype, k_scale, v_scale,
                                  partition_tokens, flags);
  if (st != PA_OK) return st;
  const size_t need = pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                               max_context_len, dtype, cache_dtype, partition_tokens);
  if (need > PA_DECODE_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  if (num_seqs == 0) return PA_OK;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = current_scratch(&ws);
    if (rc != PA_OK) return rc;
  }
  return pa_decode(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, seq_order,
                   num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                   scale, dtype, cache_dtype, k_scale, v_scale, partition_tokens, flags, ws,
                   need > 0 ? PA_DECODE_NOALLOC_SCRATCH_BYTES : 0, stream);
}
