// cb_attention_step without a workspace argument, for callers that cannot
// allocate device memory (work recorded under graph capture, tight serving
// loops, harnesses that forbid allocation).  The bf16 path's work lists and
// split-K partial results live in a fixed file-scope device array instead of
// a caller-provided workspace.  Semantics in include/cb.h.
//
// The array's name is a host-side stand-in in host code: the device address
// of each GPU's copy is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cb_internal.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(CB_NOALLOC_SCRATCH_BYTES);
static_assert(kScratchBytes % 256 == 0, "scratch size is a multiple of its alignment");

// The scratch memory: one copy per device, alive until the process ends.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device (null: not looked up yet)

// Device address of the current device's scratch array.
int scratch_for_current_device(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return cb::fail(CB_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return cb::fail(CB_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess || !p)
      return cb::fail(CB_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(r));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return CB_OK;
}

}  // namespace

extern "C" {

size_t cb_attention_noalloc_scratch_bytes(void) { return kScratchBytes; }

int cb_attention_step_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* query_start_loc, const int32_t* context_lens,
                              const int32_t* q_offsets, int32_t num_seqs, int32_t num_decodes,
                              int32_t num_tokens, int32_t max_context_len, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t num_pages, float scale, int32_t sliding_window, int32_t dtype,
                              void* out, void* stream) {
  cb::clear_error();
  void* ws = nullptr;
  if (dtype == CB_BF16 && num_tokens > 0) {
    // the size check is host arithmetic and comes before any device call
    const size_t need = cb_attention_workspace_bytes(num_seqs, num_decodes, num_tokens, num_q_heads, num_kv_heads,
                                                     head_dim, max_context_len, dtype);
    if (need != (size_t)-1 && need > kScratchBytes)
      return cb::fail(CB_ERR_WORKSPACE,
                      "the step needs %zu bytes of scratch; the allocation-free entry point holds %zu",
                      need, kScratchBytes);
    if (need != (size_t)-1 && need > 0) {
      if (int st = scratch_for_current_device(&ws)) return st;
    }
  }
  // same validation, kernels and launches as cb_attention_step
  return cb::attention_step_impl(q, k_cache, v_cache, block_tables, block_table_stride, query_start_loc,
                                 context_lens, q_offsets, num_seqs, num_decodes, num_tokens, max_context_len,
                                 num_q_heads, num_kv_heads, head_dim, page_size, num_pages, scale, sliding_window,
                                 dtype, out, ws, ws ? kScratchBytes : 0, stream, nullptr);
}

}  // extern "C"
