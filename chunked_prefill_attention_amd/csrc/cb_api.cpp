// C ABI entry points: argument validation (host scalars only, no device
// reads, no synchronisation) and dispatch to the kernels on the caller's
// stream.  The semantics of each call are documented in include/cb.h.
#include <cmath>
#include <cstdio>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "cb_internal.h"
#include "kernels.h"

namespace cb {

namespace {
thread_local char g_err[512] = "";
}

thread_local hipEvent_t g_prof_start = nullptr;
thread_local hipEvent_t g_prof_stop = nullptr;
thread_local void* g_prof_clock = nullptr;

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_err[0] = '\0'; }

}  // namespace cb

namespace {

int check_common(int32_t hkv, int32_t head_dim, int32_t page_size, int32_t num_pages, int32_t dtype) {
  if (page_size != CB_PAGE_SIZE)
    return cb::fail(CB_ERR_UNSUPPORTED, "page_size must be %d (got %d)", CB_PAGE_SIZE, page_size);
  if (head_dim != 64 && head_dim != 128)
    return cb::fail(CB_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (dtype != CB_F32 && dtype != CB_BF16)
    return cb::fail(CB_ERR_UNSUPPORTED, "dtype must be CB_F32 or CB_BF16 (got %d)", dtype);
  if (hkv < 1) return cb::fail(CB_ERR_INVALID, "num_kv_heads must be >= 1 (got %d)", hkv);
  if (num_pages < 1 || (int64_t)num_pages * CB_PAGE_SIZE >= (int64_t(1) << 31))
    return cb::fail(CB_ERR_INVALID, "num_pages must be in [1, 2^27) (got %d)", num_pages);
  return CB_OK;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CB_OK;
  return cb::fail(CB_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* cb_status_string(int status) {
  switch (status) {
    case CB_OK: return "CB_OK";
    case CB_ERR_INVALID: return "CB_ERR_INVALID";
    case CB_ERR_UNSUPPORTED: return "CB_ERR_UNSUPPORTED";
    case CB_ERR_WORKSPACE: return "CB_ERR_WORKSPACE";
    case CB_ERR_DEVICE: return "CB_ERR_DEVICE";
    case CB_ERR_CAPACITY: return "CB_ERR_CAPACITY";
    default: return "CB_ERR_UNKNOWN";
  }
}

const char* cb_last_error(void) { return cb::g_err; }

int cb_abi_version(void) { return 4; }

int cb_profile_events(void* start_event, void* stop_event) {
  cb::clear_error();
  if ((start_event == nullptr) != (stop_event == nullptr))
    return cb::fail(CB_ERR_INVALID, "cb_profile_events: pass two events or none");
  cb::g_prof_start = static_cast<hipEvent_t>(start_event);
  cb::g_prof_stop = static_cast<hipEvent_t>(stop_event);
  return CB_OK;
}

int cb_profile_clock(void* device_buffer) {
  cb::clear_error();
  cb::g_prof_clock = device_buffer;
  return CB_OK;
}

int cb_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                 int32_t head_dim, int32_t num_pages, int32_t page_size, int32_t dtype, void* stream) {
  cb::clear_error();
  if (int st = check_common(num_kv_heads, head_dim, page_size, num_pages, dtype)) return st;
  if (num_tokens < 0) return cb::fail(CB_ERR_INVALID, "num_tokens must be >= 0 (got %d)", num_tokens);
  if (num_tokens == 0) return CB_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
    return cb::fail(CB_ERR_INVALID, "cb_kv_append: null pointer");
  if ((int64_t)((num_tokens + 15) / 16) * num_kv_heads >= (int64_t(1) << 31))
    return cb::fail(CB_ERR_INVALID, "cb_kv_append: too many tokens x heads for one launch");
  const int32_t es = dtype == CB_BF16 ? 2 : 4;
  hipError_t e = cb::launch_kv_append(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,
                                      head_dim, num_pages, es, static_cast<hipStream_t>(stream));
  return device_status(e, "cb_kv_append launch");
}

size_t cb_attention_workspace_bytes(int32_t num_seqs, int32_t num_decodes, int32_t num_tokens,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_context_len, int32_t dtype) {
  if (num_seqs < 0 || num_decodes < 0 || num_decodes > num_seqs || num_tokens < 0 || num_q_heads < 1 ||
      num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 || head_dim < 1 || max_context_len < 0)
    return (size_t)-1;
  if (dtype == CB_F32) return 0;
  if (dtype != CB_BF16) return (size_t)-1;
  return cb::plan_bf16(num_seqs, num_decodes, num_tokens, num_q_heads, num_kv_heads, head_dim,
                       max_context_len).bytes;
}

int cb_attention_step(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t block_table_stride,
                      const int32_t* query_start_loc, const int32_t* context_lens,
                      const int32_t* q_offsets, int32_t num_seqs, int32_t num_decodes,
                      int32_t num_tokens, int32_t max_context_len, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t num_pages, float scale, int32_t sliding_window, int32_t dtype, void* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return cb::attention_step_impl(q, k_cache, v_cache, block_tables, block_table_stride, query_start_loc,
                                 context_lens, q_offsets, num_seqs, num_decodes, num_tokens, max_context_len,
                                 num_q_heads, num_kv_heads, head_dim, page_size, num_pages, scale,
                                 sliding_window, dtype, out, workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

namespace cb {

int attention_step_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        int32_t block_table_stride, const int32_t* query_start_loc, const int32_t* context_lens,
                        const int32_t* q_offsets, int32_t num_seqs, int32_t num_decodes, int32_t num_tokens,
                        int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t page_size, int32_t num_pages, float scale, int32_t sliding_window,
                        int32_t dtype, void* out, void* workspace, size_t workspace_bytes, void* stream,
                        const WorkLists* lists, const int32_t* bt_offsets) {
  cb::clear_error();
  if (int st = check_common(num_kv_heads, head_dim, page_size, num_pages, dtype)) return st;
  if (num_q_heads < 1 || num_q_heads % num_kv_heads != 0)
    return cb::fail(CB_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                    num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 16)
    return cb::fail(CB_ERR_UNSUPPORTED, "group size num_q_heads/num_kv_heads must be <= 16 (got %d)",
                    num_q_heads / num_kv_heads);
  if (num_seqs < 0 || num_decodes < 0 || num_decodes > num_seqs || num_tokens < num_decodes ||
      max_context_len < 0)
    return cb::fail(CB_ERR_INVALID, "inconsistent sizes: num_seqs=%d num_decodes=%d num_tokens=%d max_context_len=%d",
                    num_seqs, num_decodes, num_tokens, max_context_len);
  if (num_tokens > 0 && num_seqs == 0)
    return cb::fail(CB_ERR_INVALID, "num_tokens > 0 with no sequences");
  if (!std::isfinite(scale)) return cb::fail(CB_ERR_INVALID, "scale must be finite");
  // the bf16 online softmax keeps the running maximum of raw scores, which
  // orders like the scaled scores only when the scale is positive
  if (dtype == CB_BF16 && !(scale > 0.f))
    return cb::fail(CB_ERR_UNSUPPORTED, "the bf16 path needs scale > 0 (got %g)", (double)scale);
  if (sliding_window < 0) return cb::fail(CB_ERR_INVALID, "sliding_window must be >= 0");
  if ((int64_t)num_tokens * num_q_heads * head_dim >= (int64_t(1) << 40))
    return cb::fail(CB_ERR_INVALID, "step too large");
  if (num_tokens == 0) return CB_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !query_start_loc || !context_lens || !q_offsets || !out)
    return cb::fail(CB_ERR_INVALID, "cb_attention_step: null pointer");
  if (max_context_len < 1) return cb::fail(CB_ERR_INVALID, "max_context_len must be >= 1 for a non-empty step");
  if ((int64_t)block_table_stride * CB_PAGE_SIZE < max_context_len)
    return cb::fail(CB_ERR_INVALID, "block_table_stride %d cannot hold max_context_len %d", block_table_stride,
                    max_context_len);

  cb::AttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.bt_stride = block_table_stride;
  a.bt_offsets = bt_offsets;
  a.qsl = query_start_loc;
  a.ctx_lens = context_lens;
  a.q_offsets = q_offsets;
  a.num_seqs = num_seqs;
  a.num_decodes = num_decodes;
  a.num_tokens = num_tokens;
  a.max_context_len = max_context_len;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.num_pages = num_pages;
  a.scale = scale;
  a.window = sliding_window;
  a.out = out;
  a.workspace = workspace;
  const hipStream_t st = static_cast<hipStream_t>(stream);

  if (dtype == CB_F32) {
    if ((int64_t)num_tokens * num_q_heads / 4 >= (int64_t(1) << 31))
      return cb::fail(CB_ERR_INVALID, "step too large for one launch");
    return device_status(cb::launch_attention_f32(a, st), "cb_attention_step launch (f32)");
  }
  const cb::Bf16Plan plan = cb::plan_bf16(num_seqs, num_decodes, num_tokens, num_q_heads, num_kv_heads,
                                          head_dim, max_context_len, sliding_window);
  if (plan.dec_cap * num_kv_heads >= (int64_t(1) << 31) || plan.pf_item_cap * num_kv_heads >= (int64_t(1) << 30) ||
      plan.pf_tile_cap * num_kv_heads >= (int64_t(1) << 27))   // the prefill combine runs 8 blocks per tile
    return cb::fail(CB_ERR_INVALID, "step too large for one launch");
  if (!workspace || workspace_bytes < plan.bytes)
    return cb::fail(CB_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu%s)", plan.bytes, workspace_bytes,
                    workspace ? "" : ", null pointer");
  return device_status(cb::launch_attention_bf16(a, plan, lists, st), "cb_attention_step launch (bf16)");
}

}  // namespace cb
