// Native engine step: FIFO builder -> pinned staging -> one async upload ->
// KV append -> attention, with no Python (or other host language) in the
// per-step path.  Semantics in include/cb.h ("Engine").
#include <algorithm>
#include <cstring>
#include <new>

#include <hip/hip_runtime_api.h>

#include "cb_internal.h"
#include "kernels.h"

struct cb_engine {
  cb_engine_config cfg{};
  cb_builder* builder = nullptr;
  hipEvent_t copied[2] = {nullptr, nullptr};  // last upload from each staging slot
  bool slot_used[2] = {false, false};
  int slot = 0;          // slot of the scheduled (not yet attended) step
  bool pending = false;  // a scheduled step awaits cb_engine_attend
  cb_step step{};
  int64_t slot_ints = 0;
  // device views of the pending step's metadata
  const int32_t *d_qsl = nullptr, *d_ctx = nullptr, *d_off = nullptr, *d_bt = nullptr, *d_slots = nullptr;
  bool have_lists = false;  // bf16: the step's work lists were built on the host
  cb::WorkLists lists{};
};

extern "C" {

int cb_engine_create(const cb_engine_config* config, cb_engine** out) {
  cb::clear_error();
  if (!config || !out) return cb::fail(CB_ERR_INVALID, "cb_engine_create: null argument");
  const cb_engine_config& c = *config;
  if (!c.k_cache || !c.v_cache || !c.meta_device || !c.meta_host)
    return cb::fail(CB_ERR_INVALID, "cb_engine_create: caches and metadata buffers are required");
  if (c.num_kv_heads < 1 || c.num_q_heads < 1 || c.num_q_heads % c.num_kv_heads != 0)
    return cb::fail(CB_ERR_INVALID, "cb_engine_create: bad head counts");
  if (c.head_dim != 64 && c.head_dim != 128) return cb::fail(CB_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c.dtype != CB_F32 && c.dtype != CB_BF16) return cb::fail(CB_ERR_UNSUPPORTED, "unknown dtype");
  const int64_t slot_ints = (int64_t)(c.meta_bytes / sizeof(int32_t) / 2);
  if (slot_ints < 16) return cb::fail(CB_ERR_INVALID, "cb_engine_create: metadata buffers too small");
  cb_engine* e = new (std::nothrow) cb_engine();
  if (!e) return cb::fail(CB_ERR_INVALID, "out of host memory");
  e->cfg = c;
  e->slot_ints = slot_ints;
  int st = cb_builder_create(&c.builder, &e->builder);
  if (st != CB_OK) { delete e; return st; }
  for (int i = 0; i < 2; ++i) {
    if (hipEventCreateWithFlags(&e->copied[i], hipEventDisableTiming) != hipSuccess) {
      cb_engine_destroy(e);
      return cb::fail(CB_ERR_DEVICE, "cb_engine_create: hipEventCreate failed");
    }
  }
  *out = e;
  return CB_OK;
}

void cb_engine_destroy(cb_engine* e) {
  if (!e) return;
  for (int i = 0; i < 2; ++i)
    if (e->copied[i]) {
      (void)hipEventSynchronize(e->copied[i]);
      (void)hipEventDestroy(e->copied[i]);
    }
  cb_builder_destroy(e->builder);
  delete e;
}

cb_builder* cb_engine_builder(cb_engine* e) { return e ? e->builder : nullptr; }

int cb_engine_set_metadata(cb_engine* e, int32_t* meta_device, int32_t* meta_host, size_t meta_bytes) {
  cb::clear_error();
  if (!e || !meta_device || !meta_host) return cb::fail(CB_ERR_INVALID, "cb_engine_set_metadata: null argument");
  const int64_t slot_ints = (int64_t)(meta_bytes / sizeof(int32_t) / 2);
  if (slot_ints < 16) return cb::fail(CB_ERR_INVALID, "cb_engine_set_metadata: buffers too small");
  for (int i = 0; i < 2; ++i)
    if (e->slot_used[i]) (void)hipEventSynchronize(e->copied[i]);
  e->cfg.meta_device = meta_device;
  e->cfg.meta_host = meta_host;
  e->cfg.meta_bytes = meta_bytes;
  e->slot_ints = slot_ints;
  e->slot_used[0] = e->slot_used[1] = false;
  e->slot = 0;
  e->pending = false;
  return CB_OK;
}

int cb_engine_set_workspace(cb_engine* e, void* workspace, size_t workspace_bytes) {
  cb::clear_error();
  if (!e) return cb::fail(CB_ERR_INVALID, "cb_engine_set_workspace: null engine");
  e->cfg.workspace = workspace;
  e->cfg.workspace_bytes = workspace ? workspace_bytes : 0;
  return CB_OK;
}

int cb_engine_schedule(cb_engine* e, void* stream, cb_step* out) {
  cb::clear_error();
  if (!e || !out) return cb::fail(CB_ERR_INVALID, "cb_engine_schedule: null argument");
  const cb_builder_config& bc = e->cfg.builder;
  // worst case of this step's metadata, before the builder changes state
  const int64_t B = bc.max_requests_per_batch, T = bc.max_batch_tokens;
  const int64_t stride = (int64_t)cb::builder_max_pages_held(e->builder) + cb::ceil_div(T, CB_PAGE_SIZE) + 1;
  int64_t need = (B + 1) + 2 * B + B * std::min<int64_t>(stride, bc.num_pages) + T;
  if (e->cfg.dtype == CB_BF16) {  // bound of the host-built work lists (int32 units)
    const int64_t G = e->cfg.num_q_heads / e->cfg.num_kv_heads;
    const int64_t pages = std::min<int64_t>(stride, bc.num_pages);
    const int64_t dec_cap = B * cb::ceil_div(pages, 8);
    const int64_t tiles = cb::ceil_div(T * G, 128) + B + 1;
    const int64_t items = tiles * (cb::ceil_div(pages * CB_PAGE_SIZE, 512) + 1);
    need += 4 * (dec_cap + tiles + items) + 2 * B + 32;
  }
  if (need > e->slot_ints)
    return cb::fail(CB_ERR_CAPACITY, "step metadata may need %lld int32 per slot; the engine has %lld",
                    (long long)need, (long long)e->slot_ints);
  const int slot = e->pending ? e->slot : (e->slot_used[e->slot] ? e->slot ^ 1 : e->slot);
  // the staging slot must not be rewritten while its previous upload is in flight
  if (e->slot_used[slot] && hipEventSynchronize(e->copied[slot]) != hipSuccess)
    return cb::fail(CB_ERR_DEVICE, "cb_engine_schedule: waiting for the previous upload failed");
  int st = cb_builder_step(e->builder, &e->step);
  if (st != CB_OK) return st;
  const cb_step& d = e->step;
  int32_t* h = e->cfg.meta_host + (size_t)slot * e->slot_ints;
  int32_t* dv = e->cfg.meta_device + (size_t)slot * e->slot_ints;
  size_t off = 0;
  auto put = [&](const int32_t* src, size_t n) {
    if (n) std::memcpy(h + off, src, n * sizeof(int32_t));
    const size_t at = off;
    off += n;
    return at;
  };
  const size_t o_qsl = put(d.query_start_loc, (size_t)d.num_seqs + 1);
  const size_t o_ctx = put(d.context_lens, (size_t)d.num_seqs);
  const size_t o_off = put(d.q_offsets, (size_t)d.num_seqs);
  const size_t o_bt = put(d.block_tables, (size_t)d.num_seqs * d.block_table_stride);
  const size_t o_sl = put(d.slot_mapping, (size_t)d.num_tokens);
  e->have_lists = false;
  if (e->cfg.dtype == CB_BF16 && d.num_tokens > 0) {
    // the attention step's work lists, built here instead of by a device plan kernel
    const cb::Bf16Plan pl = cb::plan_bf16(d.num_seqs, d.num_decodes, d.num_tokens, e->cfg.num_q_heads,
                                          e->cfg.num_kv_heads, e->cfg.head_dim, std::max(d.max_context_len, 1));
    const cb::WorkListLayout lay = cb::work_list_layout(pl, d.num_decodes);
    const size_t at = (off + 3) & ~size_t(3);  // 16-byte aligned (int32 units)
    if ((int64_t)(at + lay.bytes / 4) <= e->slot_ints) {
      cb::build_work_lists(pl, d.num_seqs, d.num_decodes, e->cfg.num_q_heads / e->cfg.num_kv_heads,
                           e->cfg.builder.sliding_window, d.query_start_loc, d.context_lens, d.q_offsets,
                           h + at);
      const uint8_t* db = reinterpret_cast<const uint8_t*>(dv + at);
      e->lists.dec_items = db + lay.dec_items;
      e->lists.pf_items = db + lay.pf_items;
      e->lists.pf_tiles = db + lay.pf_tiles;
      e->lists.dec_first = reinterpret_cast<const int32_t*>(db + lay.dec_first);
      e->lists.dec_rem = reinterpret_cast<const int32_t*>(db + lay.dec_rem);
      e->have_lists = true;
      off = at + lay.bytes / 4;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(dv, h, off * sizeof(int32_t), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipEventRecord(e->copied[slot], s) != hipSuccess)
    return cb::fail(CB_ERR_DEVICE, "cb_engine_schedule: metadata upload failed");
  e->slot_used[slot] = true;
  e->slot = slot;
  e->pending = true;
  e->d_qsl = dv + o_qsl;
  e->d_ctx = dv + o_ctx;
  e->d_off = dv + o_off;
  e->d_bt = dv + o_bt;
  e->d_slots = dv + o_sl;
  *out = d;
  return CB_OK;
}

int cb_engine_load_builder(cb_engine* e, const cb_builder* src) {
  cb::clear_error();
  if (!e || !src) return cb::fail(CB_ERR_INVALID, "cb_engine_load_builder: null argument");
  e->pending = false;
  return cb::builder_assign(e->builder, src);
}

size_t cb_engine_workspace_bytes(const cb_engine* e) {
  if (!e || !e->pending) return 0;
  const cb_step& d = e->step;
  return cb_attention_workspace_bytes(d.num_seqs, d.num_decodes, d.num_tokens, e->cfg.num_q_heads,
                                      e->cfg.num_kv_heads, e->cfg.head_dim, std::max(d.max_context_len, 1),
                                      e->cfg.dtype);
}

int cb_engine_attend(cb_engine* e, const void* q, const void* k_new, const void* v_new, void* out,
                     void* stream) {
  cb::clear_error();
  if (!e) return cb::fail(CB_ERR_INVALID, "cb_engine_attend: null engine");
  if (!e->pending) return cb::fail(CB_ERR_INVALID, "cb_engine_attend: no scheduled step");
  const cb_step& d = e->step;
  const cb_engine_config& c = e->cfg;
  if (d.num_tokens == 0) { e->pending = false; return CB_OK; }
  const size_t need = cb_engine_workspace_bytes(e);
  if (need > 0 && (!c.workspace || c.workspace_bytes < need))
    return cb::fail(CB_ERR_WORKSPACE, "the scheduled step needs %zu bytes of workspace (have %zu)", need,
                    c.workspace_bytes);
  int st = cb_kv_append(k_new, v_new, c.k_cache, c.v_cache, e->d_slots, d.num_tokens, c.num_kv_heads,
                        c.head_dim, c.builder.num_pages, CB_PAGE_SIZE, c.dtype, stream);
  if (st != CB_OK) return st;
  st = cb::attention_step_impl(q, c.k_cache, c.v_cache, e->d_bt, d.block_table_stride, e->d_qsl, e->d_ctx,
                               e->d_off, d.num_seqs, d.num_decodes, d.num_tokens, d.max_context_len,
                               c.num_q_heads, c.num_kv_heads, c.head_dim, CB_PAGE_SIZE, c.builder.num_pages,
                               c.scale, c.builder.sliding_window, c.dtype, out, c.workspace,
                               c.workspace_bytes, stream,
                               e->have_lists ? &e->lists : nullptr);
  if (st == CB_OK) e->pending = false;
  return st;
}

}  // extern "C"
