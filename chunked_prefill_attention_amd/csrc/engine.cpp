// Native engine step: FIFO builder -> pinned staging -> one async upload ->
// KV append -> attention, with no Python (or other host language) in the
// per-step path.  Semantics in include/cb.h ("Engine").
//
// Graph replay (transformers, "Continuous batching architecture", CUDA
// graphs): with padding intervals set, each step's metadata is laid out for a
// padded shape (tokens rounded up to the q interval, the longest context to
// the KV interval, decode and prefill sequence counts to multiples of 16 and
// 4; padding sequences are empty and padding tokens have slot -1), so that
// steps of one padded shape launch identical kernels with identical
// arguments.  The append, attention and combine launches of a shape are
// captured once into a HIP graph and replayed after that.
#include <algorithm>
#include <cstring>
#include <map>
#include <new>
#include <tuple>

#include <hip/hip_runtime_api.h>

#include "cb_internal.h"
#include "kernels.h"

namespace {
struct GraphKey {
  int slot;
  int32_t nseq, ndec, ntok, maxctx, stride;
  int64_t pull;
  const void *q, *k, *v, *out, *ws;
  size_t ws_bytes;
  auto tie() const { return std::tie(slot, nseq, ndec, ntok, maxctx, stride, pull, q, k, v, out, ws, ws_bytes); }
  bool operator<(const GraphKey& o) const { return tie() < o.tie(); }
};
constexpr size_t kMaxGraphs = 128;
int32_t round_up(int32_t x, int32_t m) { return (int32_t)cb::ceil_div(x, m) * m; }
}  // namespace

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
  const int32_t* d_btoff = nullptr;  // row offsets of the packed block tables
  // the pinned staging buffer as the device addresses it (null: not mapped,
  // then the metadata goes up with a copy in the stream)
  int32_t* meta_host_dev = nullptr;
  int64_t pull_ints = 0;                 // metadata int32s the append kernel copies up
  const int32_t* h_slots_dev = nullptr;  // the slot mapping in the staging slot, device address
  bool have_lists = false;  // bf16: the step's work lists were built on the host
  cb::WorkLists lists{};
  // the pending step as launched: the builder's sizes, or their padded shape
  int32_t x_nseq = 0, x_ndec = 0, x_ntok = 0, x_maxctx = 0, x_stride = 0;
  // graph replay
  int32_t pad_q = 0, pad_kv = 0;  // 0: no padding
  bool capture = false;
  std::map<GraphKey, hipGraphExec_t> graphs;
  int64_t n_captures = 0, n_replays = 0;
  int64_t n_scheduled = 0, n_attended = 0;
  int64_t n_slot_waits = 0;  // schedules whose staging slot was still being read, and waited
  int64_t n_cu_split = 0;    // attended steps whose lists chose the CU split
  bool step_cu_split = false;
  void drop_graphs() {
    for (auto& kv : graphs) (void)hipGraphExecDestroy(kv.second);
    graphs.clear();
  }
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
  const int64_t slot_ints = (int64_t)(c.meta_bytes / sizeof(int32_t) / 2) & ~int64_t(3);  // 16-byte slots
  if (slot_ints < 16) return cb::fail(CB_ERR_INVALID, "cb_engine_create: metadata buffers too small");
  cb_engine* e = new (std::nothrow) cb_engine();
  if (!e) return cb::fail(CB_ERR_INVALID, "out of host memory");
  e->cfg = c;
  e->slot_ints = slot_ints;
  if (hipHostGetDevicePointer(reinterpret_cast<void**>(&e->meta_host_dev), c.meta_host, 0) != hipSuccess) {
    (void)hipGetLastError();
    e->meta_host_dev = nullptr;
  }
  int st = cb_builder_create(&c.builder, &e->builder);
  if (st != CB_OK) { delete e; return st; }
  for (int i = 0; i < 2; ++i) {
    // the host only needs to know that the slot's reader finished: no
    // system-scope writeback of device memory when the event is recorded
    if (hipEventCreateWithFlags(&e->copied[i], hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess) {
      cb_engine_destroy(e);
      return cb::fail(CB_ERR_DEVICE, "cb_engine_create: hipEventCreate failed");
    }
  }
  *out = e;
  return CB_OK;
}

void cb_engine_destroy(cb_engine* e) {
  if (!e) return;
  e->drop_graphs();
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
  const int64_t slot_ints = (int64_t)(meta_bytes / sizeof(int32_t) / 2) & ~int64_t(3);
  if (slot_ints < 16) return cb::fail(CB_ERR_INVALID, "cb_engine_set_metadata: buffers too small");
  for (int i = 0; i < 2; ++i)
    if (e->slot_used[i]) (void)hipEventSynchronize(e->copied[i]);
  e->drop_graphs();  // they read the old buffers
  e->cfg.meta_device = meta_device;
  e->cfg.meta_host = meta_host;
  e->cfg.meta_bytes = meta_bytes;
  e->slot_ints = slot_ints;
  if (hipHostGetDevicePointer(reinterpret_cast<void**>(&e->meta_host_dev), meta_host, 0) != hipSuccess) {
    (void)hipGetLastError();
    e->meta_host_dev = nullptr;
  }
  e->slot_used[0] = e->slot_used[1] = false;
  e->slot = 0;
  e->pending = false;
  return CB_OK;
}

int cb_engine_set_workspace(cb_engine* e, void* workspace, size_t workspace_bytes) {
  cb::clear_error();
  if (!e) return cb::fail(CB_ERR_INVALID, "cb_engine_set_workspace: null engine");
  e->drop_graphs();
  e->cfg.workspace = workspace;
  e->cfg.workspace_bytes = workspace ? workspace_bytes : 0;
  return CB_OK;
}

int cb_engine_schedule(cb_engine* e, void* stream, cb_step* out) {
  cb::clear_error();
  if (!e || !out) return cb::fail(CB_ERR_INVALID, "cb_engine_schedule: null argument");
  const cb_builder_config& bc = e->cfg.builder;
  // worst case of this step's metadata, before the builder changes state
  const bool pad = e->pad_q > 0;
  const int64_t B = bc.max_requests_per_batch + (pad ? 18 : 0);
  const int64_t T = bc.max_batch_tokens + (pad ? e->pad_q + 16 : 0);
  const int64_t stride = (int64_t)cb::builder_max_pages_held(e->builder) + cb::ceil_div(T, CB_PAGE_SIZE) + 1 +
                         (pad ? e->pad_kv / CB_PAGE_SIZE + 1 : 0);
  const int64_t bt_pages = pad ? stride : std::min<int64_t>(stride, bc.num_pages);
  int64_t need = 2 * (B + 1) + 2 * B + B * bt_pages + T;
  if (e->cfg.dtype == CB_BF16) {  // bound of the host-built work lists (int32 units)
    const int64_t G = e->cfg.num_q_heads / e->cfg.num_kv_heads;
    const int64_t pages = bt_pages;
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
  if (e->slot_used[slot]) {
    const hipError_t q = hipEventQuery(e->copied[slot]);
    if (q == hipErrorNotReady) {
      e->n_slot_waits++;
      if (hipEventSynchronize(e->copied[slot]) != hipSuccess)
        return cb::fail(CB_ERR_DEVICE, "cb_engine_schedule: waiting for the previous upload failed");
    } else if (q != hipSuccess) {
      return cb::fail(CB_ERR_DEVICE, "cb_engine_schedule: querying the previous upload failed");
    }
  }
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
  size_t o_qsl, o_ctx, o_off, o_bt, o_btoff, o_sl;
  // block tables go up packed: row s holds the ceil(ctx / 16) pages its
  // context covers (all the kernels read), rows back to back after an
  // offsets array; src_row(s) is the descriptor row of launched sequence s
  // (-1: an empty padding sequence)
  auto put_tables = [&](int32_t nseq, auto src_row) {
    o_btoff = off;
    off += (size_t)nseq + 1;
    o_bt = off;
    int32_t acc = 0;
    for (int32_t s = 0; s < nseq; ++s) {
      h[o_btoff + s] = acc;
      const int32_t r = src_row(s);
      if (r < 0) continue;
      const int32_t n = std::min<int32_t>((d.context_lens[r] + CB_PAGE_SIZE - 1) / CB_PAGE_SIZE, d.block_table_stride);
      if (n > 0) std::memcpy(h + off, d.block_tables + (size_t)r * d.block_table_stride, (size_t)n * sizeof(int32_t));
      off += n;
      acc += n;
    }
    h[o_btoff + nseq] = acc;
  };
  if (!pad || d.num_tokens == 0) {
    e->x_nseq = d.num_seqs;
    e->x_ndec = d.num_decodes;
    e->x_ntok = d.num_tokens;
    e->x_maxctx = d.max_context_len;
    e->x_stride = d.block_table_stride;
    o_qsl = put(d.query_start_loc, (size_t)d.num_seqs + 1);
    o_ctx = put(d.context_lens, (size_t)d.num_seqs);
    o_off = put(d.q_offsets, (size_t)d.num_seqs);
    put_tables(d.num_seqs, [](int32_t s) { return s; });
    o_sl = put(d.slot_mapping, (size_t)d.num_tokens);
  } else {
    // padded shape: [decodes | empty | prefills | empty], tokens past the real
    // ones belong to no sequence and are not written (slot -1)
    const int32_t nd = d.num_decodes, np = d.num_seqs - d.num_decodes;
    const int32_t nd_p = round_up(nd, 16), np_p = round_up(np, 4), B_p = nd_p + np_p;
    e->x_nseq = B_p;
    e->x_ndec = nd_p;
    e->x_ntok = std::max(round_up(d.num_tokens, e->pad_q), nd_p);
    e->x_maxctx = round_up(std::max(d.max_context_len, 1), e->pad_kv);
    e->x_stride = e->x_maxctx / CB_PAGE_SIZE;
    auto src_of = [&](int32_t s) { return s < nd ? s : (s >= nd_p && s < nd_p + np ? nd + (s - nd_p) : -1); };
    o_qsl = off;
    for (int32_t s = 0, last = 0; s < B_p; ++s) {
      const int32_t r = src_of(s);
      h[off++] = r >= 0 ? d.query_start_loc[r] : last;
      last = r >= 0 ? d.query_start_loc[r + 1] : last;
    }
    h[off++] = d.num_tokens;
    o_ctx = off;
    for (int32_t s = 0; s < B_p; ++s) h[off++] = src_of(s) >= 0 ? d.context_lens[src_of(s)] : 0;
    o_off = off;
    for (int32_t s = 0; s < B_p; ++s) h[off++] = src_of(s) >= 0 ? d.q_offsets[src_of(s)] : 0;
    put_tables(B_p, src_of);
    // a padded shape keeps the padded tables' room, so that its metadata
    // layout and upload size (which a recorded graph holds) do not change
    off = o_bt + (size_t)B_p * e->x_stride;
    o_sl = put(d.slot_mapping, (size_t)d.num_tokens);
    for (int32_t t = d.num_tokens; t < e->x_ntok; ++t) h[off++] = -1;
  }
  e->have_lists = false;
  e->step_cu_split = false;
  if (e->cfg.dtype == CB_BF16 && e->x_ntok > 0) {
    // the attention step's work lists, built here instead of by a device plan kernel
    cb::Bf16Plan pl = cb::plan_bf16(e->x_nseq, e->x_ndec, e->x_ntok, e->cfg.num_q_heads,
                                    e->cfg.num_kv_heads, e->cfg.head_dim, std::max(e->x_maxctx, 1),
                                    e->cfg.builder.sliding_window);
    pl.slots = cb::mixed_slots(e->cfg.head_dim);  // the lists' block order depends on it
    const cb::WorkListLayout lay = cb::work_list_layout(pl, e->x_ndec);
    const size_t at = (off + 3) & ~size_t(3);  // 16-byte aligned (int32 units)
    if ((int64_t)(at + lay.bytes / 4) <= e->slot_ints) {
      const cb::WorkCounts live = cb::build_work_lists(pl, e->x_nseq, e->x_ndec, e->cfg.num_q_heads / e->cfg.num_kv_heads,
                           e->cfg.builder.sliding_window, h + o_qsl, h + o_ctx, h + o_off, h + at);
      const uint8_t* db = reinterpret_cast<const uint8_t*>(dv + at);
      e->lists.hdr = db + lay.hdr;
      e->lists.dec_items = db + lay.dec_items;
      e->lists.pf_items = db + lay.pf_items;
      e->lists.pf_tiles = db + lay.pf_tiles;
      e->lists.dec_first = reinterpret_cast<const int32_t*>(db + lay.dec_first);
      e->lists.dec_rem = reinterpret_cast<const int32_t*>(db + lay.dec_rem);
      // a recorded graph keeps its grid for every replay: it is sized by the caps
      e->lists.live_pf_items = e->capture ? -1 : live.pf_items;
      e->lists.live_dec_items = e->capture ? -1 : live.dec_items;
      e->lists.pf_split = live.pf_split;
      e->step_cu_split = live.cu_split > 0;
      e->lists.dec_split = live.dec_split;
      e->have_lists = true;
      off = at + lay.bytes / 4;
    }
  }
  if (e->meta_host_dev && e->x_ntok > 0) {
    // the append kernel that starts the step copies the slot up (and reads
    // its slot mapping from here); the staging slot stays busy until it ran
    e->pull_ints = (int64_t)((off + 3) & ~size_t(3));
    e->h_slots_dev = e->meta_host_dev + (size_t)slot * e->slot_ints + o_sl;
  } else {
    e->pull_ints = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(dv, h, off * sizeof(int32_t), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipEventRecord(e->copied[slot], s) != hipSuccess)
      return cb::fail(CB_ERR_DEVICE, "cb_engine_schedule: metadata upload failed");
    e->slot_used[slot] = true;
  }
  e->slot = slot;
  e->pending = true;
  e->n_scheduled++;
  e->d_qsl = dv + o_qsl;
  e->d_ctx = dv + o_ctx;
  e->d_off = dv + o_off;
  e->d_bt = dv + o_bt;
  e->d_btoff = dv + o_btoff;
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
  return cb_attention_workspace_bytes(e->x_nseq, e->x_ndec, e->x_ntok, e->cfg.num_q_heads, e->cfg.num_kv_heads,
                                      e->cfg.head_dim, std::max(e->x_maxctx, 1), e->cfg.dtype);
}

int32_t cb_engine_padded_tokens(const cb_engine* e) { return e && e->pending ? e->x_ntok : 0; }

int cb_engine_set_graphs(cb_engine* e, int32_t q_padding_interval, int32_t kv_padding_interval,
                         int32_t capture) {
  cb::clear_error();
  if (!e) return cb::fail(CB_ERR_INVALID, "cb_engine_set_graphs: null engine");
  const bool off = q_padding_interval == 0 && kv_padding_interval == 0;
  if (!off && (q_padding_interval < 1 || kv_padding_interval < CB_PAGE_SIZE ||
               kv_padding_interval % CB_PAGE_SIZE != 0))
    return cb::fail(CB_ERR_INVALID, "padding intervals: q >= 1 and kv a positive multiple of %d (or both 0)",
                    CB_PAGE_SIZE);
  if (off && capture) return cb::fail(CB_ERR_INVALID, "graph capture needs padding intervals");
  e->drop_graphs();
  e->pad_q = q_padding_interval;
  e->pad_kv = kv_padding_interval;
  e->capture = capture != 0;
  e->pending = false;
  return CB_OK;
}

int cb_engine_graph_stats(const cb_engine* e, int64_t* captures, int64_t* replays, int64_t* cached) {
  cb::clear_error();
  if (!e || !captures || !replays || !cached) return cb::fail(CB_ERR_INVALID, "cb_engine_graph_stats: null argument");
  *captures = e->n_captures;
  *replays = e->n_replays;
  *cached = (int64_t)e->graphs.size();
  return CB_OK;
}

int cb_engine_stats_get(const cb_engine* e, cb_engine_stats* out) {
  cb::clear_error();
  if (!e || !out) return cb::fail(CB_ERR_INVALID, "cb_engine_stats_get: null argument");
  out->steps_scheduled = e->n_scheduled;
  out->steps_attended = e->n_attended;
  out->slot_waits = e->n_slot_waits;
  out->graph_captures = e->n_captures;
  out->graph_replays = e->n_replays;
  out->graphs_cached = (int64_t)e->graphs.size();
  out->cu_split_steps = e->n_cu_split;
  return CB_OK;
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
  const hipStream_t hs0 = static_cast<hipStream_t>(stream);
  int32_t* dslot = c.meta_device + (size_t)e->slot * e->slot_ints;
  auto launch = [&]() {
    int rc;
    if (e->pull_ints > 0) {
      const hipError_t err = cb::launch_kv_append_pull(
          k_new, v_new, c.k_cache, c.v_cache, e->h_slots_dev, e->x_ntok, c.num_kv_heads, c.head_dim,
          c.builder.num_pages, c.dtype == CB_BF16 ? 2 : 4, e->meta_host_dev + (size_t)e->slot * e->slot_ints,
          dslot, e->pull_ints * 4, hs0);
      rc = err == hipSuccess ? CB_OK : cb::fail(CB_ERR_DEVICE, "append launch failed: %s", hipGetErrorString(err));
    } else {
      rc = cb_kv_append(k_new, v_new, c.k_cache, c.v_cache, e->d_slots, e->x_ntok, c.num_kv_heads, c.head_dim,
                        c.builder.num_pages, CB_PAGE_SIZE, c.dtype, stream);
    }
    if (rc != CB_OK) return rc;
    return cb::attention_step_impl(q, c.k_cache, c.v_cache, e->d_bt, e->x_stride, e->d_qsl, e->d_ctx, e->d_off,
                                   e->x_nseq, e->x_ndec, e->x_ntok, e->x_maxctx, c.num_q_heads,
                                   c.num_kv_heads, c.head_dim, CB_PAGE_SIZE, c.builder.num_pages, c.scale,
                                   c.builder.sliding_window, c.dtype, out, c.workspace, c.workspace_bytes,
                                   stream, e->have_lists ? &e->lists : nullptr, e->d_btoff);
  };
  // with the pull, the staging slot is free once the append kernel has run
  auto staged = [&]() {
    if (e->pull_ints == 0) return (int)CB_OK;
    if (hipEventRecord(e->copied[e->slot], hs0) != hipSuccess)
      return cb::fail(CB_ERR_DEVICE, "cb_engine_attend: event record failed");
    e->slot_used[e->slot] = true;
    return (int)CB_OK;
  };
  if (!e->capture) {
    int st = launch();
    if (st == CB_OK) st = staged();
    if (st == CB_OK) {
      e->pending = false;
      e->n_attended++;
      if (e->have_lists && e->step_cu_split) e->n_cu_split++;
    }
    return st;
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const GraphKey key{e->slot, e->x_nseq, e->x_ndec, e->x_ntok, e->x_maxctx, e->x_stride, e->pull_ints,
                     q, k_new, v_new, out, c.workspace, c.workspace_bytes};
  auto it = e->graphs.find(key);
  if (it == e->graphs.end()) {
    if (e->graphs.size() >= kMaxGraphs) e->drop_graphs();
    cb::ProfileEventsOff quiet;  // no event records inside a captured graph
    if (hipStreamBeginCapture(hs, hipStreamCaptureModeThreadLocal) != hipSuccess)
      return cb::fail(CB_ERR_DEVICE, "cb_engine_attend: stream capture could not begin");
    const int st = launch();
    hipGraph_t graph = nullptr;
    const hipError_t end = hipStreamEndCapture(hs, &graph);
    if (st != CB_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return st;
    }
    hipGraphExec_t exec = nullptr;
    if (end != hipSuccess || !graph || hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      return cb::fail(CB_ERR_DEVICE, "cb_engine_attend: graph capture failed");
    }
    (void)hipGraphDestroy(graph);
    it = e->graphs.emplace(key, exec).first;
    e->n_captures++;
  }
  if (hipGraphLaunch(it->second, hs) != hipSuccess)
    return cb::fail(CB_ERR_DEVICE, "cb_engine_attend: graph launch failed");
  e->n_replays++;
  const int st = staged();
  if (st == CB_OK) {
    e->pending = false;
    e->n_attended++;
    if (e->have_lists && e->step_cu_split) e->n_cu_split++;
  }
  return st;
}

}  // extern "C"
