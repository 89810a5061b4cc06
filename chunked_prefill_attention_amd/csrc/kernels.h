// Host-side interface of the device code: launch helpers and the layout of
// the attention workspace.  Everything here runs on the host; the kernels
// live in the .hip files.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace cb {

// Events recorded around the main attention kernel (cb_profile_events);
// null when profiling is off.  Per host thread.
extern thread_local hipEvent_t g_prof_start;
extern thread_local hipEvent_t g_prof_stop;
// Device buffer of 4 uint64 for the main kernel's clock record (null: off).
extern thread_local void* g_prof_clock;
// Suspends the profiling events of this thread for a scope (graph capture).
struct ProfileEventsOff {
  hipEvent_t start = g_prof_start, stop = g_prof_stop;
  void* clock = g_prof_clock;
  ProfileEventsOff() { g_prof_start = g_prof_stop = nullptr; g_prof_clock = nullptr; }
  ~ProfileEventsOff() { g_prof_start = start; g_prof_stop = stop; g_prof_clock = clock; }
};

// Arguments of one attention step, already validated on the host.
struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t bt_stride;
  // row s of the block tables starts at bt_offsets[s] when set (rows packed
  // back to back, each as long as its context), else at s * bt_stride
  const int32_t* bt_offsets;
  const int32_t* qsl;
  const int32_t* ctx_lens;
  const int32_t* q_offsets;
  int32_t num_seqs, num_decodes, num_tokens, max_context_len;
  int32_t hq, hkv, head_dim, num_pages;
  float scale;
  int32_t window;   // sliding window in tokens (keys p-window < j <= p); 0 = none
  void* out;
  void* workspace;
};

// Sizing of the bf16 path's workspace; a pure function of host scalars so
// that cb_attention_workspace_bytes and cb_attention_step agree.
struct Bf16Plan {
  int32_t split_pages;    // pages per decode wavefront (split-K unit)
  int32_t pf_split_keys;  // keys per prefill workgroup (split-K unit of a row tile)
  bool pf_may_split;      // some prefill row tile may need more than one split
  int64_t dec_cap;        // bound on (sequence, split) decode items
  int64_t pf_tile_cap;    // bound on (sequence, 128-row tile) prefill tiles
  int64_t pf_item_cap;    // bound on (tile, key split) prefill items
  int32_t hkv;            // KV heads (workgroups per prefill item)
  int32_t slots;          // workgroups of the mixed launch the device holds at once (0: ask the
                          // device at launch; the host list builder needs it set, see mixed_slots)
  size_t off_hdr, off_dec_items, off_pf_items, off_pf_tiles, off_dec_first, off_dec_rem;
  size_t off_dec_ml, off_dec_o, off_pf_ml, off_pf_o;
  size_t bytes;
};
// Workgroups of the mixed launch the current device holds at once (its
// occupancy per CU times the CU count; queried once per device and head size).
int mixed_slots(int head_dim);
Bf16Plan plan_bf16(int32_t num_seqs, int32_t num_decodes, int32_t num_tokens, int32_t hq,
                   int32_t hkv, int32_t head_dim, int32_t max_context_len, int32_t window = 0);

// Work lists of one bf16 step built by the caller (the engine builds them on
// the host and uploads them with the step's metadata); when given, the
// device plan kernel is skipped.
struct WorkLists {
  const void* hdr;           // int4 (live prefill items, live decode items, block order, prefill CUs per
                             // shader engine), then the CU split's claim queues (zero)
  int64_t live_pf_items = -1;   // when >= 0 (the caller built the lists and is not recording a
  int64_t live_dec_items = -1;  // graph), the launch sizes its grid to the live work
  bool pf_split = true;         // with live counts: whether any prefill tile / decode has more than
  bool dec_split = true;        // one split (the combine launch skips the kind that has none)
  const void* dec_items;     // int4 [dec_cap]: (sequence, split, context, query row); -1 = none
  const void* pf_items;      // int4 [pf_item_cap]: (sequence, row tile, key split, partial slot)
  const void* pf_tiles;      // int4 [pf_tile_cap]: (sequence, row tile, first item, splits)
  const int32_t* dec_first;  // [num_decodes]
  const int32_t* dec_rem;    // [num_decodes]
};

// Host layout of the work lists: byte offsets inside one buffer (16-byte aligned).
struct WorkListLayout {
  size_t hdr, dec_items, pf_items, pf_tiles, dec_first, dec_rem, bytes;
};
WorkListLayout work_list_layout(const Bf16Plan& pl, int32_t num_decodes);

// Host version of the plan kernel (same lists, same order): fills `dst`
// (laid out by work_list_layout) from the host copies of query_start_loc,
// context_lens and q_offsets.
struct WorkCounts {
  int64_t pf_items, dec_items;  // live prefill and decode items in the lists
  bool pf_split, dec_split;     // some prefill row tile / some decode has more than one split
  int cu_split;                 // prefill CUs per shader engine chosen for the CU split (0: none)
};
WorkCounts build_work_lists(const Bf16Plan& pl, int32_t num_seqs, int32_t num_decodes, int32_t group,
                      int32_t window, const int32_t* qsl, const int32_t* ctx, const int32_t* q_off,
                      void* dst);

// The same append, plus a copy of pull_bytes (a multiple of 16) from pull_src
// (device-readable host memory) to pull_dst, done by extra blocks of the launch.
hipError_t launch_kv_append_pull(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 const int32_t* slots, int32_t T, int32_t hkv, int32_t head_dim,
                                 int32_t num_pages, int32_t elem_bytes, const void* pull_src, void* pull_dst,
                                 int64_t pull_bytes, hipStream_t stream);
hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* slots, int32_t num_tokens, int32_t hkv, int32_t head_dim,
                            int32_t num_pages, int32_t elem_bytes, hipStream_t stream);
hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attention_bf16(const AttnArgs& a, const Bf16Plan& plan, const WorkLists* lists,
                                 hipStream_t stream);

}  // namespace cb
