/*
 * cb.h -- C ABI of the chunked-prefill + decode paged-attention step for
 * AMD Instinct MI355X (gfx950).
 *
 * One engine step of a continuous-batching server runs, for one attention
 * layer:
 *   1. cb_builder_step     host: choose this step's requests and tokens,
 *                          allocate KV pages, emit the ragged step descriptor;
 *   2. cb_kv_append        device: write this step's K/V rows into the pages
 *                          through the slot mapping;
 *   3. cb_attention_step   device: one ragged launch in which every query row
 *                          (decode tokens and prefill-chunk tokens alike)
 *                          attends causally to its own sequence's KV history.
 *
 * Sources of the semantics (the web pages this library is built from):
 *   [GLOSS]  Ultralytics glossary, "Chunked Prefill": section "How chunked
 *            prefill works" -- each chunk attends, under a causal mask over
 *            absolute positions, to the cached K/V of all earlier chunks plus
 *            itself; the result equals one-shot prefill.  Also the scheduling
 *            rule: one token per running decode, then chunks of waiting
 *            prompts fill the remaining token budget.
 *   [CBA]    Hugging Face transformers, "Continuous batching architecture":
 *            sections "Request lifecycle", "Chunked prefill", "Scheduler",
 *            "FIFO", "PrefillFirst", "Memory management", "Admission",
 *            "Prefix caching" and the release of cached blocks under
 *            "Eviction".
 *   [VLLM]   AI Engineering from Scratch, "vLLM serving internals": sections
 *            "PagedAttention as virtual memory" (16-token blocks, per-sequence
 *            block tables) and "What the scheduler looks like".
 *   [TNG]    TNG blog post on prefill/decode interference, "Request-parallel
 *            prefill": several prefills per step, few of them long.
 *
 * Conventions for every call:
 *   - No call allocates device memory, synchronises the device or blocks on
 *     the stream; device work is enqueued on `stream` (a hipStream_t passed as
 *     void*; NULL means the default stream) on the caller's current device.
 *   - Pointers named "device" must be device memory owned by the caller and
 *     stay valid until the enqueued work completes.  Pointers named "host"
 *     are read before the call returns.
 *   - Every call returns a status (CB_OK or a negative CB_ERR_*).  On error,
 *     nothing has been enqueued (except CB_ERR_DEVICE, which reports a failed
 *     launch) and cb_last_error() holds a thread-local message.
 *   - Page size is fixed at 16 tokens ([VLLM] "PagedAttention as virtual
 *     memory": default block of 16 tokens).
 *
 * KV cache layout (one attention layer; pages are the physical blocks):
 *   k_cache[num_pages][Hkv][16][D]   token-major within a (page, head) slab
 *   v_cache[num_pages][Hkv][D][16]   token-minor within a (page, head) slab
 *   slot = page * 16 + offset; logical position p of sequence s lives in slot
 *   block_tables[s * stride + p / 16] * 16 + p % 16.
 * Element type: float32 (CB_F32) or bfloat16 bits (CB_BF16), same for q, k,
 * v and out.
 */
#ifndef CB_H
#define CB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----------------------------------------------------------------------------
 * Status and types
 * ------------------------------------------------------------------------- */
enum {
  CB_OK = 0,
  CB_ERR_INVALID = -1,     /* null pointer, negative size, inconsistent shape  */
  CB_ERR_UNSUPPORTED = -2, /* head_dim, page_size, dtype or group size not built */
  CB_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required        */
  CB_ERR_DEVICE = -4,      /* a kernel launch failed (hipGetLastError)          */
  CB_ERR_CAPACITY = -5     /* a request can never fit the page pool             */
};

enum { CB_F32 = 0, CB_BF16 = 1 };

#define CB_PAGE_SIZE 16

/* Short static name of a status code ("CB_OK", "CB_ERR_INVALID", ...). */
const char* cb_status_string(int status);

/* Detail of the last error on the calling thread; "" if none.  Valid until the
 * thread's next cb_* call. */
const char* cb_last_error(void);

/* ABI version of this header (increments on incompatible change). */
int cb_abi_version(void);

/* ----------------------------------------------------------------------------
 * cb_kv_append -- write this step's new K/V rows into their cache slots.
 *
 * [GLOSS] "How chunked prefill works": a chunk's own keys and values are
 * cached before it attends, and later chunks read them from the cache.
 * [VLLM] "PagedAttention as virtual memory": slots live in fixed 16-token
 * blocks mapped through the sequence's block table.
 *
 *   k_new, v_new   device, [num_tokens][num_kv_heads][head_dim], contiguous
 *   k_cache        device, [num_pages][num_kv_heads][16][head_dim]
 *   v_cache        device, [num_pages][num_kv_heads][head_dim][16]
 *   slot_mapping   device int32 [num_tokens]; token t goes to slot
 *                  slot_mapping[t]; a negative slot writes nothing (padding).
 *   dtype          CB_F32 or CB_BF16; rows are copied bit for bit.
 *
 * Preconditions on device data (not checked on the host, which never reads
 * device memory): no two tokens name one slot.  A slot >= num_pages * 16 is
 * skipped by the kernel rather than written out of bounds.
 * Errors: CB_ERR_INVALID (null pointer with num_tokens > 0, negative sizes,
 * num_pages * 16 >= 2^31), CB_ERR_UNSUPPORTED (page_size != 16, head_dim not
 * 64 or 128, unknown dtype), CB_ERR_DEVICE.  num_tokens == 0 is a no-op.
 * ------------------------------------------------------------------------- */
int cb_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                 int32_t head_dim, int32_t num_pages, int32_t page_size, int32_t dtype,
                 void* stream);

/* ----------------------------------------------------------------------------
 * cb_attention_workspace_bytes -- device scratch that cb_attention_step needs.
 *
 * Host-only arithmetic on the same scalars cb_attention_step receives; an
 * upper bound for the step's work lists and split-K partial results.  Returns
 * 0 when no workspace is needed, and (size_t)-1 for invalid arguments.
 * ------------------------------------------------------------------------- */
size_t cb_attention_workspace_bytes(int32_t num_seqs, int32_t num_decodes, int32_t num_tokens,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_context_len, int32_t dtype);

/* ----------------------------------------------------------------------------
 * cb_attention_step -- causal attention of every query row of the step.
 *
 * [GLOSS] "How chunked prefill works": query row i of sequence s sits at
 * absolute position p = q_offsets[s] + i and attends to logical KV positions
 * 0..p (inclusive) of the same sequence; with
 *   x_j = scale * <q_row, k_j>,  w_j = exp(x_j - max x),  out = sum w_j v_j / sum w_j.
 * Decode requests are one-token chunks ([CBA] "Request lifecycle").
 *
 *   q, out            device, [num_tokens][num_q_heads][head_dim]
 *   k_cache, v_cache  device, layouts in the header comment; they must already
 *                     hold this step's tokens (cb_kv_append on the same
 *                     stream first)
 *   block_tables      device int32 [num_seqs][block_table_stride]; entries
 *                     past ceil(context_lens[s]/16) are never read
 *   query_start_loc   device int32 [num_seqs + 1]; sequence s owns query rows
 *                     query_start_loc[s] .. query_start_loc[s+1]-1; [0] = 0
 *                     and [num_seqs] = num_tokens
 *   context_lens      device int32 [num_seqs]; KV length including this step
 *   q_offsets         device int32 [num_seqs]; = context_lens - q_len
 *   num_decodes       the first num_decodes sequences have q_len == 1 and take
 *                     the split-K decode path; the rest take the prefill-tile
 *                     path (any q_len >= 0, including 1)
 *   max_context_len   host upper bound of context_lens (sizes the grid)
 *   Grouped-query mapping: query head h reads KV head h / (Hq / Hkv).
 *   scale             softmax scale (1/sqrt(head_dim) by convention); finite;
 *                     the bf16 path requires scale > 0 (its online softmax
 *                     tracks the maximum raw score, which orders like the
 *                     scaled scores only for a positive scale)
 *   sliding_window    0 for full causal attention; W > 0 restricts row p to
 *                     keys p-W < j <= p ([CBA] "Memory management": sliding
 *                     layers keep only a fixed window of recent tokens).  Block
 *                     table entries for pages wholly below the window of a
 *                     sequence's first query row in the step are never read
 *                     (they may be -1), and cache slots below that window do
 *                     not affect any row, NaN included.  Slots from there up
 *                     to a later row's own window start get weight zero in
 *                     that row but must hold finite values (the rows of a
 *                     prefill tile share one P V product, so 0 * NaN would
 *                     reach them); the builder's release rule keeps them so
 *   workspace         device, >= cb_attention_workspace_bytes(...) bytes
 *                     (may be NULL when that is 0); contents on entry do not
 *                     matter; two calls that share a workspace must be
 *                     ordered on one stream
 *
 * Values in cache slots at or past context_lens[s] (or NaN there) do not
 * affect the output.  A page id >= num_pages (a broken precondition) is read
 * as page 0 instead of faulting; the output is then unspecified.  Device-side preconditions that are not checked: the
 * query_start_loc / context_lens / q_offsets relations above and
 * context_lens <= max_context_len.
 * Errors: CB_ERR_INVALID (null pointers, negative or inconsistent sizes,
 * sliding_window < 0, Hq % Hkv != 0, stride < ceil(max_context_len/16)), CB_ERR_UNSUPPORTED
 * (page_size != 16, head_dim not 64/128, group size Hq/Hkv > 16, dtype),
 * CB_ERR_WORKSPACE, CB_ERR_DEVICE.  num_tokens == 0 is a no-op.
 * ------------------------------------------------------------------------- */
int cb_attention_step(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t block_table_stride,
                      const int32_t* query_start_loc, const int32_t* context_lens,
                      const int32_t* q_offsets, int32_t num_seqs, int32_t num_decodes,
                      int32_t num_tokens, int32_t max_context_len, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t num_pages, float scale, int32_t sliding_window, int32_t dtype,
                      void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * cb_attention_step_noalloc -- cb_attention_step for callers that cannot
 * allocate device memory (work recorded under graph capture, tight serving
 * loops, harnesses that forbid allocation).
 *
 * Same arguments, semantics, errors and kernels as cb_attention_step, without
 * the workspace: the bf16 path's work lists and split-K partial results live
 * in a fixed device array of CB_NOALLOC_SCRATCH_BYTES that the library holds
 * on every device it runs on until the process ends.  Nothing is allocated
 * or freed by the call.  A step whose cb_attention_workspace_bytes exceeds
 * the array is refused with CB_ERR_WORKSPACE before any device work.  The
 * array's contents on entry do not matter (every list and partial a step
 * reads is written by that step first); all calls on one device share it, so
 * calls ordered on one stream are safe and calls that overlap on one device
 * (unordered streams) race.  The f32 path needs no scratch.
 * ------------------------------------------------------------------------- */
#define CB_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

int cb_attention_step_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* query_start_loc, const int32_t* context_lens,
                              const int32_t* q_offsets, int32_t num_seqs, int32_t num_decodes,
                              int32_t num_tokens, int32_t max_context_len, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t num_pages, float scale, int32_t sliding_window, int32_t dtype,
                              void* out, void* stream);

/* Size of that array in bytes (CB_NOALLOC_SCRATCH_BYTES). */
size_t cb_attention_noalloc_scratch_bytes(void);

/* ----------------------------------------------------------------------------
 * cb_profile_events -- timing hook for the main attention kernel.
 *
 * Not on the pages; a measurement aid.  start_event / stop_event are
 * hipEvent_t handles (passed as void*) that the caller created with timing
 * enabled.  Subsequent cb_attention_step calls made by the calling thread
 * record start_event on their stream right before the main ragged attention
 * kernel and stop_event right after it, so hipEventElapsedTime gives that
 * kernel's duration alone (plan and combine kernels excluded).  Passing NULL,
 * NULL turns the hook off.  Host bookkeeping only; returns CB_OK, or
 * CB_ERR_INVALID when exactly one handle is NULL.
 * ------------------------------------------------------------------------- */
int cb_profile_events(void* start_event, void* stop_event);

/* ----------------------------------------------------------------------------
 * cb_profile_clock -- clock record of the main attention kernel.
 *
 * Not on the pages; a measurement aid.  device_buffer is caller-owned device
 * memory of 4 uint64 (or NULL to turn the hook off).  Subsequent
 * cb_attention_step calls made by the calling thread have workgroup 0 of the
 * main bf16 attention kernel write, at its start and at its end, the shader
 * clock counter (s_memtime) and the 100 MHz real-time counter
 * (s_memrealtime): {cycles0, ticks0, cycles1, ticks1}.  The shader clock in
 * MHz over that workgroup's life is (cycles1 - cycles0) * 100 / (ticks1 -
 * ticks0).  Host bookkeeping only; returns CB_OK.
 * ------------------------------------------------------------------------- */
int cb_profile_clock(void* device_buffer);

/* ----------------------------------------------------------------------------
 * FIFO batch builder (host only; touches no device).
 *
 * [CBA] "Scheduler": three limits per forward pass -- the token budget
 * (max_batch_tokens), the cache budget (KV pages) and the request cap
 * (max_requests_per_batch).  [CBA] "FIFO": active decodes first, then active
 * prefills, then waiting requests in arrival order.  [CBA] "Chunked
 * prefill": a prompt beyond the remaining budget takes every token that
 * still fits and resumes in the next step.  [CBA] "Admission": a request that
 * cannot be held is not admitted and nothing is allocated; below
 * safety_margin of free pages new prefills wait while active work continues.
 * [VLLM] "What the scheduler looks like": finished requests release their
 * blocks at the top of the step; the head of the waiting queue is admitted
 * while it fits (strict head of line).
 *
 * Chunk length = min(remaining prompt, remaining token budget,
 * max_prefill_chunk if > 0).  An active prefill is cut further to what its
 * held plus free pages can hold (stalled if that is 0).  A decode whose cached
 * length is a multiple of 16 needs one new page; with none free it is stalled
 * (skipped this step).  A waiting request is admitted only if its first
 * chunk's pages are free and free - needed >= safety_margin * num_pages.
 * The prefill step that completes a prompt yields output token 1; each decode
 * step yields one more; a request finishing in a step is released (pages
 * freed, id reported) at the start of the next step.
 * ------------------------------------------------------------------------- */
typedef struct cb_builder cb_builder;

/* Scheduling policies.  [CBA] "FIFO": active decodes, then active prefills,
 * then waiting requests.  [CBA] "PrefillFirst": split prefills are carried to
 * completion before decoding resumes -- here active prefills are picked
 * first, then active decodes, then waiting requests.  Under both the step
 * lists its decodes first. */
enum { CB_POLICY_FIFO = 0, CB_POLICY_PREFILL_FIRST = 1 };

typedef struct {
  int32_t max_batch_tokens;       /* >= 1 */
  int32_t max_requests_per_batch; /* >= 1 */
  int32_t num_pages;              /* pool size, >= 1, num_pages * 16 < 2^31 */
  int32_t page_size;              /* must be 16 */
  int32_t max_prefill_chunk;      /* 0 = no cap */
  float safety_margin;            /* in [0, 1); 0 disables the margin */
  uint64_t page_shuffle_seed;     /* 0: pages handed out 0, 1, 2, ...; else the
                                     initial free list is a seeded permutation */
  int32_t policy;                 /* CB_POLICY_* */
  /* [TNG] request-parallel prefill: prefill chunks per step (0 = no cap) and,
   * among them, chunks of prompts longer than long_prefill_threshold tokens
   * (0 = no cap).  A prefill over a cap is skipped, not stalled, and the
   * requests behind it are still considered. */
  int32_t max_partial_prefills;
  int32_t max_long_partial_prefills;
  int32_t long_prefill_threshold;
  /* [CBA] "Prefix caching": nonzero lets requests submitted with their prompt
   * tokens (cb_builder_submit_tokens) reuse registered full prompt blocks;
   * see cb_builder_submit_tokens. */
  int32_t allow_block_sharing;
  /* [CBA] "Memory management": sliding-window layers keep only the most
   * recent tokens and recycle their pages.  With sliding_window = W > 0 a
   * query at position p sees keys p-W < j <= p (pass the same W to
   * cb_attention_step); at the start of each step a request releases the
   * pages wholly below cached - W + 1, leaving -1 in its block table; an
   * import allocates only the pages inside its window; the "never fits"
   * check uses the window plus one chunk.  Incompatible with
   * allow_block_sharing (CB_ERR_INVALID).  0 = full attention. */
  int32_t sliding_window;
} cb_builder_config;

/* The step descriptor.  Arrays are owned by the builder and stay valid until
 * the next cb_builder_step / cb_builder_destroy on the same builder. */
typedef struct {
  int32_t num_seqs;           /* scheduled sequences; decodes come first */
  int32_t num_decodes;
  int32_t num_tokens;         /* sum of q_len */
  int32_t max_query_len;
  int32_t max_context_len;
  int32_t block_table_stride; /* max pages held by a scheduled sequence (>= 1) */
  int32_t num_finished;       /* released at the start of this step */
  int32_t num_stalled;
  int32_t new_pages;          /* pages taken from the free pool this step */
  int32_t prefix_hit_tokens;  /* prompt tokens reused from shared blocks this step */
  const int64_t* req_ids;         /* [num_seqs] */
  const int32_t* query_start_loc; /* [num_seqs + 1] */
  const int32_t* context_lens;    /* [num_seqs] */
  const int32_t* q_offsets;       /* [num_seqs] */
  const int32_t* block_tables;    /* [num_seqs * block_table_stride], unused = 0 */
  const int32_t* slot_mapping;    /* [num_tokens] */
  const int64_t* finished_ids;    /* [num_finished] */
  const int64_t* stalled_ids;     /* [num_stalled] */
} cb_step;

typedef struct {
  int32_t num_pages;
  int32_t free_pages;
  int32_t num_waiting;
  int32_t num_prefilling;
  int32_t num_decoding;
  int32_t num_finished_pending; /* finished, pages released next step */
  int64_t used_slots;           /* sum of cached tokens of live requests */
  int64_t allocated_slots;      /* pages in use * 16 */
  int64_t steps;
  int64_t total_stalls;
  int64_t total_finished;
  double fragmentation;         /* (allocated - used) / allocated; 0 if none */
  int64_t prefix_hit_tokens;    /* prompt tokens reused from shared blocks so far */
  int32_t cached_pages;         /* free pages still holding a registered block */
} cb_builder_stats;

/* Create a builder.  Errors: CB_ERR_INVALID (null, bad budget or margin),
 * CB_ERR_UNSUPPORTED (page_size != 16). */
int cb_builder_create(const cb_builder_config* config, cb_builder** out);

/* Deep copy of a builder's whole state (requests, pages, free list). */
int cb_builder_clone(const cb_builder* b, cb_builder** out);

void cb_builder_destroy(cb_builder* b);

/* Submit a request.  tokens_cached == 0: it waits in arrival order.
 * tokens_cached > 0 imports an in-flight request whose pages are allocated
 * now (the caller writes their K/V, slots from cb_builder_block_table): an
 * active prefill if tokens_cached < prompt_len, else a decode that has
 * produced tokens_cached - prompt_len + 1 output tokens.
 * Errors: CB_ERR_INVALID (duplicate id, prompt_len < 1, output_len < 1,
 * tokens_cached < 0, nothing left to do), CB_ERR_CAPACITY
 * (ceil((prompt_len + output_len - 1) / 16) > num_pages, or an import whose
 * pages are not free). */
int cb_builder_submit(cb_builder* b, int64_t req_id, int32_t prompt_len, int32_t output_len,
                      int32_t tokens_cached);

/* Submit a new request together with its prompt tokens (host array of
 * prompt_len ids, copied).  With allow_block_sharing set, at admission the
 * request reuses the longest chain of registered full blocks that matches
 * its prompt, stopping short of the last prompt token (always computed), and
 * its first chunk starts at the matched offset.  A block's identity is its 16
 * tokens together with the block before it; blocks wholly inside the prompt
 * are registered, in order, when the step that fills them is built, until
 * the first one whose identity is already registered.  Shared pages are
 * reference counted; a released registered block stays matchable until an
 * allocation finds no page without a registration and takes the most
 * recently released one.  Reused pages that no request held count against
 * the free pages at admission.  Without sharing this is cb_builder_submit
 * with tokens_cached = 0.
 * Errors: as cb_builder_submit, and CB_ERR_INVALID for a null token array. */
int cb_builder_submit_tokens(cb_builder* b, int64_t req_id, const int32_t* tokens, int32_t prompt_len,
                             int32_t output_len);

/* Run the scheduler for one engine step and fill *out.  A step with nothing
 * schedulable returns CB_OK with num_seqs == 0. */
int cb_builder_step(cb_builder* b, cb_step* out);

/* Copy request req_id's block table (physical page ids in logical order) into
 * out[0 .. cap-1]; *n receives the number of pages it holds.
 * Errors: CB_ERR_INVALID (unknown id, null pointers). */
int cb_builder_block_table(const cb_builder* b, int64_t req_id, int32_t* out, int32_t cap,
                           int32_t* n);

/* Slot mapping of logical positions start .. end-1 of request req_id, for
 * writing their K/V with cb_kv_append (e.g. the history of an imported
 * request).  [VLLM] "PagedAttention as virtual memory": position p lives in
 * slot block_table[p / 16] * 16 + p % 16.  out (host int32, end - start
 * entries, caller-owned) receives the slots; nothing is written on error.
 * Errors: CB_ERR_INVALID (unknown id, null out with end > start, start < 0,
 * end < start, a position whose page the request does not hold -- past its
 * block table or released below a sliding window). */
int cb_builder_slots(const cb_builder* b, int64_t req_id, int32_t start, int32_t end, int32_t* out);

int cb_builder_stats_get(const cb_builder* b, cb_builder_stats* out);


/* ----------------------------------------------------------------------------
 * Engine: the whole per-layer step in native code.
 *
 * [VLLM] "What the scheduler looks like": each iteration schedules decode
 * tokens and prefill chunks and runs them as one fused GPU call; [CBA]
 * "Continuous batching architecture" lists the CPU overhead of batch assembly
 * and dispatch as per-step cost.  The engine owns a FIFO builder and uses
 * caller-provided buffers only (it allocates no device or pinned memory):
 *
 *   cb_engine_schedule  host: builder step, descriptor written into a pinned
 *                       staging slot;
 *   cb_engine_attend    device: one launch appends the step's K/V rows and,
 *                       in extra workgroups, copies the staging slot into a
 *                       device metadata slot (the kernel reads the pinned
 *                       buffer through its device mapping); then
 *                       cb_attention_step, on `stream`.
 *
 * When the pinned buffer has no device mapping, cb_engine_schedule instead
 * enqueues a host-to-device copy of the slot on `stream`.  Two
 * staging/metadata slots alternate, so the host can schedule step N+1 while
 * step N runs; before reusing a staging slot the engine waits (on the host)
 * for the kernel or copy that last read it.  All steps of one engine must be enqueued on
 * one stream.  The caller computes q, k_new, v_new of the scheduled tokens
 * (rows in the descriptor's order) between the two calls.
 * ------------------------------------------------------------------------- */
typedef struct cb_engine cb_engine;

typedef struct {
  cb_builder_config builder;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;              /* CB_F32 or CB_BF16 */
  float scale;                /* softmax scale */
  void* k_cache;              /* device, [builder.num_pages][Hkv][16][D] */
  void* v_cache;              /* device, [builder.num_pages][Hkv][D][16] */
  int32_t* meta_device;       /* device int32 buffer, two slots */
  int32_t* meta_host;         /* pinned host int32 buffer, two slots */
  size_t meta_bytes;          /* bytes of each of meta_device and meta_host */
  void* workspace;            /* device, for cb_attention_step (may be NULL) */
  size_t workspace_bytes;
} cb_engine_config;

/* Errors: CB_ERR_INVALID (null buffers, bad shapes), CB_ERR_UNSUPPORTED,
 * CB_ERR_DEVICE (event creation failed). */
int cb_engine_create(const cb_engine_config* config, cb_engine** out);
void cb_engine_destroy(cb_engine* e);

/* The engine's builder (owned by the engine): submit requests, read block
 * tables and stats through the cb_builder_* calls. */
cb_builder* cb_engine_builder(cb_engine* e);

/* Replace the metadata buffers (e.g. after CB_ERR_CAPACITY).  The caller must
 * make sure no upload or kernel still uses the old buffers (synchronise the
 * stream first).  A scheduled step that was not attended is dropped. */
int cb_engine_set_metadata(cb_engine* e, int32_t* meta_device, int32_t* meta_host, size_t meta_bytes);

/* Replace the workspace (e.g. after CB_ERR_WORKSPACE from cb_engine_attend). */
int cb_engine_set_workspace(cb_engine* e, void* workspace, size_t workspace_bytes);

/* Schedule one step and enqueue its metadata upload on `stream`.  *out is the
 * host descriptor (builder-owned arrays, valid until the next schedule).
 * Errors: CB_ERR_CAPACITY when the step's metadata could exceed one slot
 * (checked before the builder runs, so the state is unchanged), CB_ERR_DEVICE. */
int cb_engine_schedule(cb_engine* e, void* stream, cb_step* out);

/* Append the scheduled tokens' K/V and run the attention step on `stream`.
 * q, out: device [num_tokens][Hq][D]; k_new, v_new: device [num_tokens][Hkv][D].
 * Errors: CB_ERR_INVALID (no scheduled step), CB_ERR_WORKSPACE (the step needs
 * more workspace than configured; call again after cb_engine_set_workspace),
 * and those of cb_kv_append / cb_attention_step. */
int cb_engine_attend(cb_engine* e, const void* q, const void* k_new, const void* v_new, void* out,
                     void* stream);

/* Replace the engine builder's whole state (requests, pages, free list,
 * counters) with a deep copy of `src` -- a scheduler checkpoint restore.  A
 * scheduled step that was not attended is dropped.  The handle returned by
 * cb_engine_builder stays valid. */
int cb_engine_load_builder(cb_engine* e, const cb_builder* src);

/* ----------------------------------------------------------------------------
 * Graph replay.  [CBA] "CUDA graphs": the CPU cost of building and dispatching
 * each step is removed by recording the step's GPU work once and replaying it
 * for steps of matching shape; shapes change every step, so query lengths are
 * padded to a multiple of a q interval and KV lengths to a multiple of a KV
 * interval, and recorded graphs are kept per padded shape.
 *
 * With q_padding_interval >= 1 and kv_padding_interval a positive multiple of
 * 16, cb_engine_schedule lays the step out for its padded shape: tokens
 * rounded up to the q interval (padding tokens have slot -1 and belong to no
 * sequence), the longest context rounded up to the KV interval (the block
 * table stride follows), decode and prefill sequence counts rounded up to
 * multiples of 16 and 4 (padding sequences are empty).  The descriptor
 * returned to the caller is unchanged.  With capture != 0, cb_engine_attend
 * records the append and attention launches of a new (padded shape, metadata
 * slot, buffer addresses) key into a HIP graph and launches the graph; a
 * later step with the same key replays it.  At most 128 graphs are kept (all
 * are dropped when the limit is reached, and when the metadata buffers or the
 * workspace are replaced).  capture == 0 pads without recording (the same
 * kernels, launched directly).  (0, 0, 0) turns padding off.
 *
 * In padded mode q, k_new, v_new and out must hold cb_engine_padded_tokens()
 * rows (rows past the step's tokens are read and written but mean nothing),
 * and the stream must be capturable (not the legacy default stream).
 * Errors: CB_ERR_INVALID (bad intervals, capture without padding). */
int cb_engine_set_graphs(cb_engine* e, int32_t q_padding_interval, int32_t kv_padding_interval,
                         int32_t capture);

/* Rows the scheduled step's buffers must hold (its padded token count); 0
 * without a scheduled step. */
int32_t cb_engine_padded_tokens(const cb_engine* e);

/* Graphs recorded and launched so far, and graphs held now. */
int cb_engine_graph_stats(const cb_engine* e, int64_t* captures, int64_t* replays, int64_t* cached);

/* Engine counters.  [CBA] "Async batching": the host prepares step N+1 while
 * the device runs step N; with two staging slots the host runs at most two
 * steps ahead, and slot_waits counts the schedules that found their slot's
 * previous reader (the upload or the append kernel of the step two back)
 * still pending on the device and waited for it. */
typedef struct {
  int64_t steps_scheduled;  /* cb_engine_schedule calls that produced a step */
  int64_t steps_attended;   /* steps whose device work was enqueued */
  int64_t slot_waits;       /* schedules that waited for a staging slot */
  int64_t graph_captures;   /* as cb_engine_graph_stats */
  int64_t graph_replays;
  int64_t graphs_cached;
  int64_t cu_split_steps;   /* bf16 steps whose prefill and decode workgroups took their kind
                               by the CU they ran on (a large prefill share of the step) */
} cb_engine_stats;

/* Errors: CB_ERR_INVALID (null argument). */
int cb_engine_stats_get(const cb_engine* e, cb_engine_stats* out);

/* Workspace the last scheduled step needs (0 if none). */
size_t cb_engine_workspace_bytes(const cb_engine* e);

#ifdef __cplusplus
}
#endif

#endif /* CB_H */
