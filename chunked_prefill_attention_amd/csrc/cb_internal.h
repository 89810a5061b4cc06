// Internal declarations shared by the host files of the library.
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "cb.h"

namespace cb {

// Record a thread-local error message and return `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace cb

namespace cb {
struct WorkLists;
// cb_attention_step with optional caller-built work lists (see kernels.h).
int attention_step_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        int32_t block_table_stride, const int32_t* query_start_loc, const int32_t* context_lens,
                        const int32_t* q_offsets, int32_t num_seqs, int32_t num_decodes, int32_t num_tokens,
                        int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t page_size, int32_t num_pages, float scale, int32_t sliding_window,
                        int32_t dtype, void* out, void* workspace, size_t workspace_bytes, void* stream,
                        const WorkLists* lists, const int32_t* bt_offsets = nullptr);
// Largest number of pages any live request of the builder holds.
int32_t builder_max_pages_held(const cb_builder* b);
// Deep copy of src's state into dst (dst keeps its address).
int builder_assign(cb_builder* dst, const cb_builder* src);
}  // namespace cb
