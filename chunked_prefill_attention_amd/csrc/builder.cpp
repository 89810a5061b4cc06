// FIFO batch builder: the host half of one continuous-batching engine step.
//
// Hugging Face transformers, "Continuous batching architecture": sections
// "Request lifecycle", "Chunked prefill", "Scheduler", "FIFO", "Admission".
// Ultralytics glossary, "Chunked Prefill", "How chunked prefill works": one
// token per running decode first, then prompt chunks fill the budget.
// AI Engineering from Scratch, "vLLM serving internals", "What the scheduler
// looks like": release finished requests, admit from the head of the waiting
// queue while blocks are free, then batch decode tokens and prefill chunks.
//
// transformers, "PrefillFirst": split prefills finish before decoding resumes.
// TNG blog, "Request-parallel prefill": a cap on prefills per step and on the
// long ones among them.  transformers, "Prefix caching": full blocks carry a
// content identity, later requests with the same prefix reuse them, shared
// blocks are reference counted; released ones stay matchable until their page
// is needed again (newest released first).
//
// Per step the builder walks its live requests once (O(requests + new pages))
// and writes the ragged descriptor into arrays it owns, ready to be copied to
// the device in one go.  Pages come from a LIFO stack of physical ids that
// hold no registered block; with sharing on, released registered blocks wait
// in a newest-last list and are taken only when that stack is empty.
#include <algorithm>
#include <cstring>
#include <memory>
#include <new>
#include <unordered_map>
#include <vector>

#include "cb_internal.h"

namespace {

enum class State : int { Waiting, Prefilling, Decoding, Finished };

struct Request {
  int64_t id;
  int32_t prompt_len;
  int32_t output_len;
  int64_t arrival;
  int32_t cached = 0;     // tokens whose K/V is in the cache
  int32_t generated = 0;  // output tokens produced so far
  State state = State::Waiting;
  std::vector<int32_t> pages;   // block table, logical order
  std::vector<int32_t> tokens;  // prompt tokens (empty: no sharing)
  int32_t registered = 0;       // leading blocks registered or matched
  bool stop_registering = false;
  int32_t released = 0;         // leading block-table entries released (-1) below the window
};

uint64_t splitmix64(uint64_t& x) {
  uint64_t z = (x += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Identity of a full prompt block: its tokens and the page (with that page's
// generation) holding the block before it.  Every hand-out of a page bumps its
// generation, so keys made under an earlier use of the parent page go stale.
struct BlockKey {
  int32_t parent = -1;
  uint32_t parent_gen = 0;
  int32_t tok[CB_PAGE_SIZE] = {};
  bool operator==(const BlockKey& o) const {
    return parent == o.parent && parent_gen == o.parent_gen && std::memcmp(tok, o.tok, sizeof tok) == 0;
  }
};

struct BlockKeyHash {
  size_t operator()(const BlockKey& k) const {
    uint64_t h = ((uint64_t)(uint32_t)k.parent << 32) ^ k.parent_gen;
    uint64_t x = h;
    for (int i = 0; i < CB_PAGE_SIZE; ++i) {
      x ^= (uint64_t)(uint32_t)k.tok[i] + 0x9E3779B97F4A7C15ull * (uint64_t)(i + 1);
      h ^= splitmix64(x);
    }
    return (size_t)h;
  }
};

// The physical page pool.
struct PagePool {
  std::vector<int32_t> clean;  // stack of pages holding no registered block; back() goes next
  bool sharing = false;
  // per page, sized only with sharing on
  std::vector<int32_t> ref;
  std::vector<uint32_t> gen;
  std::vector<uint8_t> hashed;
  std::vector<BlockKey> key;
  std::vector<int32_t> prev, next;  // list of released registered blocks, newest at tail
  int32_t head = -1, tail = -1, cached = 0;
  std::unordered_map<BlockKey, int32_t, BlockKeyHash> index;

  int32_t free() const { return (int32_t)clean.size() + cached; }

  void unlink(int32_t p) {
    (prev[p] >= 0 ? next[prev[p]] : head) = next[p];
    (next[p] >= 0 ? prev[next[p]] : tail) = prev[p];
    prev[p] = next[p] = -1;
    cached--;
  }
  void push_cached(int32_t p) {
    prev[p] = tail;
    next[p] = -1;
    (tail >= 0 ? next[tail] : head) = p;
    tail = p;
    cached++;
  }
  // One page for private use: a clean page if any, else the newest released
  // registered block, which loses its registration.
  int32_t take() {
    int32_t p;
    if (!clean.empty()) {
      p = clean.back();
      clean.pop_back();
    } else {
      p = tail;
      unlink(p);
      auto it = index.find(key[p]);
      if (it != index.end() && it->second == p) index.erase(it);
      hashed[p] = 0;
    }
    if (sharing) {
      gen[p]++;
      ref[p] = 1;
    }
    return p;
  }
  void release(int32_t p) {
    if (!sharing) {
      clean.push_back(p);
      return;
    }
    if (--ref[p] > 0) return;
    if (hashed[p]) push_cached(p);
    else clean.push_back(p);
  }
  // the key of block i of a request whose pages are `pages`
  BlockKey make_key(const std::vector<int32_t>& pages, const std::vector<int32_t>& tokens, int32_t i) const {
    BlockKey k;
    if (i > 0) {
      k.parent = pages[i - 1];
      k.parent_gen = gen[k.parent];
    }
    std::memcpy(k.tok, tokens.data() + (size_t)i * CB_PAGE_SIZE, sizeof k.tok);
    return k;
  }
};

}  // namespace

struct cb_builder {
  cb_builder_config cfg{};
  PagePool pool;
  std::vector<std::unique_ptr<Request>> reqs;  // arrival order
  std::unordered_map<int64_t, Request*> by_id;
  int64_t arrivals = 0;
  int64_t steps = 0;
  int64_t total_stalls = 0;
  int64_t total_finished = 0;
  int64_t prefix_hit_tokens = 0;

  // step outputs (owned, valid until the next step)
  std::vector<int64_t> o_req_ids, o_finished, o_stalled;
  std::vector<int32_t> o_qsl, o_ctx, o_off, o_bt, o_slots;

  int32_t take_page() { return pool.take(); }
  int32_t free_pages() const { return pool.free(); }

  // logical pages wholly below every later row's window, for a request with
  // `cached` tokens in the cache
  int32_t window_floor(int32_t cached) const {
    if (cfg.sliding_window <= 0) return 0;
    return std::max(0, cached - cfg.sliding_window + 1) / CB_PAGE_SIZE;
  }

  // registered blocks matching r's prompt, stopping short of its last token
  void match(const Request& r, std::vector<int32_t>& out) const {
    out.clear();
    for (int32_t i = 0; i < (r.prompt_len - 1) / CB_PAGE_SIZE; ++i) {
      auto it = pool.index.find(pool.make_key(out, r.tokens, i));
      if (it == pool.index.end()) break;
      out.push_back(it->second);
    }
  }
  // register r's full prompt blocks, in order, until one is already known
  void register_blocks(Request& r) {
    const int32_t full = std::min(r.cached, r.prompt_len) / CB_PAGE_SIZE;
    while (r.registered < full && !r.stop_registering) {
      const int32_t i = r.registered;
      BlockKey k = pool.make_key(r.pages, r.tokens, i);
      if (pool.index.count(k)) {
        r.stop_registering = true;
        break;
      }
      const int32_t p = r.pages[i];
      pool.index.emplace(k, p);
      pool.key[p] = k;
      pool.hashed[p] = 1;
      r.registered++;
    }
  }
  void copy_state_from(const cb_builder& o) {
    cfg = o.cfg;
    pool = o.pool;
    arrivals = o.arrivals;
    steps = o.steps;
    total_stalls = o.total_stalls;
    total_finished = o.total_finished;
    prefix_hit_tokens = o.prefix_hit_tokens;
    reqs.clear();
    by_id.clear();
    for (const auto& r : o.reqs) {
      reqs.emplace_back(new Request(*r));
      by_id[r->id] = reqs.back().get();
    }
  }
};

extern "C" {

int cb_builder_create(const cb_builder_config* config, cb_builder** out) {
  cb::clear_error();
  if (!config || !out) return cb::fail(CB_ERR_INVALID, "cb_builder_create: null argument");
  const cb_builder_config& c = *config;
  if (c.page_size != CB_PAGE_SIZE)
    return cb::fail(CB_ERR_UNSUPPORTED, "page_size must be %d (got %d)", CB_PAGE_SIZE, c.page_size);
  if (c.max_batch_tokens < 1 || c.max_requests_per_batch < 1 || c.num_pages < 1 ||
      (int64_t)c.num_pages * CB_PAGE_SIZE >= (int64_t(1) << 31))
    return cb::fail(CB_ERR_INVALID, "budgets and pool size must be positive (pool < 2^27 pages)");
  if (c.max_prefill_chunk < 0 || !(c.safety_margin >= 0.0f && c.safety_margin < 1.0f))
    return cb::fail(CB_ERR_INVALID, "max_prefill_chunk must be >= 0 and safety_margin in [0, 1)");
  if (c.policy != CB_POLICY_FIFO && c.policy != CB_POLICY_PREFILL_FIRST)
    return cb::fail(CB_ERR_INVALID, "unknown scheduling policy %d", c.policy);
  if (c.max_partial_prefills < 0 || c.max_long_partial_prefills < 0 || c.long_prefill_threshold < 0)
    return cb::fail(CB_ERR_INVALID, "prefill caps and the long-prompt threshold must be >= 0");
  if (c.sliding_window < 0 || (c.sliding_window > 0 && c.allow_block_sharing))
    return cb::fail(CB_ERR_INVALID, "sliding_window must be >= 0 and cannot be combined with block sharing");
  cb_builder* b = new (std::nothrow) cb_builder();
  if (!b) return cb::fail(CB_ERR_INVALID, "out of host memory");
  b->cfg = c;
  PagePool& pool = b->pool;
  pool.clean.resize(c.num_pages);
  for (int32_t i = 0; i < c.num_pages; ++i) pool.clean[i] = c.num_pages - 1 - i;
  if (c.page_shuffle_seed != 0) {
    uint64_t st = c.page_shuffle_seed;
    for (int32_t i = c.num_pages - 1; i > 0; --i) {
      int32_t j = (int32_t)(splitmix64(st) % (uint64_t)(i + 1));
      std::swap(pool.clean[i], pool.clean[j]);
    }
  }
  if (c.allow_block_sharing) {
    pool.sharing = true;
    pool.ref.assign(c.num_pages, 0);
    pool.gen.assign(c.num_pages, 0);
    pool.hashed.assign(c.num_pages, 0);
    pool.key.resize(c.num_pages);
    pool.prev.assign(c.num_pages, -1);
    pool.next.assign(c.num_pages, -1);
  }
  *out = b;
  return CB_OK;
}

int cb_builder_clone(const cb_builder* b, cb_builder** out) {
  cb::clear_error();
  if (!b || !out) return cb::fail(CB_ERR_INVALID, "cb_builder_clone: null argument");
  cb_builder* c = new (std::nothrow) cb_builder();
  if (!c) return cb::fail(CB_ERR_INVALID, "out of host memory");
  c->copy_state_from(*b);
  *out = c;
  return CB_OK;
}

void cb_builder_destroy(cb_builder* b) { delete b; }

static int submit_impl(cb_builder* b, int64_t req_id, int32_t prompt_len, int32_t output_len,
                       int32_t tokens_cached, const int32_t* tokens) {
  if (!b) return cb::fail(CB_ERR_INVALID, "cb_builder_submit: null builder");
  if (b->by_id.count(req_id)) return cb::fail(CB_ERR_INVALID, "duplicate request id %lld", (long long)req_id);
  if (prompt_len < 1 || output_len < 1 || tokens_cached < 0)
    return cb::fail(CB_ERR_INVALID, "prompt_len and output_len must be >= 1, tokens_cached >= 0");
  const int64_t final_kv = (int64_t)prompt_len + output_len - 1;
  if (tokens_cached > 0 && tokens_cached >= final_kv)
    return cb::fail(CB_ERR_INVALID, "request %lld has nothing left to do", (long long)req_id);
  int64_t peak = cb::ceil_div(final_kv, CB_PAGE_SIZE);
  if (b->cfg.sliding_window > 0) {  // the window plus one chunk, +1 page for alignment
    int64_t chunk = std::min(prompt_len, b->cfg.max_batch_tokens);
    if (b->cfg.max_prefill_chunk > 0) chunk = std::min<int64_t>(chunk, b->cfg.max_prefill_chunk);
    peak = std::min(peak, cb::ceil_div((int64_t)b->cfg.sliding_window - 1 + chunk, CB_PAGE_SIZE) + 1);
  }
  if (peak > b->cfg.num_pages)
    return cb::fail(CB_ERR_CAPACITY, "request %lld needs %lld pages at once; the pool has %d",
                    (long long)req_id, (long long)peak, b->cfg.num_pages);
  auto r = std::make_unique<Request>();
  r->id = req_id;
  r->prompt_len = prompt_len;
  r->output_len = output_len;
  r->arrival = b->arrivals;
  if (tokens && b->pool.sharing) r->tokens.assign(tokens, tokens + prompt_len);
  if (tokens_cached > 0) {
    const int32_t first = b->window_floor(tokens_cached);
    int32_t need = (int32_t)cb::ceil_div(tokens_cached, CB_PAGE_SIZE) - first;
    if (need > b->free_pages())
      return cb::fail(CB_ERR_CAPACITY, "import of %lld needs %d pages; %d free", (long long)req_id, need,
                      b->free_pages());
    r->pages.assign(first, -1);
    r->released = first;
    for (int32_t i = 0; i < need; ++i) r->pages.push_back(b->take_page());
    r->cached = tokens_cached;
    if (tokens_cached < prompt_len) {
      r->state = State::Prefilling;
    } else {
      r->state = State::Decoding;
      r->generated = tokens_cached - prompt_len + 1;
    }
  }
  b->arrivals++;
  b->by_id[req_id] = r.get();
  b->reqs.push_back(std::move(r));
  return CB_OK;
}

int cb_builder_submit(cb_builder* b, int64_t req_id, int32_t prompt_len, int32_t output_len,
                      int32_t tokens_cached) {
  cb::clear_error();
  return submit_impl(b, req_id, prompt_len, output_len, tokens_cached, nullptr);
}

int cb_builder_submit_tokens(cb_builder* b, int64_t req_id, const int32_t* tokens, int32_t prompt_len,
                             int32_t output_len) {
  cb::clear_error();
  if (!tokens) return cb::fail(CB_ERR_INVALID, "cb_builder_submit_tokens: null token array");
  return submit_impl(b, req_id, prompt_len, output_len, 0, tokens);
}

int cb_builder_step(cb_builder* b, cb_step* out) {
  cb::clear_error();
  if (!b || !out) return cb::fail(CB_ERR_INVALID, "cb_builder_step: null argument");
  const cb_builder_config& c = b->cfg;
  PagePool& pool = b->pool;
  b->o_req_ids.clear();
  b->o_finished.clear();
  b->o_stalled.clear();

  // 0. release what finished in the previous step (arrival order)
  {
    std::vector<std::unique_ptr<Request>> keep;
    keep.reserve(b->reqs.size());
    for (auto& r : b->reqs) {
      if (r->state == State::Finished) {
        for (int32_t p : r->pages)
          if (p >= 0) pool.release(p);
        b->o_finished.push_back(r->id);
        b->by_id.erase(r->id);
        b->total_finished++;
      } else {
        keep.push_back(std::move(r));
      }
    }
    b->reqs.swap(keep);
  }
  // pages that fell out of every live request's window
  if (c.sliding_window > 0) {
    for (auto& up : b->reqs) {
      Request* r = up.get();
      const int32_t lim = std::min<int32_t>(b->window_floor(r->cached), (int32_t)r->pages.size());
      for (; r->released < lim; ++r->released) {
        pool.release(r->pages[r->released]);
        r->pages[r->released] = -1;
      }
    }
  }

  struct Pick { Request* r; int32_t n; bool decode; };
  std::vector<Pick> picks;
  int32_t tokens_left = c.max_batch_tokens;
  int32_t slots_left = c.max_requests_per_batch;
  int32_t new_pages = 0, step_hits = 0, n_prefills = 0, n_long = 0;
  auto room = [&] { return tokens_left >= 1 && slots_left >= 1; };
  auto is_long = [&](const Request* r) { return r->prompt_len > c.long_prefill_threshold; };
  auto capped = [&](const Request* r) {
    if (c.max_partial_prefills > 0 && n_prefills >= c.max_partial_prefills) return true;
    return c.max_long_partial_prefills > 0 && is_long(r) && n_long >= c.max_long_partial_prefills;
  };
  auto pick_prefill = [&](Request* r, int32_t n) {
    picks.push_back({r, n, false});
    tokens_left -= n;
    slots_left -= 1;
    n_prefills++;
    n_long += is_long(r) ? 1 : 0;
  };

  // active decodes, one token each
  auto decodes = [&] {
    for (auto& up : b->reqs) {
      Request* r = up.get();
      if (r->state != State::Decoding) continue;
      if (!room()) break;
      int32_t need = (r->cached % CB_PAGE_SIZE == 0) ? 1 : 0;
      if (need > b->free_pages()) { b->o_stalled.push_back(r->id); continue; }
      if (need) { r->pages.push_back(b->take_page()); new_pages++; }
      picks.push_back({r, 1, true});
      tokens_left -= 1;
      slots_left -= 1;
    }
  };
  // active prefills, each taking every token that still fits
  auto active_prefills = [&] {
    for (auto& up : b->reqs) {
      Request* r = up.get();
      if (r->state != State::Prefilling) continue;
      if (!room()) break;
      if (capped(r)) continue;
      int64_t chunk = std::min<int64_t>(r->prompt_len - r->cached, tokens_left);
      if (c.max_prefill_chunk > 0) chunk = std::min<int64_t>(chunk, c.max_prefill_chunk);
      chunk = std::min<int64_t>(chunk, ((int64_t)r->pages.size() + b->free_pages()) * CB_PAGE_SIZE - r->cached);
      if (chunk <= 0) { b->o_stalled.push_back(r->id); continue; }
      int32_t need = (int32_t)(cb::ceil_div(r->cached + chunk, CB_PAGE_SIZE) - (int64_t)r->pages.size());
      for (int32_t i = 0; i < need; ++i) r->pages.push_back(b->take_page());
      new_pages += need;
      pick_prefill(r, (int32_t)chunk);
    }
  };
  // waiting requests, arrival order, strict head of line on pages
  std::vector<int32_t> matched;
  auto waiting = [&] {
    for (auto& up : b->reqs) {
      Request* r = up.get();
      if (r->state != State::Waiting) continue;
      if (!room()) break;
      if (capped(r)) continue;
      matched.clear();
      if (pool.sharing && !r->tokens.empty()) b->match(*r, matched);
      const int32_t start = (int32_t)matched.size() * CB_PAGE_SIZE;
      int32_t chunk = std::min(r->prompt_len - start, tokens_left);
      if (c.max_prefill_chunk > 0) chunk = std::min(chunk, c.max_prefill_chunk);
      int32_t reused = 0;
      for (int32_t p : matched) reused += pool.ref[p] == 0 ? 1 : 0;
      const int32_t fresh = (int32_t)cb::ceil_div(chunk, CB_PAGE_SIZE);
      const int32_t need = fresh + reused;
      if (need > b->free_pages()) break;
      if (c.safety_margin > 0.0f &&
          (double)(b->free_pages() - need) < (double)c.safety_margin * (double)c.num_pages)
        break;
      for (int32_t p : matched) {
        if (pool.ref[p] == 0) pool.unlink(p);
        pool.ref[p]++;
      }
      r->pages.assign(matched.begin(), matched.end());
      for (int32_t i = 0; i < fresh; ++i) r->pages.push_back(b->take_page());
      r->cached = start;
      r->registered = (int32_t)matched.size();
      r->state = State::Prefilling;
      new_pages += need;
      step_hits += start;
      pick_prefill(r, chunk);
    }
  };
  if (c.policy == CB_POLICY_PREFILL_FIRST) {
    active_prefills();
    decodes();
  } else {
    decodes();
    active_prefills();
  }
  waiting();
  // the descriptor lists decodes first, each class in picking order
  std::stable_partition(picks.begin(), picks.end(), [](const Pick& p) { return p.decode; });

  // emit the descriptor
  const int32_t n = (int32_t)picks.size();
  int32_t stride = 1, num_decodes = 0, max_q = 0, max_ctx = 0;
  int64_t total = 0;
  for (const Pick& p : picks) {
    stride = std::max<int32_t>(stride, (int32_t)p.r->pages.size());
    num_decodes += p.decode ? 1 : 0;
    max_q = std::max(max_q, p.n);
    max_ctx = std::max(max_ctx, p.r->cached + p.n);
    total += p.n;
  }
  b->o_qsl.assign(n + 1, 0);
  b->o_ctx.assign(n, 0);
  b->o_off.assign(n, 0);
  b->o_bt.assign((size_t)n * stride, 0);
  b->o_slots.assign((size_t)total, 0);
  int32_t t = 0;
  for (int32_t s = 0; s < n; ++s) {
    Request* r = picks[s].r;
    const int32_t q_len = picks[s].n;
    b->o_req_ids.push_back(r->id);
    b->o_qsl[s] = t;
    b->o_off[s] = r->cached;
    b->o_ctx[s] = r->cached + q_len;
    std::copy(r->pages.begin(), r->pages.end(), b->o_bt.begin() + (size_t)s * stride);
    for (int32_t i = 0; i < q_len; ++i) {
      const int32_t pos = r->cached + i;
      b->o_slots[t + i] = r->pages[pos / CB_PAGE_SIZE] * CB_PAGE_SIZE + pos % CB_PAGE_SIZE;
    }
    t += q_len;
    // advance the request's lifecycle
    r->cached += q_len;
    if (picks[s].decode) r->generated += 1;
    else if (r->cached == r->prompt_len) r->generated = 1;
    if (r->generated >= 1)
      r->state = (r->generated >= r->output_len) ? State::Finished : State::Decoding;
    if (pool.sharing && !r->tokens.empty()) b->register_blocks(*r);
  }
  b->o_qsl[n] = t;
  b->steps++;
  b->total_stalls += (int64_t)b->o_stalled.size();
  b->prefix_hit_tokens += step_hits;

  out->num_seqs = n;
  out->num_decodes = num_decodes;
  out->num_tokens = t;
  out->max_query_len = max_q;
  out->max_context_len = max_ctx;
  out->block_table_stride = stride;
  out->num_finished = (int32_t)b->o_finished.size();
  out->num_stalled = (int32_t)b->o_stalled.size();
  out->new_pages = new_pages;
  out->prefix_hit_tokens = step_hits;
  out->req_ids = b->o_req_ids.data();
  out->query_start_loc = b->o_qsl.data();
  out->context_lens = b->o_ctx.data();
  out->q_offsets = b->o_off.data();
  out->block_tables = b->o_bt.data();
  out->slot_mapping = b->o_slots.data();
  out->finished_ids = b->o_finished.data();
  out->stalled_ids = b->o_stalled.data();
  return CB_OK;
}

int cb_builder_block_table(const cb_builder* b, int64_t req_id, int32_t* out, int32_t cap, int32_t* n) {
  cb::clear_error();
  if (!b || !n || (cap > 0 && !out)) return cb::fail(CB_ERR_INVALID, "cb_builder_block_table: null argument");
  auto it = b->by_id.find(req_id);
  if (it == b->by_id.end()) return cb::fail(CB_ERR_INVALID, "unknown request id %lld", (long long)req_id);
  const auto& pages = it->second->pages;
  *n = (int32_t)pages.size();
  const int32_t m = std::min<int32_t>(cap, (int32_t)pages.size());
  for (int32_t i = 0; i < m; ++i) out[i] = pages[i];
  return CB_OK;
}

int cb_builder_slots(const cb_builder* b, int64_t req_id, int32_t start, int32_t end, int32_t* out) {
  cb::clear_error();
  if (!b || (end > start && !out)) return cb::fail(CB_ERR_INVALID, "cb_builder_slots: null argument");
  if (start < 0 || end < start) return cb::fail(CB_ERR_INVALID, "cb_builder_slots: bad range [%d, %d)", start, end);
  auto it = b->by_id.find(req_id);
  if (it == b->by_id.end()) return cb::fail(CB_ERR_INVALID, "unknown request id %lld", (long long)req_id);
  const auto& pages = it->second->pages;
  for (int32_t p = start; p < end; ++p) {
    const size_t lp = (size_t)(p / CB_PAGE_SIZE);
    if (lp >= pages.size() || pages[lp] < 0)
      return cb::fail(CB_ERR_INVALID, "position %d of request %lld is not in a held page", p, (long long)req_id);
  }
  for (int32_t p = start; p < end; ++p) out[p - start] = pages[(size_t)(p / CB_PAGE_SIZE)] * CB_PAGE_SIZE + p % CB_PAGE_SIZE;
  return CB_OK;
}

int cb_builder_stats_get(const cb_builder* b, cb_builder_stats* out) {
  cb::clear_error();
  if (!b || !out) return cb::fail(CB_ERR_INVALID, "cb_builder_stats_get: null argument");
  std::memset(out, 0, sizeof(*out));
  out->num_pages = b->cfg.num_pages;
  out->free_pages = b->free_pages();
  for (const auto& r : b->reqs) {
    switch (r->state) {
      case State::Waiting: out->num_waiting++; break;
      case State::Prefilling: out->num_prefilling++; break;
      case State::Decoding: out->num_decoding++; break;
      case State::Finished: out->num_finished_pending++; break;
    }
    if (!b->pool.sharing) {  // tokens in held pages
      for (size_t i = (size_t)r->released; i < r->pages.size(); ++i)
        out->used_slots += std::max(0, std::min<int32_t>(CB_PAGE_SIZE, r->cached - (int32_t)i * CB_PAGE_SIZE));
    }
  }
  if (b->pool.sharing) {  // a shared page counts once, at its fill
    std::unordered_map<int32_t, int32_t> fill;
    for (const auto& r : b->reqs)
      for (size_t i = 0; i < r->pages.size(); ++i) {
        const int32_t f = std::max(0, std::min<int32_t>(CB_PAGE_SIZE, r->cached - (int32_t)i * CB_PAGE_SIZE));
        int32_t& v = fill[r->pages[i]];
        v = std::max(v, f);
      }
    for (const auto& kv : fill) out->used_slots += kv.second;
  }
  out->allocated_slots = (int64_t)(b->cfg.num_pages - b->free_pages()) * CB_PAGE_SIZE;
  out->steps = b->steps;
  out->total_stalls = b->total_stalls;
  out->total_finished = b->total_finished;
  out->fragmentation = out->allocated_slots > 0
      ? (double)(out->allocated_slots - out->used_slots) / (double)out->allocated_slots : 0.0;
  out->prefix_hit_tokens = b->prefix_hit_tokens;
  out->cached_pages = b->pool.cached;
  return CB_OK;
}

}  // extern "C"

namespace cb {
int builder_assign(cb_builder* dst, const cb_builder* src) {
  if (!dst || !src) return fail(CB_ERR_INVALID, "builder_assign: null argument");
  if (dst == src) return CB_OK;
  dst->copy_state_from(*src);
  return CB_OK;
}

int32_t builder_max_pages_held(const cb_builder* b) {
  size_t m = 0;
  for (const auto& r : b->reqs) m = std::max(m, r->pages.size());
  return (int32_t)m;
}
}  // namespace cb
