// bf16 attention step for gfx950: one ragged launch for decode tokens and
// prefill chunks over a paged KV cache, plus its plan and split-K combine.
//
// What is computed (Ultralytics glossary, "Chunked Prefill", "How chunked
// prefill works"): a query row at absolute position p of sequence s attends,
// under a causal mask over absolute positions, to keys 0..p of the same
// sequence -- the cached K/V of all earlier chunks plus the chunk itself.  A
// decode token is a one-row chunk.  Where time goes (same page, "Prefill,
// decode and generation stalls"): prefill is compute-bound, decode reads the
// whole cache each step and is bandwidth-bound.  Hence two work-item kinds in
// one grid:
//
//  * decode item = one wavefront on (sequence, KV head, split of the page
//    list).  It streams its pages straight from HBM into registers (a ring of
//    page buffers keeps the next pages' loads in flight), scores the G query
//    heads that share the KV head with one 16x16x32 bf16 MFMA per 32 dims
//    (keys as rows, heads as columns), keeps an online softmax per head, and
//    accumulates P V with 16x16x16 bf16 MFMAs.
//  * prefill item = one 256-thread workgroup on (sequence, KV head, tile of
//    128 query rows, range of keys), where a row is a (query token, query
//    head of the group) pair so the G heads sharing a KV head read K/V once.
//    Per 64-key tile the workgroup copies K and V pages straight from the
//    cache into LDS (global_load_lds, each wavefront one page; tile k+1 is
//    copied into one LDS stage while tile k is computed from the other);
//    each wavefront computes S^T = K Q^T for its 32 rows with 32x32x16 bf16
//    MFMAs, reading its K and V fragments from LDS in batches ahead of the
//    MFMAs, masks only the tiles that straddle its diagonal, updates the
//    online softmax and accumulates O^T = V^T P^T.
//    Tiles wholly above the diagonal are never loaded.  Long key ranges are
//    cut into several items so that a long chunk spreads over every CU.
//
// Items with more than one split write partial results (row max, row sum,
// and O divided by that sum, in fp16); the combine kernel merges them by
// log-sum-exp.
//
// Block order: the work lists start with the live item counts; live blocks
// run first (prefill first when its workgroups fit in one round of the
// device's slots, else prefill and decode alternating) and blocks past the
// live work return at once.  When the host built the lists and the prefill
// part is a large share of the step, the kinds go by CU instead: workgroups
// that land on the first k CUs of each shader engine take prefill units, the
// rest decode units, each from per-XCD claim queues (see pick_unit).
//
// Layouts: K pages are token-major ([16][D] per (page, head)), so a lane's
// MFMA A-operand (one key, 8 consecutive dims) is one 16-byte load.  V pages
// are token-minor ([D][16]), so the A-operand of O^T = V^T P^T (one dim, 4 or
// 8 consecutive keys) is one or two 8-byte loads, and the B-operand P^T comes
// straight from the score accumulator registers without any shuffle.
//
// Numerics: bf16 inputs, fp32 MFMA accumulation, softmax in fp32 (scores kept
// in raw units; exponentials are exp2(s*scale*log2(e) - m*scale*log2(e)) with
// one FMA), probabilities rounded to bf16 for the P V product (and, in
// prefill, for the row sum, so numerator and normaliser weigh the same
// values), output rounded to bf16 (round to nearest even); split-K partial
// outputs are kept in fp16 divided by their own sum.  The running max
// is raised only when a score exceeds it by more than 8 in log2 units, so
// the accumulator rescale is usually skipped; weights stay <= 2^8.  Cache slots at or past the context length are masked by
// select and their V entries zeroed (in prefill, as they are read from LDS),
// so garbage or NaN there never reaches the output.
#include <hip/hip_runtime.h>
#include <atomic>
#include <type_traits>
#include <vector>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "kernels.h"

namespace cb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Tunables (compile-time).  Pages of K/V each decode wavefront keeps in
// flight ahead of the page it is computing on, and its occupancy target.
#ifndef CB_DEC_PREFETCH
#define CB_DEC_PREFETCH 2
#endif
#ifndef CB_DEC_WAVES_PER_SIMD
#define CB_DEC_WAVES_PER_SIMD 2
#endif
#ifndef CB_DEC_MIN_WAVES     // decode splits: the longest that still gives this many wavefronts
#define CB_DEC_MIN_WAVES 6144
#endif
#ifndef CB_DEC_MIN_WAVES_ALONE  // ... in a step without prefill work (the decode-only launch)
#define CB_DEC_MIN_WAVES_ALONE 4096
#endif
#ifndef CB_PF_PRIO          // wave priority raised while the prefill QK MFMAs issue
#define CB_PF_PRIO 1
#endif
#ifndef CB_NT_DECODE        // decode-only launch: K/V page loads with the non-temporal hint
#define CB_NT_DECODE 1
#endif
#ifndef CB_NT_MIXED         // the same for the decode waves of the mixed launch ...
#define CB_NT_MIXED 0
#endif
#ifndef CB_NT_MIXED_WINDOW  // ... and of its sliding-window instantiation
#define CB_NT_MIXED_WINDOW 1
#endif
#ifndef CB_PF_READAHEAD     // prefill: K and V fragments read from LDS in batches of this many (0: compiler's order)
#define CB_PF_READAHEAD 4
#endif
// threads per workgroup of the decode-only kernel (64 or 256)
#ifndef CB_DEC_WG
#define CB_DEC_WG 64
#endif
// exponent headroom before the running max is raised (log2 units)
#ifndef CB_RESCALE_SLACK
#define CB_RESCALE_SLACK 8.0f
#endif

#ifndef CB_PF_TARGET_ITEMS  // prefill key ranges are cut for about this many workgroups
#define CB_PF_TARGET_ITEMS 1024
#endif
#ifndef CB_PF_MIN_KEYS      // ... but never shorter than this (a multiple of 64)
#define CB_PF_MIN_KEYS 512
#endif
#ifndef CB_PF_THREADS
#define CB_PF_THREADS 256
#endif
constexpr int PF_THREADS = CB_PF_THREADS;   // threads of a prefill workgroup
constexpr int PF_WAVES = PF_THREADS / 64;
constexpr int PF_ROWS = PF_WAVES * 32;      // query rows per prefill workgroup (32 per wave)
constexpr int PF_KEYS = 64;   // keys per prefill tile (4 pages)
constexpr int DEC_MAX_SPLIT = 128;                         // pages one decode item covers at most
constexpr int PF_MAX_PAGES = 512;                          // page ids one prefill item stages in LDS
constexpr int PF_MAX_KEYS = (PF_MAX_PAGES - 4) * 16 / PF_KEYS * PF_KEYS;  // largest key range per item
constexpr float LOG2E = 1.4426950408889634f;

struct Params {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* bt;
  const int32_t* qsl;
  const int32_t* ctx_lens;
  const int32_t* q_off;
  uint16_t* out;
  int4* hdr;             // (live prefill items, live decode items, block order, prefill CUs per SE),
                         // then the CU split's claim queues (UnitQueues)
  int4* dec_items;       // (sequence, split, context length, query row); sequence -1 = no work
  int4* pf_items;        // (sequence, row tile, key split, partial slot); -1 = no work
  int4* pf_tiles;        // (sequence, row tile, first item, number of splits); -1 = none
  int32_t* dec_first;    // [num_decodes] first full-length decode item of each sequence
  int32_t* dec_rem;      // [num_decodes] the sequence's shorter last item, or -1
  float2* dec_ml;        // [decode wave][G] (running max in raw score units, sum)
  uint16_t* dec_o;       // [decode wave][G][D] fp16, divided by the split's own sum
  float2* pf_ml;         // [prefill item][PF_ROWS]
  uint16_t* pf_o;        // [prefill item][PF_ROWS][D] fp16, divided by the split's own sum
  int32_t bt_stride;
  const int32_t* bt_off;  // row offsets of packed block tables, or null (row s at s * bt_stride)
  int32_t num_seqs, num_decodes;
  int32_t hq, hkv, G;
  int32_t num_pages;
  int32_t split_pages;   // pages per decode item
  int32_t pf_split_keys; // keys per prefill item (multiple of PF_KEYS)
  int32_t pf_blocks;     // prefill workgroups the work lists can hold
  int32_t dec_blocks;    // decode workgroups (PF_WAVES wavefronts) the work lists can hold
  int32_t slots;         // workgroups of the mixed launch the device holds at once
  int32_t dec_cap, pf_tile_cap, pf_item_cap;
  int32_t comb_dec_blocks;
  int32_t window;        // sliding window in tokens; 0 = none
  float scale_log2;      // softmax scale * log2(e)
  // measurement hook: when set, workgroup 0 writes its (shader-clock counter,
  // 100 MHz real-time counter) at start and end here (4 values)
  unsigned long long* clk;
};

// Workgroup 0's clock record (measurement hook, off unless p.clk is set).
__device__ __forceinline__ void clock_mark(const Params& p, int at) {
  if (p.clk && blockIdx.x == 0 && threadIdx.x == 0) {
    p.clk[2 * at] = __builtin_amdgcn_s_memtime();
    p.clk[2 * at + 1] = __builtin_amdgcn_s_memrealtime();
  }
}

template <int D>
struct PfLds {
  static constexpr int KROW = D * 2;       // K row (bytes) in LDS, 16-byte chunks swizzled by row
  static constexpr int VROW = 32;          // (page, dim) row of 16 tokens (bytes), halves swapped on rows with bit 3 set
  static constexpr int K_BYTES = PF_KEYS * KROW;
  static constexpr int V_BYTES = (PF_KEYS / 16) * D * VROW;
  static constexpr int STAGE = K_BYTES + V_BYTES;  // one tile; two stages, then the item's page ids
  static_assert(2 * STAGE <= 65536, "copy destinations (M0) below 64 KB");
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ short4v as_short4(uint2 v) { return __builtin_bit_cast(short4v, v); }

// two floats -> one word of two bf16 (round to nearest even), one packed convert
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, b16x2));
}

// Split-K partial outputs are stored as fp16 after division by the split's
// own sum: a weighted mean of V rows, so |value| <= max |v| and fp16's
// 11-bit significand keeps it to 2^-11 relative (four times finer than the
// bf16 output), in half the bytes of fp32.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}
__device__ __forceinline__ float4 unpack_f16x4(uint2 v) {
  const f16x2 a = __builtin_bit_cast(f16x2, v.x), b = __builtin_bit_cast(f16x2, v.y);
  return make_float4((float)a[0], (float)a[1], (float)b[0], (float)b[1]);
}

// acc + the sum of eight bf16 values (four packed pairs), one dot2 with (1, 1) per pair
__device__ __forceinline__ float sum_bf16x8(uint4 v, float acc) {
  typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
  const b16x2 one = __builtin_bit_cast(b16x2, 0x3F803F80u);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b16x2, v.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b16x2, v.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b16x2, v.z), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b16x2, v.w), one, acc, false);
}

// Reductions over lane pairs (l, l^32) and (l, l^16) through the cross-lane
// swap instructions, without an LDS round trip.  Between them the two results
// of a swap hold x[l] and x[l^k] at every lane, so max and sum of the pair are
// the same on both lanes of a pair.
__device__ __forceinline__ float pair_max32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float pair_max16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// keep the first n (0..2*words) 16-bit elements of a little-endian word
__device__ __forceinline__ uint32_t keep16(uint32_t w, int first_elem, int n) {
  return (first_elem + 1 < n) ? w : (first_elem < n ? (w & 0xFFFFu) : 0u);
}
// drop the first n 16-bit elements (zero them), keep the rest
__device__ __forceinline__ uint32_t drop16(uint32_t w, int first_elem, int n) {
  return (first_elem >= n) ? w : (first_elem + 1 >= n ? (w & 0xFFFF0000u) : 0u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// -m*c for the exponent FMA; 0 while no key has been seen (m = -inf), so that
// masked scores (-inf) still give exp2(-inf) = 0 instead of NaN.
__device__ __forceinline__ float neg_scaled(float m, float c) { return m == -INFINITY ? 0.f : -m * c; }

// Loads through the global address space (pointers rebuilt from SGPR halves
// would otherwise become generic "flat" accesses, which the compiler must
// order against LDS traffic too).  NT selects the non-temporal hint: decode
// pages are read once per launch, prefill key tiles once per row tile.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const u32x2 gu32x2;
template <bool NT>
__device__ __forceinline__ uint4 kv_load(const uint4* p) {
  gu32x4* g = (gu32x4*)p;
  u32x4 v;
  if constexpr (NT) v = __builtin_nontemporal_load(g);
  else v = *g;
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <bool NT>
__device__ __forceinline__ uint2 kv_load(const uint2* p) {
  gu32x2* g = (gu32x2*)p;
  u32x2 v;
  if constexpr (NT) v = __builtin_nontemporal_load(g);
  else v = *g;
  return make_uint2(v.x, v.y);
}

// ---------------------------------------------------------------------------
// Plan: one workgroup turns the per-sequence lengths (device data) into
// compact work lists, so the main grid needs only host-side upper bounds.
// Unused list slots get sequence -1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive scan over the 1024 threads of the block; `total` gets the sum.
__device__ int block_exclusive_scan(int v, int* sh, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) sh[wv] = incl;
  __syncthreads();
  if (wv == 0) {
    const int x = lane < 16 ? sh[lane] : 0;
    const int xi = wave_inclusive_scan(x);
    if (lane < 16) sh[16 + lane] = xi - x;  // exclusive prefix of each wave's total
    if (lane == 15) sh[32] = xi;
  }
  __syncthreads();
  total = sh[32];
  const int r = sh[16 + wv] + incl - v;
  __syncthreads();  // sh is reused by the next call
  return r;
}

// keys a prefill row tile needs: up to the last row's position (and the context)
__host__ __device__ __forceinline__ int tile_key_end(int tile, int L, int G, int ctx, int off) {
  const int rows = L * G;
  const int last_row = (tile * PF_ROWS + PF_ROWS < rows ? tile * PF_ROWS + PF_ROWS : rows) - 1;
  const int e = off + last_row / G + 1;
  return e < ctx ? e : ctx;
}

// Sliding window (transformers, "Continuous batching architecture", Memory
// management): a row at position p sees keys p-window < j <= p.
// The first key a row at `pos` sees.
__host__ __device__ __forceinline__ int window_first_key(int pos, int window) {
  return window > 0 && pos - window + 1 > 0 ? pos - window + 1 : 0;
}
// A decode row sits at ctx-1: the first page it reads.
__host__ __device__ __forceinline__ int decode_first_page(int ctx, int window) {
  return window_first_key(ctx - 1, window) >> 4;
}
// Pages a decode row reads, and its number of split items.
__host__ __device__ __forceinline__ int decode_pages(int ctx, int window) {
  return ctx > 0 ? ((ctx + 15) >> 4) - decode_first_page(ctx, window) : 0;
}
// The first key of a prefill row tile (its first row's window start), rounded
// down to a key tile: where the tile's key splits begin.
__host__ __device__ __forceinline__ int tile_key_base(int tile, int G, int off, int window) {
  return window_first_key(off + tile * PF_ROWS / G, window) / PF_KEYS * PF_KEYS;
}
// Key splits of a prefill row tile.
__host__ __device__ __forceinline__ int tile_splits(int tile, int L, int G, int ctx, int off, int window,
                                                    int split_keys) {
  return (tile_key_end(tile, L, G, ctx, off) - tile_key_base(tile, G, off, window) + split_keys - 1) / split_keys;
}

// Block order of the mixed launch.  When the live prefill workgroups fit in
// one round of the device's workgroup slots they go first (they all start at
// once and finish early, decodes fill the rest); when they need several
// rounds, going first would run the MFMA-bound and the HBM-bound work one
// after the other, so prefill and decode blocks are interleaved instead and
// most CUs hold one of each.
// The work lists' header: (live prefill items, live decode items, block
// order, prefill CUs per shader engine) and then, for the CU split, one
// claim counter per XCD for each kind (zero when the launch starts).
constexpr int N_XCD = 8;
struct UnitQueues {
  int next_pf[N_XCD];
  int next_dec[N_XCD];
};
constexpr size_t HDR_BYTES = 16 + sizeof(UnitQueues);
#ifndef CB_CU_SPLIT         // host-built lists: prefill and decode blocks pick their kind by the CU they land on
#define CB_CU_SPLIT 1
#endif
#ifndef CB_CU_SPLIT_MIN     // split only when the prefill part earns at least this many CUs per shader engine
#define CB_CU_SPLIT_MIN 3
#endif
#ifndef CB_CU_SPLIT_MAX     // at most this many prefill CUs per shader engine (of 8)
#define CB_CU_SPLIT_MAX 6
#endif
__host__ __device__ inline int mix_order(int64_t pf_live_items, int64_t dec_live_items, int hkv, int slots) {
  return (pf_live_items * hkv > slots && dec_live_items > 0) ? 1 : 0;
}

__global__ __launch_bounds__(1024) void plan_kernel(Params p) {
  __shared__ int sh[40];
  const int tid = threadIdx.x;
  // decode items, longest first: every full split (split_pages pages) of every
  // sequence, then each sequence's shorter last split, by decreasing length.
  // dec_first[s] = first full split of s; dec_rem[s] = its short split or -1.
  __shared__ int bucket[DEC_MAX_SPLIT + 1], cursor[DEC_MAX_SPLIT + 1];
  const int SP = p.split_pages;  // <= DEC_MAX_SPLIT
  if (tid <= DEC_MAX_SPLIT) { bucket[tid] = 0; cursor[tid] = 0; }
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < p.num_decodes; base += 1024) {
    const int s = base + tid;
    int nfull = 0, ctx = 0, t = 0, rem = 0;
    if (s < p.num_decodes) {
      ctx = p.ctx_lens[s];
      t = p.qsl[s];
      const int np = decode_pages(ctx, p.window);
      nfull = np / SP;
      rem = np - nfull * SP;
      if (rem > 0) atomicAdd(&bucket[SP - rem], 1);
    }
    int total;
    const int ex = block_exclusive_scan(nfull, sh, total) + carry;
    if (s < p.num_decodes) p.dec_first[s] = ex;
    for (int k = 0; k < nfull && ex + k < p.dec_cap; ++k) p.dec_items[ex + k] = make_int4(s, k, ctx, t);
    carry += total;
  }
  __syncthreads();
  {  // bucket starts: an exclusive scan of the bucket counts
    const int n = tid < DEC_MAX_SPLIT ? bucket[tid] : 0;
    int total;
    const int ex = block_exclusive_scan(n, sh, total);
    if (tid < DEC_MAX_SPLIT) bucket[tid] = carry + ex;
  }
  __syncthreads();
  for (int base = 0; base < p.num_decodes; base += 1024) {
    const int s = base + tid;
    if (s < p.num_decodes) {
      const int ctx = p.ctx_lens[s];
      const int np = decode_pages(ctx, p.window);
      const int nfull = np / SP, rem = np - nfull * SP;
      int idx = -1;
      if (rem > 0) {
        idx = bucket[SP - rem] + atomicAdd(&cursor[SP - rem], 1);
        if (idx < p.dec_cap) p.dec_items[idx] = make_int4(s, nfull, ctx, p.qsl[s]);
      }
      p.dec_rem[s] = idx;
      if (rem > 0) atomicMax(&cursor[DEC_MAX_SPLIT], idx + 1);
    }
  }
  __syncthreads();
  const int dec_total = max(carry, cursor[DEC_MAX_SPLIT]);
  for (int i = dec_total + tid; i < p.dec_cap; i += 1024) p.dec_items[i] = make_int4(-1, 0, 0, 0);

  // prefill tiles and their key splits; heaviest (last) tiles first.  One
  // wavefront lists one sequence (its lanes share the row tiles), 16 at a
  // time; a block-wide scan over the sequences places them.
  __shared__ int seq_tiles[1024], seq_items[1024], seq_tex[1024], seq_iex[1024];
  const int lane = tid & 63, wv = tid >> 6;
  int tcarry = 0, icarry = 0;
  for (int base = p.num_decodes; base < p.num_seqs; base += 1024) {
    const int nchunk = min(1024, p.num_seqs - base);
    // counts: tiles and items (key splits) of each sequence
    for (int i = wv; i < nchunk; i += 16) {
      const int s = base + i;
      const int L = p.qsl[s + 1] - p.qsl[s], ctx = p.ctx_lens[s], off = p.q_off[s];
      const int ntiles = L > 0 ? (L * p.G + PF_ROWS - 1) / PF_ROWS : 0;
      int n = 0;
      for (int t = lane; t < ntiles; t += 64) n += tile_splits(t, L, p.G, ctx, off, p.window, p.pf_split_keys);
      n = __builtin_amdgcn_readlane(wave_inclusive_scan(n), 63);
      if (lane == 0) { seq_tiles[i] = ntiles; seq_items[i] = n; }
    }
    __syncthreads();
    int ttotal, itotal;
    const int ntl = tid < nchunk ? seq_tiles[tid] : 0, nit = tid < nchunk ? seq_items[tid] : 0;
    const int tex = block_exclusive_scan(ntl, sh, ttotal) + tcarry;
    const int iex = block_exclusive_scan(nit, sh, itotal) + icarry;
    if (tid < nchunk) { seq_tex[tid] = tex; seq_iex[tid] = iex; }
    __syncthreads();
    // tile records heaviest first, each with its block of partial slots;
    // items split-major (every tile's split 0, then split 1, ...) so that
    // workgroups running together read the same keys: item (k, ks) goes to
    // the sequence's first item + the items of all splits below ks + the
    // tiles before k with more than ks splits
    for (int i = wv; i < nchunk; i += 16) {
      const int s = base + i;
      const int L = p.qsl[s + 1] - p.qsl[s], ctx = p.ctx_lens[s], off = p.q_off[s];
      const int ntiles = seq_tiles[i], t0x = seq_tex[i], i0x = seq_iex[i];
      int slot = i0x, maxns = 0;
      for (int k0 = 0; k0 < ntiles; k0 += 64) {
        const int k = k0 + lane;
        const int t = ntiles - 1 - k;
        const int ns = k < ntiles ? tile_splits(t, L, p.G, ctx, off, p.window, p.pf_split_keys) : 0;
        const int incl = wave_inclusive_scan(ns);
        if (k < ntiles && t0x + k < p.pf_tile_cap) p.pf_tiles[t0x + k] = make_int4(s, t, slot + incl - ns, ns);
        slot += __builtin_amdgcn_readlane(incl, 63);
        maxns = max(maxns, ns);
      }
      for (int o = 32; o > 0; o >>= 1) maxns = max(maxns, __shfl_xor(maxns, o));
      int below = 0;  // items of the splits below ks
      for (int ks = 0; ks < maxns; ++ks) {
        int before = 0, sslot = i0x;  // tiles before this chunk with > ks splits; their partial slots
        for (int k0 = 0; k0 < ntiles; k0 += 64) {
          const int k = k0 + lane;
          const int t = ntiles - 1 - k;
          const int ns = k < ntiles ? tile_splits(t, L, p.G, ctx, off, p.window, p.pf_split_keys) : 0;
          const int has = ns > ks ? 1 : 0;
          const int hincl = wave_inclusive_scan(has);
          const int sincl = wave_inclusive_scan(ns);
          const int it = i0x + below + before + hincl - has;
          if (has && it < p.pf_item_cap) p.pf_items[it] = make_int4(s, t, ks, sslot + sincl - ns + ks);
          before += __builtin_amdgcn_readlane(hincl, 63);
          sslot += __builtin_amdgcn_readlane(sincl, 63);
        }
        below += before;
      }
    }
    tcarry += ttotal;
    icarry += itotal;
    __syncthreads();  // the shared per-sequence arrays are refilled by the next chunk
  }
  for (int i = tcarry + tid; i < p.pf_tile_cap; i += 1024) p.pf_tiles[i] = make_int4(-1, 0, 0, 0);
  for (int i = icarry + tid; i < p.pf_item_cap; i += 1024) p.pf_items[i] = make_int4(-1, 0, 0, 0);
  if (tid == 0) {
    const int pl = min(icarry, p.pf_item_cap), dl = min(dec_total, p.dec_cap);
    *p.hdr = make_int4(pl, dl, mix_order(pl, dl, p.hkv, p.slots), 0);
    UnitQueues* uq = reinterpret_cast<UnitQueues*>(p.hdr + 1);
    for (int x = 0; x < N_XCD; ++x) uq->next_pf[x] = uq->next_dec[x] = 0;
  }
}

// ---------------------------------------------------------------------------
// Decode: one wavefront per (sequence, KV head, split).
// ---------------------------------------------------------------------------
template <int D>
struct DecodeBuf {
  uint4 k[D / 32];  // this lane's slice of one K page (one key, 8 dims per MFMA)
  uint2 v[D / 16];  // this lane's slice of one V page (4 keys for each of D/16 dims)
};

// A wave-uniform pointer: both halves in SGPRs, so loads use the
// scalar-base + vector-offset + immediate-offset addressing form.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Issue one page's loads.  Every call issues exactly the same loads with
// constant offsets, so the next pages stay in flight while the current one is
// computed (a conditional load would make the compiler drain every load at the
// join).  `phys` is wave-uniform; an id out of range (a broken precondition,
// or the slots past the end of the split, which are never computed) reads
// page 0 instead.
template <int D, bool NT>
__device__ __forceinline__ void decode_issue(DecodeBuf<D>& B, const Params& p, int phys, int kvh,
                                             int koff, int voff) {
  const int pg = (unsigned)phys < (unsigned)p.num_pages ? phys : 0;
  const size_t slab = (size_t)pg * p.hkv + kvh;
  const uint16_t* kb = uniform_ptr(p.k_cache + slab * 16 * D);
  const uint16_t* vb = uniform_ptr(p.v_cache + slab * D * 16);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) B.k[c] = kv_load<NT>(reinterpret_cast<const uint4*>(kb + koff + 32 * c));
#pragma unroll
  for (int t = 0; t < D / 16; ++t) B.v[t] = kv_load<NT>(reinterpret_cast<const uint2*>(vb + voff + 256 * t));
}

// WIN: a sliding window is set (the full-attention instance carries none of its code)
template <int D, bool WIN>
__device__ __forceinline__ void decode_compute(DecodeBuf<D>& B, int pg, int ctx, int lo, int g,
                                               const bf16x8 (&qf)[D / 32], floatx4 (&o)[D / 16],
                                               float& m, float& l, float c) {
  floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cc = 0; cc < D / 32; ++cc)
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(B.k[cc]), qf[cc], sacc, 0, 0, 0);
  // lane holds S^T[key 4g + r][head lane % 16] (raw scores)
  float x[4] = {sacc[0], sacc[1], sacc[2], sacc[3]};
  if (pg * 16 + 16 > ctx) {  // the page that holds the context end
    const int n = ctx - (pg * 16 + 4 * g);  // valid keys among this lane's 4
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (r < n) ? x[r] : -INFINITY;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      B.v[t].x = keep16(B.v[t].x, 0, n);
      B.v[t].y = keep16(B.v[t].y, 2, n);
    }
  }
  if (WIN && pg * 16 < lo) {  // the page that holds the window start
    const int n = lo - (pg * 16 + 4 * g);  // keys below the window among this lane's 4
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (r < n) ? -INFINITY : x[r];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      B.v[t].x = drop16(B.v[t].x, 0, n);
      B.v[t].y = drop16(B.v[t].y, 2, n);
    }
  }
  float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  mx = pair_max32(pair_max16(mx));
  if ((mx - m) * c > CB_RESCALE_SLACK) {  // raise the running max (per head column)
    const float alpha = fast_exp2((m - mx) * c);  // m = -inf -> 0
    l *= alpha;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) o[t] *= alpha;
    m = mx;
  }
  const float nm = neg_scaled(m, c);
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(fmaf(x[r], c, nm));
  l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  const uint2 pk = make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_short4(B.v[t]), as_short4(pk), o[t], 0, 0, 0);
}

// NT: page loads with the non-temporal hint (the decode-only launch and the
// windowed mixed launch; in the unwindowed mixed launch plain loads measured
// slightly faster)
template <int D, bool WIN, bool NT>
__device__ __forceinline__ void decode_wave(const Params& p, int w) {
  const int kvh = w % p.hkv;
  const int j = w / p.hkv;
  if (j >= p.dec_cap) return;
  const int4 item = p.dec_items[j];
  // the record is the same for the whole wavefront: keep its fields in SGPRs
  const int s = __builtin_amdgcn_readfirstlane(item.x);
  if (s < 0) return;
  const int split = __builtin_amdgcn_readfirstlane(item.y);
  const int ctx = __builtin_amdgcn_readfirstlane(item.z);
  const int t = __builtin_amdgcn_readfirstlane(item.w);
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15, g = lane >> 4;
  const int G = p.G;
  const int npages = (ctx + 15) >> 4;
  const int lo = WIN ? window_first_key(ctx - 1, p.window) : 0;  // first key in the window
  const int pg0 = (lo >> 4) + split * p.split_pages;
  const int pg1 = min(pg0 + p.split_pages, npages);
  const int nsplit = ((WIN ? decode_pages(ctx, p.window) : npages) + p.split_pages - 1) / p.split_pages;
  const int32_t* btrow = p.bt + (p.bt_off ? (size_t)p.bt_off[s] : (size_t)s * p.bt_stride);
  // per-lane element offsets inside a (page, head) slab: K row hl, dims 8g + 32c;
  // V dim rows 16t + hl, keys 4g..4g+3
  const int koff = hl * D + g * 8;
  const int voff = hl * 16 + g * 4;

  // this split's physical page ids, one per lane in two registers (pages
  // 0..63 and 64..127 of the split, split_pages <= DEC_MAX_SPLIT); the wait
  // for them happens here, before any page load is in flight
  static_assert(DEC_MAX_SPLIT <= 128, "two page ids per lane");
  const int my_page = __builtin_amdgcn_readfirstlane(0) + ((lane < pg1 - pg0) ? btrow[pg0 + lane] : 0);
  const int my_page2 = pg1 - pg0 > 64 ? ((lane + 64 < pg1 - pg0) ? btrow[pg0 + 64 + lane] : 0) : 0;
  const int first_page = __builtin_amdgcn_readlane(my_page, 0);
  // ring of NB page buffers: page pg+PF is loading while page pg is computed
  constexpr int PF = CB_DEC_PREFETCH;
  constexpr int NB = PF + 1;
  DecodeBuf<D> buf[NB];
  decode_issue<D, NT>(buf[0], p, pg0 < pg1 ? first_page : -1, kvh, koff, voff);
#pragma unroll
  for (int r = 1; r < PF; ++r)
    decode_issue<D, NT>(buf[r], p, pg0 + r < pg1 ? __builtin_amdgcn_readlane(my_page, r) : -1, kvh, koff, voff);

  bf16x8 qf[D / 32];
  {
    const uint16_t* qrow = p.q + ((size_t)t * p.hq + kvh * G + hl) * D + g * 8;
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc)
      qf[cc] = as_bf16x8(hl < G ? *reinterpret_cast<const uint4*>(qrow + 32 * cc) : make_uint4(0, 0, 0, 0));
  }
  floatx4 o[D / 16];
#pragma unroll
  for (int tt = 0; tt < D / 16; ++tt) o[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const float c = p.scale_log2;

  for (int pg = pg0; pg < pg1; pg += NB) {
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const int cur = pg + r;
      const int nxt = cur + PF;
      // the lane index is taken mod 64 (pages past pg1 are never used)
      const int ix = nxt - pg0;
      const int phys = nxt < pg1 ? (ix < 64 ? __builtin_amdgcn_readlane(my_page, ix & 63)
                                            : __builtin_amdgcn_readlane(my_page2, ix & 63))
                                 : -1;
      decode_issue<D, NT>(buf[(r + PF) % NB], p, phys, kvh, koff, voff);
      if (cur < pg1) decode_compute<D, WIN>(buf[r], cur, ctx, lo, g, qf, o, m, l, c);
    }
  }

  l = pair_sum32(pair_sum16(l));
  if (hl >= G) return;
  if (nsplit == 1) {
    const float inv = 1.f / l;
    uint16_t* orow = p.out + ((size_t)t * p.hq + kvh * G + hl) * D;
#pragma unroll
    for (int tt = 0; tt < D / 16; ++tt) {
      const uint2 v = make_uint2(pack_bf16x2(o[tt][0] * inv, o[tt][1] * inv),
                                 pack_bf16x2(o[tt][2] * inv, o[tt][3] * inv));
      *reinterpret_cast<uint2*>(orow + 16 * tt + 4 * g) = v;
    }
  } else {
    const size_t prow = (size_t)w * G + hl;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* po = p.dec_o + prow * D;
#pragma unroll
    for (int tt = 0; tt < D / 16; ++tt)
      *reinterpret_cast<uint2*>(po + 16 * tt + 4 * g) = make_uint2(pack_f16x2(o[tt][0] * inv, o[tt][1] * inv),
                                                                   pack_f16x2(o[tt][2] * inv, o[tt][3] * inv));
    if (g == 0) p.dec_ml[prow] = make_float2(m, l);
  }
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup per (sequence, KV head, 128-row tile, key split).
// ---------------------------------------------------------------------------
// Direct copy of K/V tiles into LDS (global_load_lds_dwordx4: lane i of a
// wave's load writes 16 bytes at the LDS address in M0 plus 16 i, from any
// address of its own).  Each wave copies one page of a tile, K and V, in 1 KB
// loads; the per-lane source offsets are fixed, so a tile costs a wave one
// page address.  The immediate offset advances the source and the LDS
// destination together.
//
// K rows are stored unpadded with their 16-byte chunks permuted: logical chunk
// c of tile row r sits at chunk c ^ kswz(r), so the 16 rows that one chunk
// read of 16 lanes touches fall on 16 different 16-byte bank groups.
template <int D>
__host__ __device__ constexpr int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }

template <int J>
__device__ __forceinline__ void lds_copy16(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), reinterpret_cast<void*>(dst), 16, J * 1024, 0);
}

// Source offsets, per lane, of the NJ 1 KB loads that fill one page of K
// (each less the load's immediate offset J * 1 KB), and of the loads of one
// page of V (the same for every J: V rows of 32 bytes, halves swapped on rows
// with bit 3 set, as the P V reads expect).
template <int D>
struct PfDmaOffsets {
  static constexpr int NJ = D / 32;  // 1 KB loads per page slab (16 x D bf16)
  uint32_t k[NJ];
  uint32_t v;
  __device__ __forceinline__ explicit PfDmaOffsets(int lane) {
    constexpr int CPR = D / 8;           // 16-byte chunks per K row
    constexpr int RPL = 1024 / (2 * D);  // K rows per 1 KB load
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int rl = RPL * j + lane / CPR;  // page row this lane fills
      const int c = (lane % CPR) ^ kswz<D>(rl);
      k[j] = (uint32_t)((lane / CPR) * 2 * D + 16 * c);
    }
    v = (uint32_t)((lane >> 1) * 32 + 16 * ((lane & 1) ^ ((lane >> 4) & 1)));
  }
};

// Wave w copies page w of tile kt (K and V) into the LDS stage at `st`.
// Pages past the context (id -1) read page 0; their keys are masked and
// their V tokens zeroed where they are read.
template <int D>
__device__ __forceinline__ void pf_dma(uint8_t* st, const Params& p, const int* pids, int kt, int kt0, int kvh, int w,
                                       const PfDmaOffsets<D>& od) {
  constexpr int SLAB = 32 * D;  // bytes of one page of one KV head, K or V
  const int id = __builtin_amdgcn_readfirstlane(pids[(kt - kt0) * 4 + w]);
  const size_t slab = (size_t)((unsigned)id < (unsigned)p.num_pages ? id : 0) * p.hkv + kvh;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(p.k_cache) + slab * SLAB;
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(p.v_cache) + slab * SLAB;
  uint8_t* kl = st + w * SLAB;
  uint8_t* vl = st + PfLds<D>::K_BYTES + w * SLAB;
  // unsigned 32-bit offsets from a uniform base: the loads take their
  // scalar-base form (the empty asm keeps each offset 32-bit at its load)
  uint32_t o[PfDmaOffsets<D>::NJ + 1];
#pragma unroll
  for (int j = 0; j < PfDmaOffsets<D>::NJ; ++j) o[j] = od.k[j];
  o[PfDmaOffsets<D>::NJ] = od.v;
#pragma unroll
  for (int j = 0; j <= PfDmaOffsets<D>::NJ; ++j) asm volatile("" : "+v"(o[j]));
  lds_copy16<0>(kb + o[0], kl);
  lds_copy16<1>(kb + o[1], kl);
  if constexpr (PfDmaOffsets<D>::NJ > 2) {
    lds_copy16<2>(kb + o[2], kl);
    lds_copy16<3>(kb + o[3], kl);
  }
  const uint32_t ov = o[PfDmaOffsets<D>::NJ];
  lds_copy16<0>(vb + ov, vl);
  lds_copy16<1>(vb + ov, vl);
  if constexpr (PfDmaOffsets<D>::NJ > 2) {
    lds_copy16<2>(vb + ov, vl);
    lds_copy16<3>(vb + ov, vl);
  }
}

// Wait for this wave's LDS copies (vmcnt 0; the other counters untouched).
__device__ __forceinline__ void wait_lds_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Once wave w's copy of a tile has landed: the V tokens of its page outside
// [lo, hi) (page-relative; wave-uniform) are zeroed in the LDS stage.  The
// copy brings whatever the page holds past the context end (and, under a
// window, below the tile's floor); P is 0 there, but 0 * NaN is not, and
// zeroing them here once keeps the P V product free of per-tile masks.
// V rows are 32 bytes (one dim, 16 tokens); physical half ph of row r holds
// tokens 8 (ph ^ r[3]) .. +7.
template <int D>
__device__ __forceinline__ void pf_zero_v(uint8_t* st, int w, int lane, int lo, int hi) {
  uint8_t* vp = st + PfLds<D>::K_BYTES + w * 32 * D;
#pragma unroll
  for (int r0 = 0; r0 < D; r0 += 64) {
    const int r = r0 + lane;
    const int f = (r >> 3) & 1;
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      uint4* a = reinterpret_cast<uint4*>(vp + r * 32 + 16 * ph);
      const int e = 8 * (ph ^ f);  // first token of this half
      uint4 x = *a;
      x.x = drop16(keep16(x.x, e + 0, hi), e + 0, lo);
      x.y = drop16(keep16(x.y, e + 2, hi), e + 2, lo);
      x.z = drop16(keep16(x.z, e + 4, hi), e + 4, lo);
      x.w = drop16(keep16(x.w, e + 6, hi), e + 6, lo);
      *a = x;
    }
  }
}

// Order of the N LDS fragment reads and the N MFMAs that take them, one each
// (scheduler groups), in batches of R: the next batch's reads go out right
// after the first MFMA of the current one.  While LDS copies are in flight
// the compiler waits for all outstanding LDS reads before an MFMA that needs
// one; in this order such a wait only covers reads issued R-1 MFMAs earlier.
template <int N>
__device__ __forceinline__ void pf_read_schedule() {
  constexpr int R = CB_PF_READAHEAD;
  static_assert(R > 0 && N % R == 0, "batches of R");
  __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // DS reads
#pragma unroll
  for (int b = 0; b < N / R; ++b) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if (b + 1 < N / R) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, R - 1, 0);
  }
}

template <int D, bool WIN>
__device__ __forceinline__ void prefill_tile(const Params& p, int b) {
  using Lds = PfLds<D>;
  const int kvh = b % p.hkv;
  const int j = b / p.hkv;
  if (j >= p.pf_item_cap) return;
  const int4 item = p.pf_items[j];  // uniform over the workgroup
  const int s = __builtin_amdgcn_readfirstlane(item.x);
  if (s < 0) return;
  const int tile = __builtin_amdgcn_readfirstlane(item.y);
  const int ks = __builtin_amdgcn_readfirstlane(item.z);
  const int slot = __builtin_amdgcn_readfirstlane(item.w);  // where this split's partials go
  const int G = p.G;
  const int t0 = p.qsl[s];
  const int L = p.qsl[s + 1] - t0;
  const int ctx = p.ctx_lens[s];
  const int off = p.q_off[s];
  const int nsplit = tile_splits(tile, L, G, ctx, off, WIN ? p.window : 0, p.pf_split_keys);
  if (nsplit > 1 && slot >= p.pf_item_cap) return;  // work list overflowed (precondition broken)
  const int npages = (ctx + 15) >> 4;
  const int R = L * G;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, gg = lane >> 5;
  const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);  // l32 with bits 2, 3 swapped
  const int vhalf = 16 * (gg ^ ((l32 >> 3) & 1));  // this lane's 16-byte half of a V row in LDS
  const int W = WIN ? p.window : 0;

  // this lane's row (GQA-packed: row = query token * G + head in the group)
  const int row = tile * PF_ROWS + wv * 32 + l32;
  const bool rvalid = row < R;
  const int qi = row / G, hh = row - qi * G;
  const int kcap = min(off + qi, ctx - 1);           // last key this row may see
  const int kfirst = window_first_key(off + qi, W);  // first key this row may see

  // this item's key range, in whole 64-key tiles, from the tile's first row's window
  const int k_lo = (WIN ? tile_key_base(tile, G, off, W) : 0) + ks * p.pf_split_keys;
  const int k_hi = min(k_lo + p.pf_split_keys, tile_key_end(tile, L, G, ctx, off));
  const int kt0 = k_lo / PF_KEYS, kt1 = (k_hi + PF_KEYS - 1) / PF_KEYS;
  const int kfloor = window_first_key(off + tile * PF_ROWS / G, W);  // no row of the tile sees below
  const int w_first_row = tile * PF_ROWS + wv * 32;
  const int w_last_row = min(w_first_row + 31, R - 1);
  const int w_kend = __builtin_amdgcn_readfirstlane((w_first_row < R) ? min(ctx, off + w_last_row / G + 1) : 0);
  // keys below are visible to every row...
  const int w_kfull = __builtin_amdgcn_readfirstlane(min(ctx, off + w_first_row / G + 1));
  const int w_klo_min = window_first_key(off + w_first_row / G, W);  // ...and at or above the window
  const int w_klo_max = window_first_key(off + w_last_row / G, W);  // of the wave's last row

  constexpr int NK = D / 16;  // QK k-steps of 16 dims
  constexpr int NO = D / 32;  // 32-dim output tiles
  const int32_t* btrow = p.bt + (p.bt_off ? (size_t)p.bt_off[s] : (size_t)s * p.bt_stride);
  // LDS: two tile stages and the item's page ids.  The stages are separate
  // arrays so that the compiler can tell a copy in flight into one stage does
  // not touch the stage being read; being larger and more aligned they are
  // laid out first, which keeps the copies' LDS destinations below 64 KB.
  static_assert(PF_WAVES == 4, "one wave per page of a 64-key tile");
  __shared__ __attribute__((aligned(1024))) uint8_t lds_st0[Lds::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_st1[Lds::STAGE];
  __shared__ __attribute__((aligned(4))) int lds_ids[PF_MAX_PAGES];
  // the item's page ids, staged once (at most PF_MAX_PAGES; the host caps the key range)
  int* pids = lds_ids;
  for (int i = tid; i < (kt1 - kt0) * 4; i += PF_THREADS) {
    const int pg = kt0 * 4 + i;
    pids[i] = pg < npages ? btrow[pg] : -1;
  }
  __syncthreads();
  // The query fragments first: they are waited for once, before the loop (a
  // load still pending at the loop header would make the compiler wait for
  // it inside the loop, behind the tile copies).
  bf16x8 qf[NK];
  {
    const uint16_t* qrow = p.q + ((size_t)(t0 + qi) * p.hq + kvh * G + hh) * D + 8 * gg;
#pragma unroll
    for (int cc = 0; cc < NK; ++cc)
      qf[cc] = as_bf16x8(rvalid ? *reinterpret_cast<const uint4*>(qrow + 16 * cc) : make_uint4(0, 0, 0, 0));
  }
  // the first tile's copy starts now; the loop below keeps one tile in flight
  const int wu = __builtin_amdgcn_readfirstlane(wv);
  const PfDmaOffsets<D> od(lane);
  uint8_t* stage0 = lds_st0;
  uint8_t* stage1 = lds_st1;
  if (kt0 < kt1) pf_dma<D>(stage0, p, pids, kt0, kt0, kvh, wu, od);
  // this lane's K read offsets in a stage: row krow, logical chunk 2 cc + gg
  uint32_t krd[NK];
#pragma unroll
  for (int cc = 0; cc < NK; ++cc) krd[cc] = (uint32_t)(krow * Lds::KROW + 16 * ((2 * cc + gg) ^ kswz<D>(krow)));
#pragma unroll
  for (int cc = 0; cc < NK; ++cc) {
    const uint4 qq = __builtin_bit_cast(uint4, qf[cc]);
    asm volatile("" ::"v"(qq.x), "v"(qq.y), "v"(qq.z), "v"(qq.w));
  }
  floatx16 o[NO];
#pragma unroll
  for (int dt = 0; dt < NO; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float c = p.scale_log2;

  // this wave's page of tile kt, just landed in `st`: zero the V tokens no
  // row of the tile may see (only on the tile that holds the context end, or
  // under a window the one that holds the floor)
  auto fix_tile = [&](int kt, uint8_t* st) {
    const int kb = kt * PF_KEYS + 16 * wu;
    const int hi = ctx - kb, lo = WIN ? kfloor - kb : 0;
    if (hi < 16 || (WIN && lo > 0)) pf_zero_v<D>(st, wu, lane, lo, hi);
  };
  wait_lds_copies();
  if (kt0 < kt1) fix_tile(kt0, stage0);
  __syncthreads();
  auto tile_step = [&](int kt, const uint8_t* cur) {
    const int kbase = kt * PF_KEYS;
    if (kbase < w_kend && (!WIN || kbase + PF_KEYS > w_klo_min)) {
      const uint8_t* kl = cur;
      const uint8_t* vl = cur + Lds::K_BYTES;
      // S^T = K Q^T for two 32-key subtiles.  MFMA row m reads key krow(m)
      // (bits 2 and 3 of m swapped), so that lane (l32, gg) receives, for
      // r = 0..15, key 16(r/8) + 8gg + r%8 of its subtile: the 8 consecutive
      // keys the P V product takes from it, with no exchange between lanes.
      floatx16 sc[2];
      if (CB_PF_PRIO) __builtin_amdgcn_s_setprio(1);  // the other wave's VALU work fills the MFMA gaps
      // the two subtiles' accumulations alternate; the K fragment reads go
      // out in batches ahead of their MFMAs
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[sub][r] = 0.f;
#pragma unroll
      for (int cc = 0; cc < NK; ++cc)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const uint4 ka = *reinterpret_cast<const uint4*>(kl + sub * 32 * Lds::KROW + krd[cc]);
          sc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), qf[cc], sc[sub], 0, 0, 0);
        }
      if constexpr (CB_PF_READAHEAD > 0) pf_read_schedule<2 * NK>();
      if (CB_PF_PRIO) __builtin_amdgcn_s_setprio(0);
      // straddles this wave's diagonal (or the context end), or its window's lower edge
      if (kbase + PF_KEYS > w_kfull || (WIN && kbase < w_klo_max)) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + sub * 32 + 16 * (r >> 3) + 8 * gg + (r & 7);
            sc[sub][r] = (key <= kcap && (!WIN || key >= kfirst)) ? sc[sub][r] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[sub][r]);
      mx = pair_max32(mx);
      const bool raise = (mx - m) * c > CB_RESCALE_SLACK;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float alpha = raise ? fast_exp2((m - mx) * c) : 1.f;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < NO; ++dt) o[dt] *= alpha;
        m = raise ? mx : m;
      }
      const float nm = neg_scaled(m, c);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[sub][r] = fast_exp2(fmaf(sc[sub][r], c, nm));

      // O^T += V^T P^T, four 16-key steps (page 2*sub + half of the tile):
      // lane (l32, gg) holds P for keys 8gg..8gg+7 of the page, and reads V
      // for the same keys as one contiguous 16-byte load.  The row sum is
      // taken from the same bf16 P (a two-term dot product with ones per
      // packed pair), so the normaliser weighs exactly what P V does.
      // V tokens past the context end (or below the window floor) were
      // zeroed in LDS when their tile landed (pf_zero_v)
      float rsum[2] = {0.f, 0.f};
      {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int r0 = 8 * half;
            const uint4 pb = make_uint4(pack_bf16x2(sc[sub][r0 + 0], sc[sub][r0 + 1]),
                                        pack_bf16x2(sc[sub][r0 + 2], sc[sub][r0 + 3]),
                                        pack_bf16x2(sc[sub][r0 + 4], sc[sub][r0 + 5]),
                                        pack_bf16x2(sc[sub][r0 + 6], sc[sub][r0 + 7]));
            rsum[half] = sum_bf16x8(pb, rsum[half]);
            const uint8_t* vpage = vl + (2 * sub + half) * D * Lds::VROW;
#pragma unroll
            for (int dt = 0; dt < NO; ++dt) {
              const uint4 va = *reinterpret_cast<const uint4*>(vpage + (32 * dt + l32) * Lds::VROW + vhalf);
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb), o[dt], 0, 0, 0);
            }
          }
        if constexpr (CB_PF_READAHEAD > 0) pf_read_schedule<4 * NO>();  // V fragments likewise
      }
      l += rsum[0] + rsum[1];
    }
  };
  // two LDS stages: tile kt+1 is copied into one while tile kt is computed
  // from the other; the barrier after each tile both publishes the next
  // tile's copy and frees the stage just read
  for (int kt = kt0; kt < kt1; kt += 2) {
    if (kt + 1 < kt1) pf_dma<D>(stage1, p, pids, kt + 1, kt0, kvh, wu, od);
    tile_step(kt, stage0);
    wait_lds_copies();
    if (kt + 1 < kt1) fix_tile(kt + 1, stage1);
    __syncthreads();
    if (kt + 1 >= kt1) break;
    if (kt + 2 < kt1) pf_dma<D>(stage0, p, pids, kt + 2, kt0, kvh, wu, od);
    tile_step(kt + 1, stage1);
    wait_lds_copies();
    if (kt + 2 < kt1) fix_tile(kt + 2, stage0);
    __syncthreads();
  }

  const float lt = pair_sum32(l);
  if (!rvalid) return;
  if (nsplit == 1) {
    const float inv = 1.f / lt;
    uint16_t* orow = p.out + ((size_t)(t0 + qi) * p.hq + kvh * G + hh) * D;
#pragma unroll
    for (int dt = 0; dt < NO; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint2 v = make_uint2(pack_bf16x2(o[dt][4 * q4 + 0] * inv, o[dt][4 * q4 + 1] * inv),
                                   pack_bf16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv));
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * q4 + 4 * gg) = v;
      }
  } else {
    const size_t prow = ((size_t)slot * p.hkv + kvh) * PF_ROWS + wv * 32 + l32;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;  // 0: every key of this range is above the row's diagonal
    uint16_t* po = p.pf_o + prow * D;
#pragma unroll
    for (int dt = 0; dt < NO; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<uint2*>(po + 32 * dt + 8 * q4 + 4 * gg) =
            make_uint2(pack_f16x2(o[dt][4 * q4 + 0] * inv, o[dt][4 * q4 + 1] * inv),
                       pack_f16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv));
    if (gg == 0) p.pf_ml[prow] = make_float2(m, lt);
  }
}

// ---------------------------------------------------------------------------
// The ragged launch: blocks [0, pf_blocks) are prefill items, the rest carry
// four decode wavefronts each.  The no-prefill instantiation needs neither
// LDS nor the prefill registers and runs at higher occupancy.
// ---------------------------------------------------------------------------
// CU split: a unit of one kind, numbered i, belongs to XCD i % 8 (blocks
// are dealt to the XCDs round-robin, so prefill unit i keeps its KV head's
// XCD); a workgroup claims the next unit of its XCD's queue, then of the
// other XCDs' queues.  -1: every unit of this kind is taken.
__device__ __forceinline__ int take_unit(int* next, int n, int xcc) {
  for (int k = 0; k < N_XCD; ++k) {
    const int x = (xcc + k) & (N_XCD - 1);
    const int cnt = n > x ? (n - x + N_XCD - 1) / N_XCD : 0;
    if (cnt == 0) continue;
    const int q = atomicAdd(&next[x], 1);
    if (q < cnt) return x + N_XCD * q;
  }
  return -1;
}
// Workgroups on CUs 1..k of each shader engine take prefill units, the
// others decode units; either kind falls back to the other when its own is
// used up.  The launch holds exactly as many workgroups as units, so every
// workgroup gets one.  Returns the prefill unit, -2 - (decode unit), or -1.
__device__ int pick_unit(const Params& p, int lp, int ld, int k) {
  const unsigned hw = (unsigned)__builtin_amdgcn_s_getreg(63492);          // HW_ID
  const int xcc = (int)((unsigned)__builtin_amdgcn_s_getreg(63508) & 7u);  // XCC_ID
  const int cu = (int)((hw >> 8) & 15u);
  UnitQueues* q = reinterpret_cast<UnitQueues*>(p.hdr + 1);
  if (cu >= 1 && cu <= k) {
    const int r = take_unit(q->next_pf, lp, xcc);
    if (r >= 0) return r;
    const int d = take_unit(q->next_dec, ld, xcc);
    return d >= 0 ? -2 - d : -1;
  }
  const int d = take_unit(q->next_dec, ld, xcc);
  if (d >= 0) return -2 - d;
  const int r = take_unit(q->next_pf, lp, xcc);
  return r >= 0 ? r : -1;
}

template <int D, bool WIN>
__global__ __launch_bounds__(PF_THREADS, 512 / PF_THREADS) void attn_mixed_kernel(Params p) {
  const int b = blockIdx.x;
  const int np = p.pf_blocks, nd = p.dec_blocks;
  // live blocks first, in the order the header names; a grid sized by the
  // caps has blocks past the live work, which return at once
  const int4 h = *p.hdr;
  const int lp = min(h.x * p.hkv, np);
  const int ld = min((h.y * p.hkv + PF_WAVES - 1) / PF_WAVES, nd);
  int pf = -1, dec = -1;
  if (CB_CU_SPLIT && h.w > 0 && lp > 0 && ld > 0) {
    if (b >= lp + ld) return;
    __shared__ int picked;
    if (threadIdx.x == 0) picked = pick_unit(p, lp, ld, h.w);
    __syncthreads();
    const int r = picked;
    if (r >= 0) pf = r;
    else if (r <= -2) dec = -2 - r;
    else return;
  } else if (b < lp + ld) {
    // interleaved: groups of 8 alternate; blocks go to the XCDs round-robin,
    // so every prefill index stays on the XCD it has in prefill-first order
    const int m8 = h.z ? (min(lp, ld) & ~7) : 0;
    if (b < 2 * m8) {
      const int grp = b >> 4, w = b & 15;
      if (w < 8) pf = 8 * grp + w;
      else dec = 8 * grp + w - 8;
    } else {
      const int r = b - 2 * m8;
      if (r < lp - m8) pf = m8 + r;
      else dec = m8 + r - (lp - m8);
    }
  } else {
    return;  // past the live work (the grid is sized by the caps): nothing to do
  }
  clock_mark(p, 0);
  if (pf >= 0) {
    prefill_tile<D, WIN>(p, pf);
    clock_mark(p, 1);
    return;
  }
  decode_wave<D, WIN, (WIN ? CB_NT_MIXED_WINDOW : CB_NT_MIXED) != 0>(p, dec * PF_WAVES + (threadIdx.x >> 6));
  clock_mark(p, 1);
}

template <int D, bool WIN>
__global__ __launch_bounds__(CB_DEC_WG, CB_DEC_WAVES_PER_SIMD) void attn_decode_kernel(Params p) {
  clock_mark(p, 0);
  decode_wave<D, WIN, CB_NT_DECODE>(p, (int)blockIdx.x * (CB_DEC_WG / 64) + (threadIdx.x >> 6));
  clock_mark(p, 1);
}

// ---------------------------------------------------------------------------
// Combine: blocks [0, comb_dec_blocks) merge decode splits, one wavefront per
// (decode sequence, query head); the rest merge prefill key splits, one
// workgroup per (row tile, KV head), two threads per row.
// ---------------------------------------------------------------------------
template <int D>
__device__ void combine_decode(const Params& p, int wave) {
  constexpr int E = D / 64;
  if (wave >= p.num_decodes * p.hq) return;
  const int lane = threadIdx.x & 63;
  const int s = wave / p.hq, h = wave % p.hq;
  const int G = p.G, kvh = h / G, hl = h % G;
  const int ctx = p.ctx_lens[s];
  const int nsplit = (decode_pages(ctx, p.window) + p.split_pages - 1) / p.split_pages;
  if (nsplit <= 1) return;
  const int j0 = p.dec_first[s];
  const int jr = p.dec_rem[s];
  const int nfull = jr >= 0 ? nsplit - 1 : nsplit;
  if (j0 + nfull > p.dec_cap || jr >= p.dec_cap) return;  // work list overflowed (precondition broken)
  // split i lives at item j0 + i (full splits) or jr (the short last split)
  auto item_of = [&](int i) { return i < nfull ? j0 + i : jr; };
  const float c = p.scale_log2;
  // lane l merges output dims E*l .. E*l + E-1 (one 4-byte fp16 pair at D 128)
  static_assert(E == 1 || E == 2, "D 64 or 128");
  constexpr int U = 8;  // splits whose values are loaded together
  auto prow_of = [&](int i) { return ((size_t)item_of(min(i, nsplit - 1)) * p.hkv + kvh) * G + hl; };
  auto load_vals = [&](int i0, float (&val)[U][E]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint16_t* po = p.dec_o + prow_of(i0 + u) * D + E * lane;
      if constexpr (E == 2) {
        const f16x2 h2 = __builtin_bit_cast(f16x2, *reinterpret_cast<const uint32_t*>(po));
        val[u][0] = (float)h2[0];
        val[u][1] = (float)h2[1];
      } else {
        val[u][0] = (float)__builtin_bit_cast(_Float16, *po);
      }
    }
  };
  // the first splits' values are in flight while the weights are formed
  float val[U][E];
  load_vals(0, val);
  // split i's weight is its sum rescaled to the common maximum M; up to 128
  // splits the weights stay in two registers per lane (splits l and l + 64)
  // and the loop below takes them with readlane, with no second load
  const bool few = nsplit <= 128;
  float M = -INFINITY, lsum = 0.f, w0 = 0.f, w1 = 0.f;
  if (few) {
    const float2 a = lane < nsplit ? p.dec_ml[prow_of(lane)] : make_float2(-INFINITY, 0.f);
    const float2 b = lane + 64 < nsplit ? p.dec_ml[prow_of(lane + 64)] : make_float2(-INFINITY, 0.f);
    M = fmaxf(a.x, b.x);
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    w0 = lane < nsplit ? fast_exp2((a.x - M) * c) * a.y : 0.f;
    w1 = lane + 64 < nsplit ? fast_exp2((b.x - M) * c) * b.y : 0.f;
    lsum = w0 + w1;
  } else {
    for (int i = lane; i < nsplit; i += 64) M = fmaxf(M, p.dec_ml[prow_of(i)].x);
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    for (int i = lane; i < nsplit; i += 64) {
      const float2 ml = p.dec_ml[prow_of(i)];
      lsum += fast_exp2((ml.x - M) * c) * ml.y;
    }
  }
  for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int i0 = 0; i0 < nsplit; i0 += U) {
    if (i0 > 0) load_vals(i0, val);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u;
      float w;
      if (few) {
        const int li = i & 63;
        const float wa = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w0), li));
        const float wb = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w1), li));
        w = i < 64 ? wa : wb;
      } else {
        const float2 ml = p.dec_ml[prow_of(i)];
        w = fast_exp2((ml.x - M) * c) * ml.y;
      }
      w = i < nsplit ? w : 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(w, val[u][e], acc[e]);
    }
  }
  const float inv = 1.f / lsum;
  uint16_t* orow = p.out + ((size_t)p.qsl[s] * p.hq + h) * D + E * lane;
  if constexpr (E == 2) {
    *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    *orow = __builtin_bit_cast(uint16_t, (__bf16)(acc[0] * inv));
  }
}

// One workgroup per (row tile, KV head, block of 16 rows): 16 threads per row,
// each merging D/16 output dimensions over the tile's key splits.
constexpr int CP_ROWS = 16;
template <int D>
__device__ void combine_prefill(const Params& p, int gb) {
  constexpr int E = D / 16;                 // dims per thread
  const int rb = gb % (PF_ROWS / CP_ROWS);
  const int tk = gb / (PF_ROWS / CP_ROWS);
  const int kvh = tk % p.hkv;
  const int tj = tk / p.hkv;
  if (tj >= p.pf_tile_cap) return;
  const int4 tr = p.pf_tiles[tj];
  if (tr.x < 0 || tr.w <= 1) return;
  const int s = tr.x, tile = tr.y, first = tr.z, nsplit = tr.w;
  if (first + nsplit > p.pf_item_cap) return;
  const int G = p.G;
  const int t0 = p.qsl[s];
  const int R = (p.qsl[s + 1] - t0) * G;
  const int rl = rb * CP_ROWS + (threadIdx.x >> 4);   // row within the tile
  const int dc = (threadIdx.x & 15) * E;               // first output dim
  const int row = tile * PF_ROWS + rl;
  if (row >= R) return;
  const float c = p.scale_log2;
  // Splits are merged in groups of U with a running maximum; the next
  // group's loads are in flight while one group is merged, so a long list of
  // splits costs about one memory round trip per group, a short one one.
  constexpr int U = 4;
  struct Group {
    float2 ml[U];
    uint2 v[U][E / 4];
  };
  auto load = [&](int i0, Group& g) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < nsplit) {  // the same for the whole workgroup
        const size_t prow = ((size_t)(first + i0 + u) * p.hkv + kvh) * PF_ROWS + rl;
        g.ml[u] = p.pf_ml[prow];
        const uint2* po = reinterpret_cast<const uint2*>(p.pf_o + prow * D + dc);
#pragma unroll
        for (int e = 0; e < E / 4; ++e) g.v[u][e] = po[e];
      } else {
        g.ml[u] = make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int e = 0; e < E / 4; ++e) g.v[u][e] = make_uint2(0, 0);
      }
    }
  };
  float M = -INFINITY, lsum = 0.f;
  floatx4 acc[E / 4];
#pragma unroll
  for (int e = 0; e < E / 4; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
  Group cur, nxt;
  load(0, cur);
  for (int i0 = 0; i0 < nsplit; i0 += U) {
    if (i0 + U < nsplit) load(i0 + U, nxt);
    float gm = M;
#pragma unroll
    for (int u = 0; u < U; ++u) gm = fmaxf(gm, cur.ml[u].x);
    // a larger maximum rescales what is merged so far (nothing while M = -inf)
    const float r = M == -INFINITY ? 0.f : fast_exp2((M - gm) * c);
    lsum *= r;
#pragma unroll
    for (int e = 0; e < E / 4; ++e) acc[e] *= r;
    M = gm;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // the split's weight: its sum, rescaled to the running maximum (0 when
      // every key of the range was above the row's diagonal, or past the list)
      const float2 ml = cur.ml[u];
      const float w = ml.x == -INFINITY ? 0.f : fast_exp2((ml.x - M) * c) * ml.y;
      lsum += w;
#pragma unroll
      for (int e = 0; e < E / 4; ++e) {
        const float4 v = unpack_f16x4(cur.v[u][e]);
        acc[e] += w * floatx4{v.x, v.y, v.z, v.w};
      }
    }
    if (i0 + U < nsplit) cur = nxt;
  }
  const float inv = 1.f / lsum;
  const int qi = row / G, hh = row - qi * G;
  uint16_t* orow = p.out + ((size_t)(t0 + qi) * p.hq + kvh * G + hh) * D + dc;
#pragma unroll
  for (int e = 0; e < E / 4; ++e) {
    const uint2 v = make_uint2(pack_bf16x2(acc[e][0] * inv, acc[e][1] * inv),
                               pack_bf16x2(acc[e][2] * inv, acc[e][3] * inv));
    *reinterpret_cast<uint2*>(orow + 4 * e) = v;
  }
}

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(Params p) {
  if ((int)blockIdx.x < p.comb_dec_blocks)
    combine_decode<D>(p, (int)blockIdx.x * 4 + (threadIdx.x >> 6));
  else
    combine_prefill<D>(p, (int)blockIdx.x - p.comb_dec_blocks);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const Bf16Plan& pl, const WorkLists* lists, hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k_cache = static_cast<const uint16_t*>(a.k_cache);
  p.v_cache = static_cast<const uint16_t*>(a.v_cache);
  p.bt = a.block_tables;
  p.qsl = a.qsl;
  p.ctx_lens = a.ctx_lens;
  p.q_off = a.q_offsets;
  p.out = static_cast<uint16_t*>(a.out);
  p.hdr = reinterpret_cast<int4*>(ws + pl.off_hdr);
  p.dec_items = reinterpret_cast<int4*>(ws + pl.off_dec_items);
  p.pf_items = reinterpret_cast<int4*>(ws + pl.off_pf_items);
  p.pf_tiles = reinterpret_cast<int4*>(ws + pl.off_pf_tiles);
  p.dec_first = reinterpret_cast<int32_t*>(ws + pl.off_dec_first);
  p.dec_rem = reinterpret_cast<int32_t*>(ws + pl.off_dec_rem);
  p.dec_ml = reinterpret_cast<float2*>(ws + pl.off_dec_ml);
  p.dec_o = reinterpret_cast<uint16_t*>(ws + pl.off_dec_o);
  p.pf_ml = reinterpret_cast<float2*>(ws + pl.off_pf_ml);
  p.pf_o = reinterpret_cast<uint16_t*>(ws + pl.off_pf_o);
  p.bt_stride = a.bt_stride;
  p.bt_off = a.bt_offsets;
  p.num_seqs = a.num_seqs;
  p.num_decodes = a.num_decodes;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.G = a.hq / a.hkv;
  p.num_pages = a.num_pages;
  p.split_pages = pl.split_pages;
  p.pf_split_keys = pl.pf_split_keys;
  p.dec_cap = (int32_t)pl.dec_cap;
  p.pf_tile_cap = (int32_t)pl.pf_tile_cap;
  p.pf_item_cap = (int32_t)pl.pf_item_cap;
  p.scale_log2 = a.scale * LOG2E;
  p.clk = static_cast<unsigned long long*>(g_prof_clock);
  p.window = a.window;
  const int64_t pf_blocks = pl.pf_item_cap * a.hkv;
  const int64_t dec_blocks = (pl.dec_cap * a.hkv + PF_WAVES - 1) / PF_WAVES;
  p.pf_blocks = (int32_t)pf_blocks;
  p.dec_blocks = (int32_t)dec_blocks;
  p.slots = pl.slots > 0 ? pl.slots : mixed_slots(D);
  const bool dec_splits = a.num_decodes > 0 && (int64_t)pl.split_pages * 16 < a.max_context_len;
  int64_t comb_dec = dec_splits ? ((int64_t)a.num_decodes * a.hq + 3) / 4 : 0;
  int64_t comb_pf = pl.pf_may_split ? pl.pf_tile_cap * a.hkv * (PF_ROWS / CP_ROWS) : 0;
  if (lists && lists->live_pf_items >= 0 && lists->live_dec_items >= 0) {
    // the caller's lists say which kinds actually split this step
    if (!lists->dec_split) comb_dec = 0;
    if (!lists->pf_split) comb_pf = 0;
  }
  p.comb_dec_blocks = (int32_t)comb_dec;

  if (lists) {  // built by the caller: read them where they were uploaded
    p.hdr = const_cast<int4*>(static_cast<const int4*>(lists->hdr));
    p.dec_items = const_cast<int4*>(static_cast<const int4*>(lists->dec_items));
    p.pf_items = const_cast<int4*>(static_cast<const int4*>(lists->pf_items));
    p.pf_tiles = const_cast<int4*>(static_cast<const int4*>(lists->pf_tiles));
    p.dec_first = const_cast<int32_t*>(lists->dec_first);
    p.dec_rem = const_cast<int32_t*>(lists->dec_rem);
  } else {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, p);
  }
  if (g_prof_start) (void)hipEventRecord(g_prof_start, stream);
  const bool win = a.window > 0;
  if (pf_blocks > 0) {
    int64_t nblk = pf_blocks + dec_blocks;
    if (lists && lists->live_pf_items >= 0 && lists->live_dec_items >= 0)
      nblk = std::min<int64_t>(pf_blocks, lists->live_pf_items * a.hkv) +
             std::min<int64_t>(dec_blocks, (lists->live_dec_items * a.hkv + PF_WAVES - 1) / PF_WAVES);
    const dim3 grid((unsigned)std::max<int64_t>(nblk, 1));
    if (win) hipLaunchKernelGGL((attn_mixed_kernel<D, true>), grid, dim3(PF_THREADS), 0, stream, p);
    else hipLaunchKernelGGL((attn_mixed_kernel<D, false>), grid, dim3(PF_THREADS), 0, stream, p);
  } else if (dec_blocks > 0) {
    int64_t waves = pl.dec_cap * a.hkv;
    if (lists && lists->live_dec_items >= 0) waves = std::min<int64_t>(waves, lists->live_dec_items * a.hkv);
    const dim3 grid((unsigned)std::max<int64_t>((waves + CB_DEC_WG / 64 - 1) / (CB_DEC_WG / 64), 1));
    if (win) hipLaunchKernelGGL((attn_decode_kernel<D, true>), grid, dim3(CB_DEC_WG), 0, stream, p);
    else hipLaunchKernelGGL((attn_decode_kernel<D, false>), grid, dim3(CB_DEC_WG), 0, stream, p);
  }
  if (g_prof_stop) (void)hipEventRecord(g_prof_stop, stream);
  if (comb_dec + comb_pf > 0)
    hipLaunchKernelGGL(combine_kernel<D>, dim3((unsigned)(comb_dec + comb_pf)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Workgroups of the mixed launch the current device holds at once: the
// kernel's occupancy per CU (LDS and registers; 2 for D 128) times the CU
// count.  Cached per device and head size; 512 when there is no device.
int mixed_slots(int head_dim) {
  static std::atomic<int> cache[64][2];
  const int hd = head_dim == 64 ? 1 : 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  int v = cache[dev][hd].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  const void* f = hd ? reinterpret_cast<const void*>(&attn_mixed_kernel<64, false>)
                     : reinterpret_cast<const void*>(&attn_mixed_kernel<128, false>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, f, PF_THREADS, 0) != hipSuccess || per <= 0) per = 2;
  v = cus * per;
  cache[dev][hd].store(v, std::memory_order_relaxed);
  return v;
}

Bf16Plan plan_bf16(int32_t num_seqs, int32_t num_decodes, int32_t num_tokens, int32_t hq, int32_t hkv,
                   int32_t head_dim, int32_t max_context_len, int32_t window) {
  Bf16Plan pl{};
  const int64_t max_pages = (max_context_len + 15) / 16;
  const int64_t G = hkv > 0 ? hq / hkv : 1;
  // decode: the longest split (pages per wavefront) that still gives the
  // decode grid >= 6k wavefronts (three rounds of the mixed launch's 2k slots),
  // or >= 4k when no prefill work shares the launch; longer splits write
  // fewer partials for the combine and start fewer wavefronts.  max_pages is
  // the step's longest context, which in a mixed step is usually a prefill
  // sequence's, so there the wave count is overestimated: mixed launches
  // stop at 64-page splits.
  const int64_t lanes = (int64_t)num_decodes * hkv;
  const bool with_prefill = num_seqs > num_decodes;
  const int64_t min_waves = with_prefill ? CB_DEC_MIN_WAVES : CB_DEC_MIN_WAVES_ALONE;
  pl.split_pages = 8;
  for (int sp : {DEC_MAX_SPLIT, 64, 32, 16}) {
    if (with_prefill && sp > 64) continue;
    if (lanes * ((max_pages + sp - 1) / sp) >= min_waves) { pl.split_pages = sp; break; }
  }
  // the items per decode sequence this allows sizes the work lists and the
  // partials (the workspace bound, which does not depend on the window)
  const int64_t budget = (max_pages + pl.split_pages - 1) / pl.split_pages;
  pl.dec_cap = (int64_t)num_decodes * budget;
  if (window > 0) {
    // a decode reads only its window's pages: within the same item budget,
    // the longest split that still reaches the wavefront count, else the
    // one that gives the most wavefronts
    const int64_t wpages = std::min<int64_t>(max_pages, ((int64_t)window + 15) / 16 + 1);
    int best = pl.split_pages;
    for (int sp : {DEC_MAX_SPLIT, 64, 32, 16, 8}) {
      if (with_prefill && sp > 64) continue;
      const int64_t items = (wpages + sp - 1) / sp;
      if (items > budget) break;  // shorter splits need even more items
      best = sp;
      if (lanes * items >= min_waves) break;
    }
    pl.split_pages = best;
  }
  // prefill: row tiles bound by the query tokens; key ranges cut so that about
  // 1024 workgroups exist when the tiles are long, never below 512 keys
  const int64_t np = num_seqs - num_decodes;
  pl.pf_tile_cap = np > 0 ? ((int64_t)(num_tokens - num_decodes) * G + PF_ROWS - 1) / PF_ROWS + np : 0;
  const int64_t tiles = pl.pf_tile_cap * hkv;
  int64_t ks = tiles > 0 ? ((int64_t)max_context_len * tiles / CB_PF_TARGET_ITEMS + PF_KEYS - 1) / PF_KEYS * PF_KEYS
                         : PF_KEYS;
  ks = ks < CB_PF_MIN_KEYS ? CB_PF_MIN_KEYS : ks;
  pl.pf_split_keys = (int32_t)(ks > PF_MAX_KEYS ? PF_MAX_KEYS : ks);
  const int64_t max_splits = (max_context_len + pl.pf_split_keys - 1) / pl.pf_split_keys;
  pl.pf_item_cap = pl.pf_tile_cap * (max_splits > 0 ? max_splits : 1);
  pl.pf_may_split = max_splits > 1;
  pl.hkv = hkv;
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  size_t off = 0;
  pl.off_hdr = off;         off = align(off + HDR_BYTES);
  pl.off_dec_items = off;   off = align(off + (size_t)pl.dec_cap * 16);
  pl.off_pf_items = off;    off = align(off + (size_t)pl.pf_item_cap * 16);
  pl.off_pf_tiles = off;    off = align(off + (size_t)pl.pf_tile_cap * 16);
  pl.off_dec_first = off;   off = align(off + (size_t)num_decodes * sizeof(int32_t));
  pl.off_dec_rem = off;     off = align(off + (size_t)num_decodes * sizeof(int32_t));
  const size_t drows = (size_t)pl.dec_cap * hkv * G;
  pl.off_dec_ml = off;      off = align(off + drows * 8);
  pl.off_dec_o = off;       off = align(off + drows * head_dim * sizeof(uint16_t));
  const size_t prows = pl.pf_may_split ? (size_t)pl.pf_item_cap * hkv * PF_ROWS : 0;
  pl.off_pf_ml = off;       off = align(off + prows * 8);
  pl.off_pf_o = off;        off = align(off + prows * head_dim * sizeof(uint16_t));
  pl.bytes = off;
  return pl;
}

hipError_t launch_attention_bf16(const AttnArgs& a, const Bf16Plan& pl, const WorkLists* lists,
                                 hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, pl, lists, stream);
  if (a.head_dim == 64) return launch_d<64>(a, pl, lists, stream);
  return hipErrorInvalidValue;
}

WorkListLayout work_list_layout(const Bf16Plan& pl, int32_t num_decodes) {
  auto align = [](size_t x) { return (x + 15) & ~size_t(15); };
  WorkListLayout L{};
  size_t off = 0;
  L.hdr = off;        off = align(off + HDR_BYTES);
  L.dec_items = off;  off = align(off + (size_t)pl.dec_cap * 16);
  L.pf_items = off;   off = align(off + (size_t)pl.pf_item_cap * 16);
  L.pf_tiles = off;   off = align(off + (size_t)pl.pf_tile_cap * 16);
  L.dec_first = off;  off = align(off + (size_t)num_decodes * 4);
  L.dec_rem = off;    off = align(off + (size_t)num_decodes * 4);
  L.bytes = off;
  return L;
}

// Mirrors plan_kernel: decode items longest first (every full split, then the
// short last splits by decreasing length, sequences in order within a
// length), prefill tiles heaviest (last) first with their key splits.
WorkCounts build_work_lists(const Bf16Plan& pl, int32_t num_seqs, int32_t num_decodes, int32_t G, int32_t window,
                      const int32_t* qsl, const int32_t* ctx, const int32_t* q_off, void* dst) {
  bool any_pf_split = false, any_dec_split = false;
  const WorkListLayout L = work_list_layout(pl, num_decodes);
  uint8_t* base = static_cast<uint8_t*>(dst);
  int4* dec = reinterpret_cast<int4*>(base + L.dec_items);
  int4* pfi = reinterpret_cast<int4*>(base + L.pf_items);
  int4* pft = reinterpret_cast<int4*>(base + L.pf_tiles);
  int32_t* first = reinterpret_cast<int32_t*>(base + L.dec_first);
  int32_t* rem_at = reinterpret_cast<int32_t*>(base + L.dec_rem);
  const int SP = pl.split_pages;
  int64_t n = 0;
  int counts[DEC_MAX_SPLIT + 1] = {0};
  for (int s = 0; s < num_decodes; ++s) {
    const int np = decode_pages(ctx[s], window);
    const int nfull = np / SP, rem = np - nfull * SP;
    any_dec_split = any_dec_split || np > SP;
    first[s] = (int32_t)n;
    for (int k = 0; k < nfull && n < pl.dec_cap; ++k) dec[n++] = make_int4(s, k, ctx[s], qsl[s]);
    if (rem > 0) counts[SP - rem]++;
  }
  int starts[DEC_MAX_SPLIT + 1];
  for (int b = 0, acc = (int)n; b <= DEC_MAX_SPLIT; ++b) { starts[b] = acc; acc += counts[b]; }
  for (int s = 0; s < num_decodes; ++s) {
    const int np = decode_pages(ctx[s], window);
    const int nfull = np / SP, rem = np - nfull * SP;
    rem_at[s] = -1;
    if (rem > 0) {
      const int idx = starts[SP - rem]++;
      rem_at[s] = idx;
      if (idx < pl.dec_cap) dec[idx] = make_int4(s, nfull, ctx[s], qsl[s]);
      n = std::max<int64_t>(n, idx + 1);
    }
  }
  for (int64_t i = n; i < pl.dec_cap; ++i) dec[i] = make_int4(-1, 0, 0, 0);
  int64_t nt = 0, ni = 0;
  std::vector<int> tns;
  for (int s = num_decodes; s < num_seqs; ++s) {
    const int Lq = qsl[s + 1] - qsl[s];
    const int ntiles = Lq > 0 ? (Lq * G + PF_ROWS - 1) / PF_ROWS : 0;
    tns.assign(ntiles, 0);
    const int64_t base = ni;
    int maxns = 0;
    for (int k = 0; k < ntiles; ++k) {  // tile records heaviest first, slots per tile
      const int t = ntiles - 1 - k;
      tns[k] = tile_splits(t, Lq, G, ctx[s], q_off[s], window, pl.pf_split_keys);
      if (nt < pl.pf_tile_cap) pft[nt] = make_int4(s, t, (int)ni, tns[k]);
      ++nt;
      ni += tns[k];
      maxns = std::max(maxns, tns[k]);
      any_pf_split = any_pf_split || tns[k] > 1;
    }
    int64_t it = base;
    for (int ks = 0; ks < maxns; ++ks) {  // items split-major
      int64_t first = base;
      for (int k = 0; k < ntiles; ++k) {
        if (ks < tns[k]) {
          if (it < pl.pf_item_cap) pfi[it] = make_int4(s, ntiles - 1 - k, ks, (int)(first + ks));
          ++it;
        }
        first += tns[k];
      }
    }
  }
  for (int64_t i = nt; i < pl.pf_tile_cap; ++i) pft[i] = make_int4(-1, 0, 0, 0);
  for (int64_t i = ni; i < pl.pf_item_cap; ++i) pfi[i] = make_int4(-1, 0, 0, 0);
  const int64_t pl_live = std::min<int64_t>(ni, pl.pf_item_cap), dl_live = std::min<int64_t>(n, pl.dec_cap);
  // CU split: prefill CUs per shader engine (of 8) in proportion to the
  // prefill part's share of the step's estimated time (MFMA work at ~0.95
  // PFLOP/s, K/V bytes at ~6 TB/s; head size and KV heads cancel out)
  int k = 0;
  if (CB_CU_SPLIT && pl_live > 0 && dl_live > 0) {
    double pairs = 0, pages = 0;
    for (int s = 0; s < num_decodes; ++s) pages += decode_pages(ctx[s], window);
    for (int s = num_decodes; s < num_seqs; ++s)
      for (int i = 0; i < qsl[s + 1] - qsl[s]; ++i) {
        const int64_t pos = (int64_t)q_off[s] + i;
        pairs += (double)(window > 0 ? std::min<int64_t>(pos + 1, window) : pos + 1);
      }
    const double t_pf = pairs * 4.0 * G / 0.95e15, t_dec = pages * 64.0 / 6.0e12;
    k = std::min(CB_CU_SPLIT_MAX, std::max(1, (int)std::lround(8.0 * t_pf / (t_pf + t_dec))));
    if (k < CB_CU_SPLIT_MIN) k = 0;  // a small prefill part: the block order above
  }
  *reinterpret_cast<int4*>(base + L.hdr) =
      make_int4((int)pl_live, (int)dl_live, mix_order(pl_live, dl_live, pl.hkv, pl.slots), k);
  std::memset(base + L.hdr + 16, 0, sizeof(UnitQueues));
  return WorkCounts{pl_live, dl_live, any_pf_split, any_dec_split, k};
}

}  // namespace cb
