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
//    list).  It streams its pages straight from HBM into registers (one
//    16-token page of K and of V per iteration, the next page's loads in
//    flight), scores the G query heads that share the KV head with one
//    16x16x32 bf16 MFMA per 32 dims (keys as rows, heads as columns), keeps
//    an online softmax per head, and accumulates P V with 16x16x16 bf16
//    MFMAs.  Partial (max, sum, O) go to the workspace when the sequence has
//    more than one split; a combine kernel merges them by log-sum-exp.
//  * prefill item = one 256-thread workgroup on (sequence, KV head, tile of
//    128 query rows), where a row is a (query token, query head of the
//    group) pair so the G heads sharing a KV head read K/V once.  Per
//    64-key tile the workgroup stages K and V pages in LDS; each wavefront
//    computes S^T = K Q^T for its 32 rows with 32x32x16 bf16 MFMAs, applies
//    the causal mask only on tiles that straddle its diagonal, updates the
//    online softmax and accumulates O^T = V^T P^T.  Tiles wholly above the
//    diagonal are never loaded.
//
// Layouts: K pages are token-major ([16][D] per (page, head)), so a lane's
// MFMA A-operand (one key, 8 consecutive dims) is one 16-byte load.  V pages
// are token-minor ([D][16]), so the A-operand of O^T = V^T P^T (one dim, 4 or
// 8 consecutive keys) is one or two 8-byte loads, and the B-operand P^T comes
// straight from the score accumulator registers without any shuffle.
//
// Numerics: bf16 inputs, fp32 MFMA accumulation, softmax in fp32 on the
// base-2 scale (scores multiplied by scale*log2(e)), probabilities rounded to
// bf16 for the P V product, output rounded to bf16 (round to nearest even).
// Cache slots at or past the context length are masked by select and their V
// entries zeroed, so garbage or NaN there never reaches the output.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.h"

namespace cb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int PF_ROWS = 128;  // query rows per prefill workgroup (4 waves x 32)
constexpr int PF_KEYS = 64;   // keys per prefill tile (4 pages)
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
  int32_t* counts;      // [0] decode items, [1] prefill items
  int32_t* dec_first;   // [num_decodes] first decode item of each sequence
  int2* dec_items;      // (sequence, split)
  int2* pf_items;       // (sequence, row tile)
  float2* part_ml;      // [decode wave][G] (running max in log2 units, sum)
  float* part_o;        // [decode wave][G][D] unnormalised
  int32_t bt_stride;
  int32_t num_seqs, num_decodes;
  int32_t hq, hkv, G;
  int32_t num_pages;
  int32_t split_pages;
  int32_t pf_blocks;    // grid blocks reserved for prefill items
  int32_t dec_cap, pf_cap;
  float scale_log2;     // softmax scale * log2(e)
};

template <int D>
struct PfLds {
  static constexpr int KROW = D * 2 + 16;  // padded K row (bytes) in LDS
  static constexpr int VROW = 40;          // padded (page, dim) row of 16 tokens (bytes)
  static constexpr int K_BYTES = PF_KEYS * KROW;
  static constexpr int V_BYTES = (PF_KEYS / 16) * D * VROW;
  static constexpr int BYTES = K_BYTES + V_BYTES;
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ short4v as_short4(uint2 v) { return __builtin_bit_cast(short4v, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// keep the first n (0..2*words) 16-bit elements of a little-endian word
__device__ __forceinline__ uint32_t keep16(uint32_t w, int first_elem, int n) {
  return (first_elem + 1 < n) ? w : (first_elem < n ? (w & 0xFFFFu) : 0u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Plan: one workgroup turns the per-sequence lengths (device data) into
// compact work lists, so the main grid needs only host-side upper bounds.
// ---------------------------------------------------------------------------
__device__ int block_exclusive_scan(int v, int* sh, int& total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  total = sh[1023];
  const int incl = sh[tid];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(1024) void plan_kernel(Params p) {
  __shared__ int sh[1024];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < p.num_decodes; base += 1024) {
    const int s = base + tid;
    int n = 0;
    if (s < p.num_decodes) {
      const int ctx = p.ctx_lens[s];
      const int np = (ctx + 15) >> 4;
      n = ctx > 0 ? (np + p.split_pages - 1) / p.split_pages : 0;
    }
    int total;
    const int ex = block_exclusive_scan(n, sh, total) + carry;
    if (s < p.num_decodes) p.dec_first[s] = ex;
    for (int k = 0; k < n && ex + k < p.dec_cap; ++k) p.dec_items[ex + k] = make_int2(s, k);
    carry += total;
  }
  const int dec_total = min(carry, p.dec_cap);
  carry = 0;
  for (int base = p.num_decodes; base < p.num_seqs; base += 1024) {
    const int s = base + tid;
    int n = 0;
    if (s < p.num_seqs) {
      const int L = p.qsl[s + 1] - p.qsl[s];
      n = L > 0 ? (L * p.G + PF_ROWS - 1) / PF_ROWS : 0;
    }
    int total;
    const int ex = block_exclusive_scan(n, sh, total) + carry;
    // longest-running tiles (last rows see the most keys) first
    for (int k = 0; k < n && ex + k < p.pf_cap; ++k) p.pf_items[ex + k] = make_int2(s, n - 1 - k);
    carry += total;
  }
  if (tid == 0) {
    p.counts[0] = dec_total;
    p.counts[1] = min(carry, p.pf_cap);
  }
}

// ---------------------------------------------------------------------------
// Decode: one wavefront per (sequence, KV head, split).
// ---------------------------------------------------------------------------
template <int D>
struct DecodeBuf {
  uint4 k[D / 32];  // this lane's slice of one K page (one key, D/4 dims)
  uint2 v[D / 16];  // this lane's slice of one V page (4 keys for each of D/16 dims)
};

template <int D>
__device__ __forceinline__ void decode_load(DecodeBuf<D>& B, const Params& p, const int32_t* btrow,
                                            int pg, int kvh, int hl, int g) {
  constexpr int DQ = D / 4;
  const int phys = btrow[pg];
  const bool ok = (unsigned)phys < (unsigned)p.num_pages;
  const size_t slab = (size_t)(ok ? phys : 0) * p.hkv + kvh;
  const uint16_t* kb = p.k_cache + slab * 16 * D + hl * D + g * DQ;
  const uint16_t* vb = p.v_cache + slab * D * 16 + hl * 16 + g * 4;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    B.k[c] = ok ? *reinterpret_cast<const uint4*>(kb + 8 * c) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    B.v[t] = ok ? *reinterpret_cast<const uint2*>(vb + t * 256) : make_uint2(0, 0);
}

template <int D>
__device__ __forceinline__ void decode_compute(const DecodeBuf<D>& B, int pg, int ctx, int g,
                                               const bf16x8 (&qf)[D / 32], floatx4 (&o)[D / 16],
                                               float& m, float& l, float scale_log2) {
  floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(B.k[c]), qf[c], sacc, 0, 0, 0);
  // lane holds S^T[key 4g + r][head lane % 16]
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = sacc[r] * scale_log2;
  uint2 vv[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) vv[t] = B.v[t];
  const int key0 = pg * 16 + 4 * g;
  if (pg * 16 + 16 > ctx) {  // the page that holds the context end
    const int n = ctx - key0;  // valid keys among this lane's 4
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (r < n) ? x[r] : -INFINITY;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      vv[t].x = keep16(vv[t].x, 0, n);
      vv[t].y = keep16(vv[t].y, 2, n);
    }
  }
  float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mnew = fmaxf(m, mx);
  const float alpha = fast_exp2(m - mnew);
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(x[r] - mnew);
  l = l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
  const uint2 pk = make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    o[t] *= alpha;
    o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_short4(vv[t]), as_short4(pk), o[t], 0, 0, 0);
  }
  m = mnew;
}

template <int D>
__device__ __forceinline__ void decode_wave(const Params& p, int w) {
  const int kvh = w % p.hkv;
  const int j = w / p.hkv;
  if (j >= p.counts[0]) return;
  const int2 item = p.dec_items[j];
  const int s = item.x, split = item.y;
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15, g = lane >> 4;
  const int G = p.G;
  const int ctx = p.ctx_lens[s];
  const int npages = (ctx + 15) >> 4;
  const int pg0 = split * p.split_pages;
  const int pg1 = min(pg0 + p.split_pages, npages);
  const int nsplit = (npages + p.split_pages - 1) / p.split_pages;
  const int t = p.qsl[s];
  constexpr int DQ = D / 4;

  bf16x8 qf[D / 32];
  {
    const uint16_t* qrow = p.q + ((size_t)t * p.hq + kvh * G + hl) * D + g * DQ;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      qf[c] = as_bf16x8(hl < G ? *reinterpret_cast<const uint4*>(qrow + 8 * c) : make_uint4(0, 0, 0, 0));
  }
  floatx4 o[D / 16];
#pragma unroll
  for (int tt = 0; tt < D / 16; ++tt) o[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const int32_t* btrow = p.bt + (size_t)s * p.bt_stride;

  DecodeBuf<D> b0, b1;
  int pg = pg0;
  if (pg < pg1) decode_load<D>(b0, p, btrow, pg, kvh, hl, g);
  for (; pg + 1 < pg1; pg += 2) {
    decode_load<D>(b1, p, btrow, pg + 1, kvh, hl, g);
    decode_compute<D>(b0, pg, ctx, g, qf, o, m, l, p.scale_log2);
    if (pg + 2 < pg1) decode_load<D>(b0, p, btrow, pg + 2, kvh, hl, g);
    decode_compute<D>(b1, pg + 1, ctx, g, qf, o, m, l, p.scale_log2);
  }
  if (pg < pg1) decode_compute<D>(b0, pg, ctx, g, qf, o, m, l, p.scale_log2);

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
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
    float* po = p.part_o + prow * D;
#pragma unroll
    for (int tt = 0; tt < D / 16; ++tt) *reinterpret_cast<floatx4*>(po + 16 * tt + 4 * g) = o[tt];
    if (g == 0) p.part_ml[prow] = make_float2(m, l);
  }
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup per (sequence, KV head, 128-row tile).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void prefill_tile(const Params& p, int b, uint8_t* smem) {
  using Lds = PfLds<D>;
  const int kvh = b % p.hkv;
  const int j = b / p.hkv;
  if (j >= p.counts[1]) return;  // uniform over the workgroup
  const int2 item = p.pf_items[j];
  const int s = item.x, tile = item.y;
  const int G = p.G;
  const int t0 = p.qsl[s];
  const int L = p.qsl[s + 1] - t0;
  const int ctx = p.ctx_lens[s];
  const int off = p.q_off[s];
  const int npages = (ctx + 15) >> 4;
  const int R = L * G;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, gg = lane >> 5;

  const int row = tile * PF_ROWS + wv * 32 + l32;
  const bool rvalid = row < R;
  const int qi = row / G;
  const int hh = row - qi * G;
  const int kcap = min(off + qi, ctx - 1);  // last key this row may see

  const int wg_last_row = min(tile * PF_ROWS + PF_ROWS, R) - 1;
  const int wg_kend = min(ctx, off + wg_last_row / G + 1);
  const int w_first_row = tile * PF_ROWS + wv * 32;
  const int w_last_row = min(w_first_row + 31, R - 1);
  const int w_kend = (w_first_row < R) ? min(ctx, off + w_last_row / G + 1) : 0;
  const int w_kfull = min(ctx, off + w_first_row / G + 1);  // keys below are visible to every row

  constexpr int NK = D / 16;  // QK k-steps of 16 dims
  constexpr int NO = D / 32;  // 32-dim output tiles
  bf16x8 qf[NK];
  {
    const uint16_t* qrow = p.q + ((size_t)(t0 + qi) * p.hq + kvh * G + hh) * D + 8 * gg;
#pragma unroll
    for (int c = 0; c < NK; ++c)
      qf[c] = as_bf16x8(rvalid ? *reinterpret_cast<const uint4*>(qrow + 16 * c) : make_uint4(0, 0, 0, 0));
  }
  floatx16 o[NO];
#pragma unroll
  for (int dt = 0; dt < NO; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int32_t* btrow = p.bt + (size_t)s * p.bt_stride;
  uint8_t* kl = smem;
  uint8_t* vl = smem + Lds::K_BYTES;
  const int ntiles = (wg_kend + PF_KEYS - 1) / PF_KEYS;

  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    // stage K: 4 pages x 16 rows x D bf16, 16-byte chunks
    for (int e = tid; e < 8 * D; e += 256) {
      const int pgl = e / (2 * D), rem = e % (2 * D);
      const int r = rem / (D / 8), c16 = rem % (D / 8);
      const int pg = kt * 4 + pgl;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (pg < npages) {
        const int phys = btrow[pg];
        if ((unsigned)phys < (unsigned)p.num_pages)
          val = *reinterpret_cast<const uint4*>(p.k_cache + (((size_t)phys * p.hkv + kvh) * 16 + r) * D + c16 * 8);
      }
      *reinterpret_cast<uint4*>(kl + (pgl * 16 + r) * Lds::KROW + c16 * 16) = val;
    }
    // stage V: 4 pages x D rows x 16 tokens, 16-byte chunks (8 tokens)
    for (int e = tid; e < 8 * D; e += 256) {
      const int pgl = e / (2 * D), rem = e % (2 * D);
      const int dr = rem >> 1, hf = rem & 1;
      const int pg = kt * 4 + pgl;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (pg < npages) {
        const int phys = btrow[pg];
        if ((unsigned)phys < (unsigned)p.num_pages) {
          val = *reinterpret_cast<const uint4*>(p.v_cache + (((size_t)phys * p.hkv + kvh) * D + dr) * 16 + hf * 8);
          const int n = ctx - (pg * 16 + hf * 8);  // valid tokens among these 8
          if (n < 8) {
            val.x = keep16(val.x, 0, n);
            val.y = keep16(val.y, 2, n);
            val.z = keep16(val.z, 4, n);
            val.w = keep16(val.w, 6, n);
          }
        }
      }
      uint8_t* dst = vl + (pgl * D + dr) * Lds::VROW + hf * 16;
      *reinterpret_cast<uint2*>(dst) = make_uint2(val.x, val.y);
      *reinterpret_cast<uint2*>(dst + 8) = make_uint2(val.z, val.w);
    }
    __syncthreads();
    const int kbase = kt * PF_KEYS;
    if (kbase >= w_kend) continue;

    // S^T = K Q^T for two 32-key subtiles: lane holds S^T[key 8(r/4)+4gg+r%4][row l32]
    floatx16 st[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[sub][r] = 0.f;
#pragma unroll
      for (int c = 0; c < NK; ++c) {
        const uint4 ka = *reinterpret_cast<const uint4*>(kl + (sub * 32 + l32) * Lds::KROW + (16 * c + 8 * gg) * 2);
        st[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), qf[c], st[sub], 0, 0, 0);
      }
    }
    const bool full = kbase + PF_KEYS <= w_kfull;
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = st[sub][r] * p.scale_log2;
        if (!full) {
          const int key = kbase + sub * 32 + 8 * (r >> 2) + 4 * gg + (r & 3);
          x = key <= kcap ? x : -INFINITY;
        }
        st[sub][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mnew);
    float rs = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(st[sub][r] - mnew);
        st[sub][r] = pv;
        rs += pv;
      }
    l = l * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < NO; ++dt) o[dt] *= alpha;
    m = mnew;

    // O^T += V^T P^T, four 16-key steps (page 2*sub + half of the tile)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r0 = 8 * half;
        const uint4 pb = make_uint4(pack_bf16x2(st[sub][r0 + 0], st[sub][r0 + 1]),
                                    pack_bf16x2(st[sub][r0 + 2], st[sub][r0 + 3]),
                                    pack_bf16x2(st[sub][r0 + 4], st[sub][r0 + 5]),
                                    pack_bf16x2(st[sub][r0 + 6], st[sub][r0 + 7]));
        const uint8_t* vpage = vl + (2 * sub + half) * D * Lds::VROW;
#pragma unroll
        for (int dt = 0; dt < NO; ++dt) {
          const uint8_t* vr = vpage + (32 * dt + l32) * Lds::VROW;
          const uint2 a0 = *reinterpret_cast<const uint2*>(vr + 8 * gg);
          const uint2 a1 = *reinterpret_cast<const uint2*>(vr + 16 + 8 * gg);
          const uint4 va = make_uint4(a0.x, a0.y, a1.x, a1.y);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb), o[dt], 0, 0, 0);
        }
      }
  }

  l += __shfl_xor(l, 32);
  if (!rvalid) return;
  const float inv = 1.f / l;
  uint16_t* orow = p.out + ((size_t)(t0 + qi) * p.hq + kvh * G + hh) * D;
#pragma unroll
  for (int dt = 0; dt < NO; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint2 v = make_uint2(pack_bf16x2(o[dt][4 * q4 + 0] * inv, o[dt][4 * q4 + 1] * inv),
                                 pack_bf16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv));
      *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * q4 + 4 * gg) = v;
    }
}

// ---------------------------------------------------------------------------
// The ragged launch: blocks [0, pf_blocks) are prefill tiles, the rest carry
// four decode wavefronts each.  The no-prefill instantiation needs neither
// LDS nor the prefill registers and runs at higher occupancy.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void attn_mixed_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[PfLds<D>::BYTES];
  if ((int)blockIdx.x < p.pf_blocks) {
    prefill_tile<D>(p, blockIdx.x, smem);
    return;
  }
  decode_wave<D>(p, ((int)blockIdx.x - p.pf_blocks) * 4 + (threadIdx.x >> 6));
}

template <int D>
__global__ __launch_bounds__(256, 3) void attn_decode_kernel(Params p) {
  decode_wave<D>(p, (int)blockIdx.x * 4 + (threadIdx.x >> 6));
}

// ---------------------------------------------------------------------------
// Split-K combine: one wavefront per (decode sequence, query head).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(Params p) {
  constexpr int E = D / 64;
  const int wave = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= p.num_decodes * p.hq) return;
  const int lane = threadIdx.x & 63;
  const int s = wave / p.hq, h = wave % p.hq;
  const int G = p.G, kvh = h / G, hl = h % G;
  const int ctx = p.ctx_lens[s];
  const int npages = (ctx + 15) >> 4;
  const int nsplit = (npages + p.split_pages - 1) / p.split_pages;
  if (nsplit <= 1) return;
  const int j0 = p.dec_first[s];
  if (j0 + nsplit > p.counts[0]) return;  // work list overflowed (precondition broken)
  float M = -INFINITY;
  for (int i = lane; i < nsplit; i += 64)
    M = fmaxf(M, p.part_ml[((size_t)(j0 + i) * p.hkv + kvh) * G + hl].x);
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float acc[E], lsum = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int i = 0; i < nsplit; ++i) {
    const size_t prow = ((size_t)(j0 + i) * p.hkv + kvh) * G + hl;
    const float2 ml = p.part_ml[prow];
    const float wgt = fast_exp2(ml.x - M);
    lsum = fmaf(wgt, ml.y, lsum);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(wgt, p.part_o[prow * D + lane + 64 * e], acc[e]);
  }
  const float inv = 1.f / lsum;
  uint16_t* orow = p.out + ((size_t)p.qsl[s] * p.hq + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const __bf16 v = (__bf16)(acc[e] * inv);
    orow[lane + 64 * e] = __builtin_bit_cast(uint16_t, v);
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const Bf16Plan& pl, hipStream_t stream) {
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
  p.counts = reinterpret_cast<int32_t*>(ws + pl.off_counts);
  p.dec_first = reinterpret_cast<int32_t*>(ws + pl.off_dec_first);
  p.dec_items = reinterpret_cast<int2*>(ws + pl.off_dec_items);
  p.pf_items = reinterpret_cast<int2*>(ws + pl.off_pf_items);
  p.part_ml = reinterpret_cast<float2*>(ws + pl.off_part_ml);
  p.part_o = reinterpret_cast<float*>(ws + pl.off_part_o);
  p.bt_stride = a.bt_stride;
  p.num_seqs = a.num_seqs;
  p.num_decodes = a.num_decodes;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.G = a.hq / a.hkv;
  p.num_pages = a.num_pages;
  p.split_pages = pl.split_pages;
  p.dec_cap = (int32_t)pl.dec_cap;
  p.pf_cap = (int32_t)pl.pf_cap;
  p.scale_log2 = a.scale * LOG2E;
  const int64_t pf_blocks = (a.num_seqs > a.num_decodes) ? pl.pf_cap * a.hkv : 0;
  const int64_t dec_blocks = (pl.dec_cap * a.hkv + 3) / 4;
  p.pf_blocks = (int32_t)pf_blocks;

  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, p);
  if (g_prof_start) (void)hipEventRecord(g_prof_start, stream);
  if (pf_blocks > 0) {
    hipLaunchKernelGGL(attn_mixed_kernel<D>, dim3((unsigned)(pf_blocks + dec_blocks)), dim3(256), 0, stream, p);
  } else if (dec_blocks > 0) {
    hipLaunchKernelGGL(attn_decode_kernel<D>, dim3((unsigned)dec_blocks), dim3(256), 0, stream, p);
  }
  if (g_prof_stop) (void)hipEventRecord(g_prof_stop, stream);
  if (a.num_decodes > 0 && (int64_t)pl.split_pages * 16 < a.max_context_len) {
    const int64_t waves = (int64_t)a.num_decodes * a.hq;
    hipLaunchKernelGGL(combine_kernel<D>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

Bf16Plan plan_bf16(int32_t num_seqs, int32_t num_decodes, int32_t num_tokens, int32_t hq, int32_t hkv,
                   int32_t head_dim, int32_t max_context_len) {
  Bf16Plan pl{};
  const int64_t max_pages = (max_context_len + 15) / 16;
  const int64_t lanes = (int64_t)num_decodes * hkv;
  pl.split_pages = 8;
  for (int sp : {64, 32, 16}) {
    if (lanes * ((max_pages + sp - 1) / sp) >= 16384) { pl.split_pages = sp; break; }
  }
  const int64_t G = hkv > 0 ? hq / hkv : 1;
  pl.dec_cap = (int64_t)num_decodes * ((max_pages + pl.split_pages - 1) / pl.split_pages);
  const int64_t np = num_seqs - num_decodes;
  pl.pf_cap = np > 0 ? ((int64_t)(num_tokens - num_decodes) * G + PF_ROWS - 1) / PF_ROWS + np : 0;
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  size_t off = 0;
  pl.off_counts = off;      off = align(off + 2 * sizeof(int32_t));
  pl.off_dec_first = off;   off = align(off + (size_t)num_decodes * sizeof(int32_t));
  pl.off_dec_items = off;   off = align(off + (size_t)pl.dec_cap * 8);
  pl.off_pf_items = off;    off = align(off + (size_t)pl.pf_cap * 8);
  const size_t nrows = (size_t)pl.dec_cap * hkv * G;
  pl.off_part_ml = off;     off = align(off + nrows * 8);
  pl.off_part_o = off;      off = align(off + nrows * head_dim * sizeof(float));
  pl.bytes = off;
  return pl;
}

hipError_t launch_attention_bf16(const AttnArgs& a, const Bf16Plan& pl, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, pl, stream);
  if (a.head_dim == 64) return launch_d<64>(a, pl, stream);
  return hipErrorInvalidValue;
}

}  // namespace cb
