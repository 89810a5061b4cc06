// fp32 attention step: a plain VALU kernel, one wavefront per query row.
//
// Ultralytics glossary, "Chunked Prefill", "How chunked prefill works": a
// query row at absolute position p attends to keys 0..p of its own sequence
// (causal over absolute positions), whether it belongs to a prefill chunk or
// is a decode token.
//
// This path serves float32 inputs, where exactness matters more than speed.
// Each wavefront owns one (token, query head) row: lanes take 64 keys at a
// time, compute their scores from the block table, keep an online softmax
// (running max and sum), and accumulate the weighted values with each lane
// owning head_dim/64 output dimensions.  Only keys 0..min(p, ctx-1) are ever
// read (from p-window+1 on with a sliding window: transformers, "Continuous
// batching architecture", Memory management), so slots outside never reach
// the arithmetic.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.h"

namespace cb {
namespace {

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  constexpr int E = D / 64;  // output dims per lane
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= (int64_t)a.num_tokens * a.hq) return;
  const int t = (int)(wave / a.hq);
  const int h = (int)(wave % a.hq);
  const int G = a.hq / a.hkv;
  const int kvh = h / G;

  // sequence owning token t: the last s with qsl[s] <= t
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int ctx = a.ctx_lens[s];
  const int pos = a.q_offsets[s] + (t - a.qsl[s]);
  const int nk = min(pos + 1, ctx);
  const int k0 = a.window > 0 ? max(0, pos - a.window + 1) : 0;

  const float* __restrict__ qrow = static_cast<const float*>(a.q) + ((size_t)t * a.hq + h) * D;
  const float* __restrict__ kc = static_cast<const float*>(a.k_cache);
  const float* __restrict__ vc = static_cast<const float*>(a.v_cache);
  const int32_t* __restrict__ bt = a.block_tables + (a.bt_offsets ? (size_t)a.bt_offsets[s] : (size_t)s * a.bt_stride);

  float qv[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const float4 x = *reinterpret_cast<const float4*>(qrow + d);
    qv[d] = x.x; qv[d + 1] = x.y; qv[d + 2] = x.z; qv[d + 3] = x.w;
  }
  float m = -INFINITY, l = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  for (int kb = k0; kb < nk; kb += 64) {
    const int j = kb + lane;
    const bool valid = j < nk;
    int page = valid ? bt[j >> 4] : 0;
    const bool pok = valid && (unsigned)page < (unsigned)a.num_pages;
    if (!pok) page = -1;
    float x = -INFINITY;
    if (valid) {
      float dot = 0.f;
      if (pok) {
        const float* kr = kc + (((size_t)page * a.hkv + kvh) * 16 + (j & 15)) * D;
#pragma unroll
        for (int d = 0; d < D; d += 4) {
          const float4 kk = *reinterpret_cast<const float4*>(kr + d);
          dot = fmaf(qv[d], kk.x, dot);
          dot = fmaf(qv[d + 1], kk.y, dot);
          dot = fmaf(qv[d + 2], kk.z, dot);
          dot = fmaf(qv[d + 3], kk.w, dot);
        }
      }
      x = dot * a.scale;
    }
    const float mnew = fmaxf(m, wave_max(x));
    const float alpha = expf(m - mnew);
    const float p = valid ? expf(x - mnew) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= alpha;
    const int nb = min(64, nk - kb);
    for (int jj = 0; jj < nb; ++jj) {
      const float pj = __shfl(p, jj);
      const int pgj = __shfl(page, jj);
      if (pgj < 0) continue;
      const float* vr = vc + ((size_t)pgj * a.hkv + kvh) * D * 16 + ((kb + jj) & 15);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(pj, vr[(lane + 64 * e) * 16], acc[e]);
    }
    m = mnew;
  }
  float* __restrict__ orow = static_cast<float*>(a.out) + ((size_t)t * a.hq + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < E; ++e) orow[lane + 64 * e] = acc[e] * inv;
}

}  // namespace

hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.num_tokens * a.hq;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (a.head_dim != 128 && a.head_dim != 64) return hipErrorInvalidValue;
  if (g_prof_start) (void)hipEventRecord(g_prof_start, stream);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, stream, a);
  if (g_prof_stop) (void)hipEventRecord(g_prof_stop, stream);
  return hipGetLastError();
}

}  // namespace cb
