// KV append: copy this step's K/V rows into their cache slots, bit for bit.
//
// Ultralytics glossary, "Chunked Prefill", "How chunked prefill works": a
// chunk's own keys and values are cached before it attends, and later chunks
// read them from the cache.  AI Engineering from Scratch, "vLLM serving
// internals", "PagedAttention as virtual memory": slots live in fixed
// 16-token blocks.
//
// One workgroup handles 16 consecutive tokens of one KV head.  K rows are
// token-major in the page, so each row is a straight 16-byte-vector copy.  V
// is token-minor in the page ([D][16] per slab), so the 16 rows are staged in
// LDS and written back transposed: consecutive lanes write consecutive
// tokens of one dimension, which are adjacent bytes when the tokens share a
// page.  No arithmetic touches the values (integer loads and stores only).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels.h"

namespace cb {
namespace {

// Optional second job of the same launch: blocks past the append grid copy
// `pull_n16` 16-byte chunks from `pull_src` (the engine's pinned staging
// slot, mapped into the device's address space) to `pull_dst` (the device
// metadata slot).  The step's metadata then reaches the device inside the
// kernel that starts the step, with no separate copy in the stream.
struct Pull {
  const uint4* src;
  uint4* dst;
  int64_t n16;
  int32_t append_blocks;
};

template <int D, int ES>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint8_t* __restrict__ k_new,
                                                        const uint8_t* __restrict__ v_new,
                                                        uint8_t* __restrict__ k_cache,
                                                        uint8_t* __restrict__ v_cache,
                                                        const int32_t* __restrict__ slots,
                                                        int32_t num_tokens, int32_t hkv,
                                                        int32_t num_pages, Pull pull) {
  if ((int)blockIdx.x >= pull.append_blocks) {
    const int64_t nb = (int64_t)gridDim.x - pull.append_blocks;
    for (int64_t i = ((int64_t)blockIdx.x - pull.append_blocks) * 256 + threadIdx.x; i < pull.n16; i += nb * 256)
      pull.dst[i] = pull.src[i];
    return;
  }
  constexpr int ROWB = D * ES;        // bytes of one token row of one head
  constexpr int CH = ROWB / 16;       // 16-byte chunks per row
  constexpr int LROW = ROWB + 16;     // padded LDS row (spreads the column reads over banks)
  constexpr int NE = (16 * CH + 255) / 256;  // row chunks per thread
  __shared__ __attribute__((aligned(16))) uint8_t vbuf[16 * LROW];
  __shared__ int32_t sslot[16];       // the group's slots (-1: not written)

  const int tid = threadIdx.x;
  const int h = blockIdx.x % hkv;
  const int t0 = (blockIdx.x / hkv) * 16;
  const int64_t slot_limit = (int64_t)num_pages * 16;

  // The slot mapping may live in mapped host memory (the engine's staging
  // slot): it is read once per group, here, and shared through LDS.
  if (tid < 16) {
    const int t = t0 + tid;
    int32_t sl = t < num_tokens ? slots[t] : -1;
    sslot[tid] = (sl >= 0 && sl < slot_limit) ? sl : -1;
  }
  uint4 kreg[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = tid + 256 * i;
    kreg[i] = make_uint4(0, 0, 0, 0);
    if (e < 16 * CH) {
      const int r = e / CH, c = e % CH;
      const int t = t0 + r;
      uint4 vv = make_uint4(0, 0, 0, 0);
      if (t < num_tokens) {
        const size_t src = ((size_t)t * hkv + h) * ROWB + c * 16;
        vv = *reinterpret_cast<const uint4*>(v_new + src);
        kreg[i] = *reinterpret_cast<const uint4*>(k_new + src);
      }
      *reinterpret_cast<uint4*>(vbuf + r * LROW + c * 16) = vv;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = tid + 256 * i;
    if (e < 16 * CH) {
      const int r = e / CH, c = e % CH;
      const int32_t slot = sslot[r];
      if (slot >= 0) {
        const size_t dst = (((size_t)(slot >> 4) * hkv + h) * 16 + (slot & 15)) * ROWB + c * 16;
        *reinterpret_cast<uint4*>(k_cache + dst) = kreg[i];
      }
    }
  }
  for (int e = tid; e < 16 * D; e += 256) {
    const int r = e & 15, d = e >> 4;
    const int32_t slot = sslot[r];
    if (slot < 0) continue;
    const size_t dst = ((((size_t)(slot >> 4) * hkv + h) * D + d) * 16 + (slot & 15)) * ES;
    if constexpr (ES == 2) {
      *reinterpret_cast<uint16_t*>(v_cache + dst) = *reinterpret_cast<const uint16_t*>(vbuf + r * LROW + d * 2);
    } else {
      *reinterpret_cast<uint32_t*>(v_cache + dst) = *reinterpret_cast<const uint32_t*>(vbuf + r * LROW + d * 4);
    }
  }
}

template <int D, int ES>
hipError_t launch(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const int32_t* slots,
                  int32_t T, int32_t hkv, int32_t num_pages, Pull pull, hipStream_t stream) {
  const int64_t groups = (T + 15) / 16;
  pull.append_blocks = (int32_t)(groups * hkv);
  const int64_t pull_blocks = pull.n16 > 0 ? std::min<int64_t>((pull.n16 + 255) / 256, 64) : 0;
  const dim3 grid((unsigned)(groups * hkv + pull_blocks));
  if (grid.x == 0) return hipSuccess;
  hipLaunchKernelGGL((kv_append_kernel<D, ES>), grid, dim3(256), 0, stream,
                     static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new),
                     static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), slots, T, hkv, num_pages,
                     pull);
  return hipGetLastError();
}

hipError_t dispatch(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const int32_t* slots,
                    int32_t T, int32_t hkv, int32_t head_dim, int32_t num_pages, int32_t elem_bytes, Pull pull,
                    hipStream_t stream) {
  if (head_dim == 128 && elem_bytes == 2) return launch<128, 2>(k_new, v_new, k_cache, v_cache, slots, T, hkv, num_pages, pull, stream);
  if (head_dim == 64 && elem_bytes == 2) return launch<64, 2>(k_new, v_new, k_cache, v_cache, slots, T, hkv, num_pages, pull, stream);
  if (head_dim == 128 && elem_bytes == 4) return launch<128, 4>(k_new, v_new, k_cache, v_cache, slots, T, hkv, num_pages, pull, stream);
  if (head_dim == 64 && elem_bytes == 4) return launch<64, 4>(k_new, v_new, k_cache, v_cache, slots, T, hkv, num_pages, pull, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* slots, int32_t T, int32_t hkv, int32_t head_dim,
                            int32_t num_pages, int32_t elem_bytes, hipStream_t stream) {
  return dispatch(k_new, v_new, k_cache, v_cache, slots, T, hkv, head_dim, num_pages, elem_bytes,
                  Pull{nullptr, nullptr, 0, 0}, stream);
}

hipError_t launch_kv_append_pull(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 const int32_t* slots, int32_t T, int32_t hkv, int32_t head_dim,
                                 int32_t num_pages, int32_t elem_bytes, const void* pull_src, void* pull_dst,
                                 int64_t pull_bytes, hipStream_t stream) {
  return dispatch(k_new, v_new, k_cache, v_cache, slots, T, hkv, head_dim, num_pages, elem_bytes,
                  Pull{static_cast<const uint4*>(pull_src), static_cast<uint4*>(pull_dst), pull_bytes / 16, 0},
                  stream);
}

}  // namespace cb
