// HBM probe: the achievable streaming bandwidth of this GPU, and a copy
// kernel of known size for scaling the FETCH_SIZE / WRITE_SIZE counters.
//
//   hbm_probe read  <bytes> <iters>   each launch reads <bytes> once (16-byte loads)
//   hbm_probe copy  <bytes> <iters>   each launch reads and writes <bytes>
//
// Prints one line per mode: bytes per launch, average launch time (HIP
// events) and GB/s.  Not part of the library; a measurement aid.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, size_t n, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x12345678u) sink[0] = acc;  // keeps the loads alive; practically never stores
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

int main(int argc, char** argv) {
  const char* mode = argc > 1 ? argv[1] : "read";
  const size_t bytes = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : (size_t(1) << 30);
  const int iters = argc > 3 ? std::atoi(argv[3]) : 20;
  const size_t n = bytes / 16;
  uint4 *src = nullptr, *dst = nullptr;
  uint32_t* sink = nullptr;
  CHECK(hipMalloc(&src, n * 16));
  CHECK(hipMemset(src, 1, n * 16));
  CHECK(hipMalloc(&sink, 4));
  const bool copy = std::strcmp(mode, "copy") == 0;
  if (copy) CHECK(hipMalloc(&dst, n * 16));
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  const dim3 grid((unsigned)(cus * 16)), block(256);
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  for (int w = 0; w < 2; ++w) {
    if (copy) hipLaunchKernelGGL(copy_kernel, grid, block, 0, 0, src, dst, n);
    else hipLaunchKernelGGL(read_kernel, grid, block, 0, 0, src, n, sink);
  }
  CHECK(hipDeviceSynchronize());
  float total = 0.f;
  for (int it = 0; it < iters; ++it) {
    CHECK(hipEventRecord(a, 0));
    if (copy) hipLaunchKernelGGL(copy_kernel, grid, block, 0, 0, src, dst, n);
    else hipLaunchKernelGGL(read_kernel, grid, block, 0, 0, src, n, sink);
    CHECK(hipEventRecord(b, 0));
    CHECK(hipEventSynchronize(b));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, a, b));
    total += ms;
  }
  CHECK(hipGetLastError());
  const double avg_s = total / iters / 1e3;
  const double moved = copy ? 2.0 * n * 16 : 1.0 * n * 16;
  std::printf("{\"mode\": \"%s\", \"bytes_per_launch\": %.0f, \"avg_us\": %.2f, \"GBps\": %.1f, \"cus\": %d}\n", mode,
              moved, avg_s * 1e6, moved / avg_s / 1e9, cus);
  return 0;
}
