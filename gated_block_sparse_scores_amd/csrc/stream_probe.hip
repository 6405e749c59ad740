// Read floor of cold HBM streams at the decode's sizes (measurement only, not
// part of the library): a plain read kernel, 16-byte loads over a grid-stride
// loop (one or four loads in flight per thread), one partial per workgroup,
// over buffers rotated through at least 1 GiB (four times the last-level
// cache), so that every launch reads from HBM.  Back-to-back launches are
// timed with HIP events; one JSON line per (bytes, grid, loads in flight).
//
//   stream_probe [bytes ...]   (default: 8388608 16760832 134217728, the
//                               selected K/V of the 512K decode, one layer's
//                               pooled keys, the selected K/V of 8 x 64K)
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define PROBE_CHECK(x)                                                                \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      std::fprintf(stderr, "stream_probe: %s at line %d\n", hipGetErrorString(e_), \
                   __LINE__);                                                         \
      std::exit(1);                                                                   \
    }                                                                                 \
  } while (0)

template <int U>
__global__ void __launch_bounds__(256) read_kernel(const uint4* __restrict__ p, size_t n16,
                                                   uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int j = 0; j < 256; ++j) a ^= red[j];
    out[blockIdx.x] = a;
  }
}

int main(int argc, char** argv) {
  std::vector<size_t> sizes;
  for (int a = 1; a < argc; ++a) sizes.push_back(std::strtoull(argv[a], nullptr, 10));
  if (sizes.empty()) sizes = {8388608ull, 16760832ull, 134217728ull};
  const int grids[] = {256, 512, 1024, 2048, 4096};
  const int reps = 256;
  uint32_t* out = nullptr;
  PROBE_CHECK(hipMalloc(&out, 4096 * sizeof(uint32_t)));
  hipEvent_t e0, e1;
  PROBE_CHECK(hipEventCreate(&e0));
  PROBE_CHECK(hipEventCreate(&e1));
  for (const size_t bytes : sizes) {
    if (bytes < 16 || bytes % 16 != 0) {
      std::fprintf(stderr, "stream_probe: %zu is not a positive multiple of 16\n", bytes);
      return 2;
    }
    const size_t rotate = (size_t)1 << 30;
    const size_t want = (rotate + bytes - 1) / bytes;
    const int nbuf = want < 2 ? 2 : (int)want;
    std::vector<void*> bufs(nbuf);
    for (int i = 0; i < nbuf; ++i) {
      PROBE_CHECK(hipMalloc(&bufs[i], bytes));
      PROBE_CHECK(hipMemset(bufs[i], i & 0xFF, bytes));
    }
    PROBE_CHECK(hipDeviceSynchronize());
    for (const int g : grids) {
      for (const int u : {1, 4}) {
        float ms = 0.0f;
        for (int pass = 0; pass < 2; ++pass) {  // the first pass warms up
          PROBE_CHECK(hipEventRecord(e0));
          for (int r = 0; r < reps; ++r) {
            const uint4* p = (const uint4*)bufs[r % nbuf];
            if (u == 1)
              hipLaunchKernelGGL(read_kernel<1>, dim3(g), dim3(256), 0, 0, p, bytes / 16, out);
            else
              hipLaunchKernelGGL(read_kernel<4>, dim3(g), dim3(256), 0, 0, p, bytes / 16, out);
          }
          PROBE_CHECK(hipGetLastError());
          PROBE_CHECK(hipEventRecord(e1));
          PROBE_CHECK(hipEventSynchronize(e1));
          PROBE_CHECK(hipEventElapsedTime(&ms, e0, e1));
        }
        const double us = ms * 1e3 / reps;
        std::printf(
            "{\"bytes\": %zu, \"grid\": %d, \"loads_in_flight\": %d, \"buffers\": %d, "
            "\"us_per_launch\": %.2f, \"GBps\": %.1f}\n",
            bytes, g, u, nbuf, us, bytes / (us * 1e3));
        std::fflush(stdout);
      }
    }
    for (void* b : bufs) PROBE_CHECK(hipFree(b));
  }
  PROBE_CHECK(hipFree(out));
  return 0;
}
