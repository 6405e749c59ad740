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
//   stream_probe --gather      the 8 x 64K decode's access pattern without its
//                               arithmetic: K and V caches [8, 8, 65536, 128]
//                               bf16 (1 GiB each), every (batch, KV head) row
//                               reading 64 distinct 16 KiB blocks of K and the
//                               same blocks of V, two blocks per workgroup of
//                               256 threads, all loads issued before the first
//                               use; each launch draws a fresh ascending block
//                               set per row ("random"), or takes 64 adjacent
//                               blocks at a rotating offset ("adjacent").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
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

constexpr int kRows = 64;             // batch 8 x 8 KV heads
constexpr int kBlocksPerRow = 1024;   // 65536 keys / 64
constexpr int kSel = 64;              // selected blocks per row (Top-63 + the current one)
constexpr size_t kBlockU4 = 64 * 128 * 2 / 16;  // one block of 64 keys, in 16-byte units

__global__ void __launch_bounds__(256) gather_kernel(const uint4* __restrict__ K,
                                                     const uint4* __restrict__ V,
                                                     const int* __restrict__ blocks,
                                                     uint32_t* __restrict__ out) {
  const int row = blockIdx.x / (kSel / 2), pair = blockIdx.x % (kSel / 2);
  uint4 v[16];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int blk = blocks[row * kSel + pair * 2 + j];
    const size_t base = ((size_t)row * kBlocksPerRow + blk) * kBlockU4 + threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[j * 8 + i] = K[base + i * 256];
      v[j * 8 + 4 + i] = V[base + i * 256];
    }
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int j = 0; j < 256; ++j) a ^= red[j];
    out[blockIdx.x] = a;
  }
}

// The same blocks read in the decode kernel's per-wave layout: wave w of the
// workgroup takes keys 32 (w % 2) .. + 32 of block w / 2; K as sixteen-byte
// loads (lane l: rows l % 16 and 16 + l % 16, dims 8 (l / 16) + 32 ch), V as
// one row per wave instruction, four bytes per lane (V4 = false: 32 loads per
// lane) or sixteen (V4 = true: lane l takes rows 4 i + l / 16, dims 8 (l % 16),
// 8 loads per lane).
template <bool V4>
__global__ void __launch_bounds__(256) gather_layout_kernel(const uint4* __restrict__ K,
                                                            const uint4* __restrict__ V,
                                                            const int* __restrict__ blocks,
                                                            uint32_t* __restrict__ out) {
  const int row = blockIdx.x / (kSel / 2), pair = blockIdx.x % (kSel / 2);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int blk = blocks[row * kSel + pair * 2 + (wave >> 1)];
  const size_t block_u4 = ((size_t)row * kBlocksPerRow + blk) * kBlockU4;
  const int key0 = (wave & 1) * 32;
  // K: row-major [64 keys][128 dims] bf16 = 16 uint4 per key row
  uint4 kf[8];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
      kf[kt * 4 + ch] = K[block_u4 + (size_t)(key0 + kt * 16 + (lane & 15)) * 16 + ch * 4 + (lane >> 4)];
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc ^= kf[i].x ^ kf[i].y ^ kf[i].z ^ kf[i].w;
  if constexpr (V4) {
    uint4 vv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      vv[i] = V[block_u4 + (size_t)(key0 + 4 * i + (lane >> 4)) * 16 + (lane & 15)];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= vv[i].x ^ vv[i].y ^ vv[i].z ^ vv[i].w;
  } else {
    const uint32_t* Vw = reinterpret_cast<const uint32_t*>(V);
    uint32_t vr[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) vr[r] = Vw[(block_u4 + (size_t)(key0 + r) * 16) * 4 + lane];
#pragma unroll
    for (int r = 0; r < 32; ++r) acc ^= vr[r];
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

static int gather_main() {
  const size_t cache_bytes = (size_t)kRows * kBlocksPerRow * kBlockU4 * 16;  // 1 GiB
  const int reps = 256;
  void *K = nullptr, *V = nullptr;
  int* dblocks = nullptr;
  uint32_t* out = nullptr;
  PROBE_CHECK(hipMalloc(&K, cache_bytes));
  PROBE_CHECK(hipMalloc(&V, cache_bytes));
  PROBE_CHECK(hipMemset(K, 1, cache_bytes));
  PROBE_CHECK(hipMemset(V, 2, cache_bytes));
  PROBE_CHECK(hipMalloc(&out, kRows * (kSel / 2) * sizeof(uint32_t)));
  const size_t per_launch = (size_t)kRows * kSel;
  PROBE_CHECK(hipMalloc(&dblocks, reps * per_launch * sizeof(int)));
  hipEvent_t e0, e1;
  PROBE_CHECK(hipEventCreate(&e0));
  PROBE_CHECK(hipEventCreate(&e1));
  const size_t bytes = per_launch * 2 * kBlockU4 * 16;  // K and V
  for (const char* pattern : {"random", "adjacent", "random-dwordV", "random-16BV"}) {
    std::vector<int> h(reps * per_launch);
    uint64_t st = 0x9E3779B97F4A7C15ull;
    std::vector<int> perm(kBlocksPerRow);
    for (int r = 0; r < reps; ++r)
      for (int row = 0; row < kRows; ++row) {
        int* dst = &h[(r * kRows + row) * kSel];
        if (pattern[0] == 'r') {  // partial Fisher-Yates with a 64-bit LCG
          for (int i = 0; i < kBlocksPerRow; ++i) perm[i] = i;
          for (int i = 0; i < kSel; ++i) {
            st = st * 6364136223846793005ull + 1442695040888963407ull;
            const int j = i + (int)((st >> 33) % (uint64_t)(kBlocksPerRow - i));
            std::swap(perm[i], perm[j]);
          }
          std::copy(perm.begin(), perm.begin() + kSel, dst);
          std::sort(dst, dst + kSel);
        } else {
          for (int i = 0; i < kSel; ++i) dst[i] = (r % (kBlocksPerRow / kSel)) * kSel + i;
        }
      }
    PROBE_CHECK(hipMemcpy(dblocks, h.data(), h.size() * sizeof(int), hipMemcpyHostToDevice));
    float ms = 0.0f;
    for (int pass = 0; pass < 2; ++pass) {  // the first pass warms up
      PROBE_CHECK(hipEventRecord(e0));
      for (int r = 0; r < reps; ++r) {
        const int* blk = dblocks + r * per_launch;
        if (std::strcmp(pattern, "random-dwordV") == 0)
          hipLaunchKernelGGL(gather_layout_kernel<false>, dim3(kRows * (kSel / 2)), dim3(256), 0,
                             0, (const uint4*)K, (const uint4*)V, blk, out);
        else if (std::strcmp(pattern, "random-16BV") == 0)
          hipLaunchKernelGGL(gather_layout_kernel<true>, dim3(kRows * (kSel / 2)), dim3(256), 0,
                             0, (const uint4*)K, (const uint4*)V, blk, out);
        else
          hipLaunchKernelGGL(gather_kernel, dim3(kRows * (kSel / 2)), dim3(256), 0, 0,
                             (const uint4*)K, (const uint4*)V, blk, out);
      }
      PROBE_CHECK(hipGetLastError());
      PROBE_CHECK(hipEventRecord(e1));
      PROBE_CHECK(hipEventSynchronize(e1));
      PROBE_CHECK(hipEventElapsedTime(&ms, e0, e1));
    }
    const double us = ms * 1e3 / reps;
    std::printf(
        "{\"gather\": \"%s\", \"bytes\": %zu, \"grid\": %d, \"us_per_launch\": %.2f, "
        "\"GBps\": %.1f}\n",
        pattern, bytes, kRows * (kSel / 2), us, bytes / (us * 1e3));
    std::fflush(stdout);
  }
  PROBE_CHECK(hipFree(dblocks));
  PROBE_CHECK(hipFree(out));
  PROBE_CHECK(hipFree(K));
  PROBE_CHECK(hipFree(V));
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && std::strcmp(argv[1], "--gather") == 0) return gather_main();
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
