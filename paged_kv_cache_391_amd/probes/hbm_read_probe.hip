// HBM read-bandwidth probe (measurement tool, not part of the library).
// Sets the practical ceiling the decode kernel is judged against:
//   (a) contiguous streaming reads of 2 GiB, 16-byte loads;
//   (b) reads of 4 KiB K and V tiles at random places in two 1.2 GiB pools,
//       which is the access pattern of a paged KV cache with random block
//       placement (each wave streams one K and one V tile per step).
// Every access is in bounds by construction; times are HIP events over 10
// launches after 3 warm-ups.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#include <vector>
#include <algorithm>
#include <random>
#include <cstdlib>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                          \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      printf("%s failed: %s\n", #x, hipGetErrorString(e_));              \
      exit(1);                                                            \
    }                                                                     \
  } while (0)

// each workgroup reads `per_wg` bytes contiguous starting at its chunk; UNROLL loads in flight per thread
template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ p, uint32_t* out, int64_t chunks_per_wg, int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * chunks_per_wg * 256;
  uint32_t acc = 0;
  for (int64_t i = 0; i < chunks_per_wg; i += UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      int64_t idx = base + (i + u) * 256 + threadIdx.x;
      v[u] = idx < n16 ? p[idx] : u32x4{0,0,0,0};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x12345678u) out[blockIdx.x] = acc;
}

// each wave reads TILES tiles of 4 KiB (K) + 4 KiB (V) at random tile indices from two pools
template <int DEPTH>
__global__ __launch_bounds__(256) void tile_read(const u32x4* __restrict__ kp, const u32x4* __restrict__ vp, const int* __restrict__ tiles,
                                                 uint32_t* out, int tiles_per_wave) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * 4) + (threadIdx.x >> 6);
  uint32_t acc = 0;
  for (int i = 0; i < tiles_per_wave; i += DEPTH) {
    u32x4 v[DEPTH][8];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int64_t t = tiles[(int64_t)wave * tiles_per_wave + i + d];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[d][j] = kp[t * 256 + j * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[d][4 + j] = vp[t * 256 + j * 64 + lane];
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc ^= v[d][j][0] ^ v[d][j][3];
  }
  if (acc == 0x12345678u) out[wave] = acc;
}

int main() {
  const int64_t bytes = 2LL << 30;  // 2 GiB per pool
  const int64_t n16 = bytes / 16;
  u32x4 *a, *b; uint32_t* out; int* tiles;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMalloc(&out, 1 << 24));
  CHECK(hipMemset(a, 1, bytes));
  CHECK(hipMemset(b, 2, bytes));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  auto time_it = [&](auto launch, double moved, const char* name) {
    for (int i = 0; i < 3; ++i) launch();
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int i = 0; i < 10; ++i) launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    printf("%-48s %8.1f GB/s  (%.1f us/launch)\n", name, moved * 10 / (ms * 1e-3) / 1e9, ms * 100);
  };
  for (int64_t cpw : {16, 64, 256}) {
    int64_t nwg = (n16 + cpw * 256 - 1) / (cpw * 256);
    char nm[128];
    snprintf(nm, sizeof nm, "stream unroll4 chunks/wg=%lld (wgs=%lld)", (long long)cpw, (long long)nwg);
    time_it([&] { hipLaunchKernelGGL(stream_read<4>, dim3(nwg), dim3(256), 0, 0, a, out, cpw, n16); }, bytes, nm);
    snprintf(nm, sizeof nm, "stream unroll8 chunks/wg=%lld", (long long)cpw);
    time_it([&] { hipLaunchKernelGGL(stream_read<8>, dim3(nwg), dim3(256), 0, 0, a, out, cpw, n16); }, bytes, nm);
  }
  // random 4 KiB tiles from a 1.2 GiB window of each pool, like a permuted paged cache
  const int64_t ntile_pool = (1200LL << 20) / 4096;
  const int tiles_per_wave = 32;
  const int nwaves = (int)(ntile_pool / tiles_per_wave);
  std::vector<int> h(ntile_pool);
  for (int64_t i = 0; i < ntile_pool; ++i) h[i] = (int)i;
  std::mt19937 rng(1); std::shuffle(h.begin(), h.end(), rng);
  CHECK(hipMalloc(&tiles, h.size() * 4));
  CHECK(hipMemcpy(tiles, h.data(), h.size() * 4, hipMemcpyHostToDevice));
  const double moved = (double)nwaves * tiles_per_wave * 8192;
  time_it([&] { hipLaunchKernelGGL(tile_read<1>, dim3(nwaves / 4), dim3(256), 0, 0, a, b, tiles, out, tiles_per_wave); }, moved, "random 4K K+V tiles depth1");
  time_it([&] { hipLaunchKernelGGL(tile_read<2>, dim3(nwaves / 4), dim3(256), 0, 0, a, b, tiles, out, tiles_per_wave); }, moved, "random 4K K+V tiles depth2");
  time_it([&] { hipLaunchKernelGGL(tile_read<4>, dim3(nwaves / 4), dim3(256), 0, 0, a, b, tiles, out, tiles_per_wave); }, moved, "random 4K K+V tiles depth4");
  for (int i = 0; i < ntile_pool; ++i) h[i] = i;
  CHECK(hipMemcpy(tiles, h.data(), h.size() * 4, hipMemcpyHostToDevice));
  time_it([&] { hipLaunchKernelGGL(tile_read<2>, dim3(nwaves / 4), dim3(256), 0, 0, a, b, tiles, out, tiles_per_wave); }, moved, "sequential 4K K+V tiles depth2");
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  printf("device %s CUs %d clock %d kHz memclock %d kHz bus %d bits L2 %d\n", prop.gcnArchName, prop.multiProcessorCount, prop.clockRate, prop.memoryClockRate, prop.memoryBusWidth, prop.l2CacheSize);
  return 0;
}
