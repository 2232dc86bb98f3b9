// HBM read-bandwidth probe (measurement tool, not part of the library).
// Sets the practical ceiling the decode kernel is measured against:
//   (a) contiguous streaming reads of 2 GiB, 16-byte loads, plain and with
//       the non-temporal (streaming) cache hint;
//   (b) reads of 4 KiB K and V tiles, the access pattern of a paged KV cache:
//       fully random tiles, and the decode kernel's own pattern (one wave per
//       (sequence, head) walking its sequence's blocks in a random pool), at
//       the LLaMA-7B decode working-set size (2 x 570 MB).
// Every access is in bounds by construction; times are HIP events over 10
// launches after 3 warm-ups.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                          \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      printf("%s failed: %s\n", #x, hipGetErrorString(e_));              \
      exit(1);                                                            \
    }                                                                     \
  } while (0)

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// each workgroup reads chunks_per_wg * 256 chunks contiguous; UNROLL loads in flight per thread
template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ p, uint32_t* out, int64_t chunks_per_wg,
                                                   int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * chunks_per_wg * 256;
  uint32_t acc = 0;
  for (int64_t i = 0; i < chunks_per_wg; i += UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t idx = base + (i + u) * 256 + threadIdx.x;
      v[u] = idx < n16 ? ld<NT>(p + idx) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x12345678u) out[blockIdx.x] = acc;
}

// one wave per workgroup reads tiles_per_wave tiles of 4 KiB (K) + 4 KiB (V);
// tile ids come from `tiles`, two tiles (16 loads) in flight
template <bool NT>
__global__ __launch_bounds__(64) void tile_read(const u32x4* __restrict__ kp, const u32x4* __restrict__ vp,
                                                const int* __restrict__ tiles, uint32_t* out, int tiles_per_wave) {
  const int lane = threadIdx.x;
  const int wave = blockIdx.x;
  uint32_t acc = 0;
  for (int i = 0; i < tiles_per_wave; i += 2) {
    u32x4 v[2][8];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int64_t t = tiles[(int64_t)wave * tiles_per_wave + i + d];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[d][j] = ld<NT>(kp + t * 256 + j * 64 + lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[d][4 + j] = ld<NT>(vp + t * 256 + j * 64 + lane);
    }
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc ^= v[d][j][0] ^ v[d][j][3];
  }
  if (acc == 0x12345678u) out[wave] = acc;
}

int main() {
  const int64_t bytes = 2LL << 30;  // 2 GiB per pool
  const int64_t n16 = bytes / 16;
  u32x4 *a, *b;
  uint32_t* out;
  int* tiles;
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
    printf("%-58s %8.1f GB/s  (%.1f us/launch)\n", name, moved * 10 / (ms * 1e-3) / 1e9, ms * 100);
    fflush(stdout);
  };
  for (int64_t cpw : {16, 64}) {
    const int64_t nwg = (n16 + cpw * 256 - 1) / (cpw * 256);
    char nm[128];
    snprintf(nm, sizeof nm, "stream 2 GiB, 8 loads/thread, %lld chunks/wg, plain", (long long)cpw);
    time_it([&] { hipLaunchKernelGGL((stream_read<8, false>), dim3(nwg), dim3(256), 0, 0, a, out, cpw, n16); },
            bytes, nm);
    snprintf(nm, sizeof nm, "stream 2 GiB, 8 loads/thread, %lld chunks/wg, nontemporal", (long long)cpw);
    time_it([&] { hipLaunchKernelGGL((stream_read<8, true>), dim3(nwg), dim3(256), 0, 0, a, out, cpw, n16); },
            bytes, nm);
  }
  // paged pools: 136 sequences x 32 blocks of 32 heads x 4 KiB (570 MB per pool)
  const int H = 32, S = 136, TPW = 32;
  const int nblk = S * TPW;
  const int nwaves = S * H;
  std::mt19937 rng(1);
  std::vector<int> perm(nblk);
  for (int i = 0; i < nblk; ++i) perm[i] = i;
  std::shuffle(perm.begin(), perm.end(), rng);
  std::vector<int> h((size_t)nwaves * TPW);
  CHECK(hipMalloc(&tiles, h.size() * 4));
  const double moved = (double)nwaves * TPW * 8192;
  for (int w = 0; w < nwaves; ++w) {
    const int s = w / H, hd = w % H;
    for (int i = 0; i < TPW; ++i) h[(size_t)w * TPW + i] = perm[s * TPW + i] * H + hd;
  }
  CHECK(hipMemcpy(tiles, h.data(), h.size() * 4, hipMemcpyHostToDevice));
  time_it([&] { hipLaunchKernelGGL((tile_read<false>), dim3(nwaves), dim3(64), 0, 0, a, b, tiles, out, TPW); },
          moved, "paged (seq, head) waves over random blocks, plain");
  time_it([&] { hipLaunchKernelGGL((tile_read<true>), dim3(nwaves), dim3(64), 0, 0, a, b, tiles, out, TPW); },
          moved, "paged (seq, head) waves over random blocks, nontemporal");
  std::vector<int> all((size_t)nblk * H);
  for (size_t i = 0; i < all.size(); ++i) all[i] = (int)i;
  std::shuffle(all.begin(), all.end(), rng);
  CHECK(hipMemcpy(tiles, all.data(), all.size() * 4, hipMemcpyHostToDevice));
  time_it([&] { hipLaunchKernelGGL((tile_read<false>), dim3(nwaves), dim3(64), 0, 0, a, b, tiles, out, TPW); },
          moved, "random 4 KiB K+V tiles, plain");
  time_it([&] { hipLaunchKernelGGL((tile_read<true>), dim3(nwaves), dim3(64), 0, 0, a, b, tiles, out, TPW); },
          moved, "random 4 KiB K+V tiles, nontemporal");
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  printf("device %s CUs %d clock %d kHz memclock %d kHz bus %d bits L2 %d\n", prop.gcnArchName,
         prop.multiProcessorCount, prop.clockRate, prop.memoryClockRate, prop.memoryBusWidth, prop.l2CacheSize);
  return 0;
}
