// Cache write (reshape_and_cache), copy-on-write of whole blocks
// (copy_blocks) and logical gather (gather_kv).
//
// reshape_and_cache puts the K/V rows of this step's new tokens into the
// block slots the allocator handed out: a new token's cache lives in some
// physical block chosen on demand, at the offset its position gives
// (devpress.csdn.net page, sections on how PagedAttention works and on the
// paged KV cache; betteryeah.com page, section 2.2). copy_blocks is the copy
// half of copy-on-write: parallel samples share the prompt's blocks, and a
// sharer about to write into a shared block first gets its own copy
// (aidocs.cortexgrid.cn page, FAQ answer on parallel sampling). All three
// kernels are pure 16-byte copies: bit-exact by construction, HBM-bound.
#include "pa_internal.h"

namespace pa {

// One thread moves one 16-byte chunk of one (token, head) row of K and of V.
// Grid: ceil(T * H * CPR / 256) workgroups of 256; CPR = row bytes / 16.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int64_t total_chunks, int H,
    int BS, int CPR, int32_t num_slots) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total_chunks) return;
  const int c = (int)(i % CPR);
  const int64_t nh = i / CPR;  // token * H + head
  const int h = (int)(nh % H);
  const int64_t n = nh / H;
  const int32_t slot = slot_mapping[n];
  if (slot < 0 || slot >= num_slots) return;  // padding (and, defensively, slots past the pool)
  const int32_t blk = slot / BS, off = slot % BS;
  const int64_t dst = (((int64_t)blk * H + h) * BS + off) * CPR + c;
  const uint4 kk = k[i];
  const uint4 vv = v[i];
  k_cache[dst] = kk;
  v_cache[dst] = vv;
}

// Block dst <- block src for every (src, dst) pair, K and V. A block is one
// contiguous run of H * BS * D elements in each cache (CPB 16-byte chunks);
// each workgroup copies 1024 chunks (4 per thread, loads first) of one pair.
// Grid: pairs * ceil(CPB / 1024). Pairs naming a block outside the pool are
// skipped.
__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ mapping, int64_t cpb,
                                                          int wgs_per_block, int num_blocks) {
  const int pair = blockIdx.x / wgs_per_block;
  const int64_t c0 = (int64_t)(blockIdx.x % wgs_per_block) * 1024 + threadIdx.x;
  const int32_t src = mapping[2 * pair], dst = mapping[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const u32x4* ks = k_cache + (int64_t)src * cpb;
  const u32x4* vs = v_cache + (int64_t)src * cpb;
  u32x4* kd = k_cache + (int64_t)dst * cpb;
  u32x4* vd = v_cache + (int64_t)dst * cpb;
  u32x4 kx[4], vx[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t c = min(c0 + 256 * u, cpb - 1);
    kx[u] = __builtin_nontemporal_load(ks + c);
    vx[u] = __builtin_nontemporal_load(vs + c);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t c = c0 + 256 * u;
    if (c < cpb) {
      __builtin_nontemporal_store(kx[u], kd + c);
      __builtin_nontemporal_store(vx[u], vd + c);
    }
  }
}

// Row r = cu[s] + t of the output is logical token t of sequence s.
// Grid: (ceil(max_ctx * H * CPR / 256), S).
__global__ __launch_bounds__(256) void gather_kv_kernel(
    uint4* __restrict__ k_out, uint4* __restrict__ v_out, const uint4* __restrict__ k_cache,
    const uint4* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_ctx, int H, int BS, int CPR,
    int max_blocks, int max_ctx, int num_blocks) {
  const int s = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // within the sequence
  const int ctx = clamp_len(context_lens[s], max_ctx);
  if (i >= (int64_t)ctx * H * CPR) return;
  const int c = (int)(i % CPR);
  const int64_t th = i / CPR;
  const int h = (int)(th % H);
  const int t = (int)(th / H);
  const int32_t phys = clamp_block(block_tables[(int64_t)s * max_blocks + t / BS], num_blocks);
  const int64_t src = kv_row_offset(phys, h, t % BS, H, BS, CPR);  // in 16-byte units
  const int64_t dst = (((int64_t)cu_ctx[s] + t) * H + h) * CPR + c;
  k_out[dst] = k_cache[src + c];
  v_out[dst] = v_cache[src + c];
}

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int T, int H, int D, int BS, int num_blocks,
                                    int elt_bytes, hipStream_t stream) {
  const int CPR = D * elt_bytes / 16;
  const int64_t total = (int64_t)T * H * CPR;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const uint4*)k,
                     (const uint4*)v, (uint4*)k_cache, (uint4*)v_cache, slot_mapping, total, H, BS, CPR,
                     (int32_t)((int64_t)num_blocks * BS));
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping, int num_pairs, int H,
                              int D, int BS, int num_blocks, int elt_bytes, hipStream_t stream) {
  const int64_t cpb = (int64_t)H * BS * D * elt_bytes / 16;
  const int wgs = (int)((cpb + 1023) / 1024);
  const int64_t grid = (int64_t)num_pairs * wgs;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (u32x4*)k_cache,
                     (u32x4*)v_cache, block_mapping, cpb, wgs, num_blocks);
  return hipGetLastError();
}

hipError_t launch_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_ctx,
                            int S, int max_ctx, int H, int D, int BS, int max_blocks, int num_blocks,
                            int elt_bytes, hipStream_t stream) {
  const int CPR = D * elt_bytes / 16;
  const int64_t per_seq = (int64_t)max_ctx * H * CPR;
  if (per_seq == 0 || S == 0) return hipSuccess;
  const int64_t gx = (per_seq + 255) / 256;
  hipLaunchKernelGGL(gather_kv_kernel, dim3((unsigned)gx, (unsigned)S), dim3(256), 0, stream, (uint4*)k_out,
                     (uint4*)v_out, (const uint4*)k_cache, (const uint4*)v_cache, block_tables, context_lens,
                     cu_ctx, H, BS, CPR, max_blocks, max_ctx, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
