// Cache write (reshape_and_cache) and logical gather (gather_kv).
//
// reshape_and_cache puts the K/V rows of this step's new tokens into the
// block slots the allocator handed out: a new token's cache lives in some
// physical block chosen on demand, at the offset its position gives
// (devpress.csdn.net page, sections on how PagedAttention works and on the
// paged KV cache; betteryeah.com page, section 2.2). Both kernels are pure
// 16-byte copies: bit-exact by construction, HBM-bound.
#include "pa_internal.h"

namespace pa {

// One thread moves one 16-byte chunk of one (token, head) row of K and of V.
// Grid: ceil(T * H * CPR / 256) workgroups of 256; CPR = row bytes / 16.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int64_t total_chunks, int H,
    int BS, int CPR) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total_chunks) return;
  const int c = (int)(i % CPR);
  const int64_t nh = i / CPR;  // token * H + head
  const int h = (int)(nh % H);
  const int64_t n = nh / H;
  const int32_t slot = slot_mapping[n];
  if (slot < 0) return;
  const int32_t blk = slot / BS, off = slot % BS;
  const int64_t dst = (((int64_t)blk * H + h) * BS + off) * CPR + c;
  const uint4 kk = k[i];
  const uint4 vv = v[i];
  k_cache[dst] = kk;
  v_cache[dst] = vv;
}

// Row r = cu[s] + t of the output is logical token t of sequence s.
// Grid: (ceil(max_ctx * H * CPR / 256), S).
__global__ __launch_bounds__(256) void gather_kv_kernel(
    uint4* __restrict__ k_out, uint4* __restrict__ v_out, const uint4* __restrict__ k_cache,
    const uint4* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_ctx, int H, int BS, int CPR,
    int max_blocks) {
  const int s = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // within the sequence
  const int ctx = context_lens[s];
  if (i >= (int64_t)ctx * H * CPR) return;
  const int c = (int)(i % CPR);
  const int64_t th = i / CPR;
  const int h = (int)(th % H);
  const int t = (int)(th / H);
  const int32_t phys = block_tables[(int64_t)s * max_blocks + t / BS];
  const int64_t src = kv_row_offset(phys, h, t % BS, H, BS, CPR);  // in 16-byte units
  const int64_t dst = (((int64_t)cu_ctx[s] + t) * H + h) * CPR + c;
  k_out[dst] = k_cache[src + c];
  v_out[dst] = v_cache[src + c];
}

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int T, int H, int D, int BS, int elt_bytes,
                                    hipStream_t stream) {
  const int CPR = D * elt_bytes / 16;
  const int64_t total = (int64_t)T * H * CPR;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const uint4*)k,
                     (const uint4*)v, (uint4*)k_cache, (uint4*)v_cache, slot_mapping, total, H, BS, CPR);
  return hipGetLastError();
}

hipError_t launch_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_ctx,
                            int S, int max_ctx, int H, int D, int BS, int max_blocks, int elt_bytes,
                            hipStream_t stream) {
  const int CPR = D * elt_bytes / 16;
  const int64_t per_seq = (int64_t)max_ctx * H * CPR;
  if (per_seq == 0 || S == 0) return hipSuccess;
  const int64_t gx = (per_seq + 255) / 256;
  hipLaunchKernelGGL(gather_kv_kernel, dim3((unsigned)gx, (unsigned)S), dim3(256), 0, stream, (uint4*)k_out,
                     (uint4*)v_out, (const uint4*)k_cache, (const uint4*)v_cache, block_tables, context_lens,
                     cu_ctx, H, BS, CPR, max_blocks);
  return hipGetLastError();
}

}  // namespace pa
