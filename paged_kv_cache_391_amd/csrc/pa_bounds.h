// Index arithmetic on caller data, shared by the host-side launch plans and
// the kernels: how lengths and block ids read from device memory are
// clamped, and how many split-K partitions a row has. Everything here is a
// pure function of integers (host and device), so a CPU test can check,
// over any input, that the kernels' reads and writes stay inside the
// buffers the host validated and sized.
//
// Lengths and block ids come from device memory the host never reads. A
// value that breaks a call's precondition must not send a kernel outside
// the caller's buffers (a fault can take the whole device down), so kernels
// clamp them: lengths to [0, max_context_len] (the host checked
// max_context_len <= max_blocks_per_seq * block_size, so a clamped length
// stays inside its table row and the partitions the grid and workspace were
// sized for), block ids to [0, num_blocks) (a negative id wraps to a large
// unsigned value and is clamped too). Valid inputs are unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

__host__ __device__ inline int clamp_len(int x, int max_len) { return x < 0 ? 0 : (x > max_len ? max_len : x); }

__host__ __device__ inline int32_t clamp_block(int32_t b, int num_blocks) {
  const uint32_t u = (uint32_t)b, top = (uint32_t)(num_blocks - 1);
  return (int32_t)(u < top ? u : top);
}

// 16-token tiles of a context (kernels walk whole tiles; the last is masked)
__host__ __device__ inline int tiles_of(int tokens) { return (tokens + 15) >> 4; }

// Split-K partitions of max_context_len tokens at part_tokens per partition
// (at least 1): the grid's partition count and the workspace's slots per
// (row, head).
__host__ __device__ inline int64_t partitions_for(int64_t max_context_len, int part_tokens) {
  return max_context_len <= 0 ? 1 : (max_context_len + part_tokens - 1) / part_tokens;
}

// Tiles of the one partition that spans a whole context when split-K is off.
__host__ __device__ inline int single_partition_tiles(int max_context_len) {
  const int t = tiles_of(max_context_len);
  return t > 0 ? t : 1;
}

// Partitions of part_tiles tiles covering tokens [tok0, ctx) of a row, tok0
// a multiple of 16 and at most ctx.
__host__ __device__ inline int own_partitions(int ctx, int tok0, int part_tiles) {
  const int own_tiles = tiles_of(ctx) - (tok0 >> 4);
  return (own_tiles + part_tiles - 1) / part_tiles;
}

// Query rows and context of one prefill chunk, from raw query_start_loc
// entries and context length: rows [q_beg, q_beg + L) with L <= ctx, so the
// chunk's first query sits at ctx - L >= 0. A range past total_q or a chunk
// longer than its context (both break the call's preconditions) is cut.
struct ChunkRows {
  int q_beg, L, ctx;
};
__host__ __device__ inline ChunkRows chunk_rows(int qsl_s, int qsl_s1, int raw_ctx, int total_q, int max_context_len) {
  ChunkRows c;
  c.ctx = clamp_len(raw_ctx, max_context_len);
  c.q_beg = clamp_len(qsl_s, total_q);
  const int q_end = clamp_len(qsl_s1, total_q);
  const int L = q_end - c.q_beg;
  c.L = L < c.ctx ? L : c.ctx;
  return c;
}

}  // namespace pa
