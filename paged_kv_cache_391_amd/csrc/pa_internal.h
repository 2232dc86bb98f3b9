// Host-side launcher declarations shared between the C-ABI layer and the
// kernel files. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

// Decode tuning: heads per workgroup (one wave each), the number of waves
// per SIMD the partition kernel's register budget must leave room for, and
// tokens per split-K partition. One head per workgroup: consecutive
// workgroups take consecutive heads of a row, so the rows of one head are H
// workgroups apart; workgroups go round-robin over the chip's 8 XCDs, and
// with H a multiple of 8 all rows of a head run on one XCD, where sequences
// that alias the same blocks share its L2.
#ifndef PA_DECODE_HEADS
#define PA_DECODE_HEADS 1
#endif
#ifndef PA_DECODE_MIN_WAVES
#define PA_DECODE_MIN_WAVES 5
#endif
#ifndef PA_PARTITION_TOKENS
#define PA_PARTITION_TOKENS 512
#endif
#ifndef PA_SHARED_PARTITION_TOKENS
#define PA_SHARED_PARTITION_TOKENS 1024
#endif

namespace pa {

constexpr int kDecodeHeadsPerGroup = PA_DECODE_HEADS;
constexpr int kPartitionTokens = PA_PARTITION_TOKENS;
static_assert(kPartitionTokens % 32 == 0, "partitions must hold whole 16- and 32-token blocks");
// Shared prefixes are split coarser than private tokens: a shared wave serves
// up to 16 members, and fewer, longer shared waves measured faster (less
// set-up and fewer partials per member). A shared partition is at most 64
// blocks (the table entries one wave holds in its lanes), so its length is
// min(kSharedPartitionTokens, 64 * block_size) -- never below
// kPartitionTokens for the supported block sizes, which keeps a row's
// shared + own partitions within ceil(ctx / kPartitionTokens) + 1 slots.
constexpr int kSharedPartitionTokens = PA_SHARED_PARTITION_TOKENS;
static_assert(kSharedPartitionTokens % 32 == 0 && kSharedPartitionTokens >= kPartitionTokens &&
                  64 * 8 >= kPartitionTokens,
              "shared partitions must hold whole 32-token steps and no fewer tokens than a private one");
inline int shared_partition_tokens(int block_size) {
  return kSharedPartitionTokens < 64 * block_size ? kSharedPartitionTokens : 64 * block_size;
}

// Which rows a partition-kernel launch walks.
enum class RowMode : int {
  Decode = 0,       // row s = sequence s, tokens [0, ctx)
  SharedTail = 2,   // row s = sequence s of a prefix-sharing group, tokens [prefix, ctx)
};

struct DecodeArgs {
  void* out;                        // [rows][H][D], fp32 or the input dtype
  float* ws;                        // split-K partials (nullptr: single partition)
  const void* q;                    // [rows][H][D]
  const void* k_cache;              // [num_blocks][H][BS][D]
  const void* v_cache;
  const int32_t* block_tables;      // [num_seqs][max_blocks]
  const int32_t* context_lens;      // [num_seqs]
  int num_rows;                     // rows of the launch (one per sequence)
  int num_seqs;
  int H;
  int max_blocks;
  int max_ctx;                      // the call's max_context_len: contexts are clamped to it
  int num_blocks;                   // pool size: block ids are clamped below it
  int max_parts;                    // partitions per row in the grid
  int ws_parts;                     // partition slots per (row, head) in the workspace
  int part_tiles;                   // 16-token tiles per partition
  int shared_part_tiles;            // 16-token tiles per shared-prefix partition
  const int32_t* group_starts;      // SharedTail / shared-prefix kernel: [num_groups+1] row ranges
  const int32_t* prefix_lens;       // [num_groups] shared tokens (whole 16-token tiles)
  int num_groups;
  int member_chunks;                // shared-prefix kernel: waves per (group, head, partition)
  float scale_log2;                 // scale * log2(e)
  int out_f32;
  // decode with the fused cache write: row r's new token (K and V rows of
  // [rows][H][D], slot slot_mapping[r]) is used by K2 as position
  // context_lens[r] - 1 and written into its slot, by K3 when write_in_reduce
  // is set (a reduction follows) and by K2 otherwise; nullptr: no write
  const void* new_k;
  const void* new_v;
  const int32_t* slot_mapping;
  int write_in_reduce;
  int block_size;
};

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int T, int H, int D, int BS, int num_blocks,
                                    int elt_bytes, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping, int num_pairs, int H,
                              int D, int BS, int num_blocks, int elt_bytes, hipStream_t stream);
hipError_t launch_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_ctx,
                            int S, int max_ctx, int H, int D, int BS, int max_blocks, int num_blocks,
                            int elt_bytes, hipStream_t stream);

// partition kernel (K2) over the rows `mode` describes
hipError_t launch_decode_partitions(const DecodeArgs& a, Dt dt, int D, int BS, RowMode mode, hipStream_t stream);
// reduction kernel (K3); shared = rows carry a shared-prefix partition offset
hipError_t launch_decode_reduce(const DecodeArgs& a, Dt dt, int D, bool shared, hipStream_t stream);
// shared-prefix decode before the reduction, in one launch: the shared
// prefixes on the matrix cores (each shared K/V tile read once per group, one
// wave per 16 members; shared_parts partitions) next to the members' private
// tails (SharedTail rows; tail_parts partitions), f16/bf16
hipError_t launch_shared_prefix_step(const DecodeArgs& a, Dt dt, int D, int BS, int shared_parts, int tail_parts,
                                     hipStream_t stream);
constexpr int kSharedMembersPerWave = 16;

// MFMA causal prefill: K4 (fp16/bf16) and its fp32 form
struct PrefillArgs {
  void* out;                        // [total_q][H][D]
  const void* q;                    // [total_q][H][D]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  int num_seqs;
  int total_q;
  int H;
  int max_blocks;
  int max_context_len;
  int num_blocks;
  int q_tiles;                      // grid: q tiles per sequence
  int grouped;                      // grid order: query tiles of a (sequence, head) pair together
  int wide;                         // f16/bf16, head dim 128: the wide workgroup shape
  int cus;                          // compute units of the device (0: unknown)
  float scale_log2;                 // |scale| * log2(e)
  uint32_t q_sign;                  // negative scale (queries negated): 0x80008000, else 0
  int out_f32;
};
hipError_t launch_prefill_mfma(const PrefillArgs& a, Dt dt, int D, int BS, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, int D, int BS, hipStream_t stream);
int prefill_mfma_q_tile();
// workgroups of the prefill kernels (f16/bf16 standard shape; f32) resident
// at once on each compute unit
constexpr int kPrefillWorkgroupsPerCU = 3;
constexpr int kPrefillF32WorkgroupsPerCU = 2;

}  // namespace pa
