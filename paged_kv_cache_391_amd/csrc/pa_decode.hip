// Paged decode attention: split-K partition kernel (K2) and reduction (K3).
//
// One query per sequence attends over the sequence's cached tokens, which sit
// in fixed-size blocks scattered through the pool and are reached through the
// sequence's block table (devpress.csdn.net page, sections on how
// PagedAttention works and on the paged KV cache; aidocs.cortexgrid.cn page,
// FAQ answer on the block table; betteryeah.com page, section 2.4). Shared
// prefix blocks are simply read through several tables.
//
// Decode moves ~1 byte per flop, so it is bound by HBM bandwidth and uses no
// matrix cores. Mapping (wave64):
//   * a workgroup takes one partition of one sequence for a group of heads,
//     one wave per head; the waves read neighbouring (block, head) tiles, so
//     the group streams contiguous runs of each block, and the partitions are
//     dispatched partition-major (every sequence's first partition first);
//   * a wave streams 16-token tiles; one 16-lane row of the wave holds one
//     token's K (or V) row, each lane 1/16 of it, so a load instruction
//     reads 4 whole rows = 4 * D * elt contiguous bytes (1 KiB at d=128 f16);
//   * q.k is a per-lane partial dot product (packed f16/bf16 dot2) finished
//     by a 4-step DPP reduction inside the 16-lane row: no LDS, no barrier;
//   * each 16-lane row keeps its own online softmax state (running max m,
//     sum l, accumulator over its D/16 output elements), so the inner loop
//     has no cross-row traffic; rows and waves are merged once at the end;
//   * the block-table entries of a wave's tiles are fetched with one vector
//     load and read out with readlane, so the dependent table load is paid
//     once per 64 tiles, and the next tile's K and V are in flight while the
//     current one is consumed;
//   * K and V are read with non-temporal loads: every cached byte is used
//     once per step, and the streaming hint lifts the measured read rate of
//     random 4 KiB tiles from ~5.9 to ~6.6 TB/s on gfx950.
// Long contexts are cut into partitions of kPartitionTokens tokens (whole
// blocks). A sequence with one partition is finished in place; otherwise
// each partition writes (m, l, acc[D]) and K3 merges them with log-sum-exp
// weights. All reductions run in a fixed order that depends only on logical
// token positions, so results are deterministic and do not change when
// physical blocks are permuted or aliased.
#include "pa_decode_device.h"

namespace pa {

// Occupancy target: f16/bf16 (and f32 at head dim 64) fit the two tile
// buffers in the VGPRs of PA_DECODE_MIN_WAVES waves per SIMD; f32 rows of
// 128 dims carry twice the bytes per lane and need ~162 VGPRs, so those
// kernels ask for three waves per SIMD instead of spilling to scratch.
template <Dt DT, int D> constexpr int decode_min_waves() {
  return DT == Dt::F32 && D == 128 ? 3 : PA_DECODE_MIN_WAVES;
}

template <Dt DT, int D, int BS, int HG, RowMode MODE>
__global__ __launch_bounds__(HG * 64, (decode_min_waves<DT, D>())) void decode_partition_kernel(const DecodeArgs a) {
  decode_partition_body<DT, D, BS, HG, MODE>(a, blockIdx.x, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
}

// K3: merge the partitions of rows that have more than one. One wave per
// (row, head), kReduceWaves heads of a row per workgroup (a quarter of the
// workgroups to dispatch; measured ~0.5 us faster than one wave each);
// lane e handles elements e, e + 64, ...
constexpr int kReduceWaves = 4;
template <Dt DT, int D, RowMode MODE>
__global__ __launch_bounds__(64 * kReduceWaves) void decode_reduce_kernel(const DecodeArgs a) {
  constexpr int NW = kReduceWaves;
  const int hg = (a.H + NW - 1) / NW;
  const int row = blockIdx.x / hg;
  const int h = (blockIdx.x % hg) * NW + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (h >= a.H) return;
  const int lane = threadIdx.x & 63;
  // The fused cache write of a decode step, when a reduction follows the
  // partition kernel: this (row, head)'s new token, which the partition
  // kernel read from new_k/new_v, goes into its slot here. 16 bytes per lane
  // for K and for V, read first (whatever the slot: the rows are always
  // there, and the loads need not wait for the slot) and stored last, unless
  // the slot is padding or past the pool.
  // (The slot is read unconditionally, another row-indexed array standing
  // in when there is none, so it arrives with the row's length in one round
  // trip.)
  constexpr int TOKEN_LANES = D * ElemT<DT>::bytes / 16;
  const bool writes = MODE == RowMode::Decode && a.write_in_reduce;
  const bool token_lane = writes && lane < TOKEN_LANES;
  const int32_t slot = (writes ? a.slot_mapping : a.context_lens)[row];
  u32x4 tk{}, tv{};
  if (token_lane) {
    const int64_t src = ((int64_t)row * a.H + h) * D * ElemT<DT>::bytes + lane * 16;
    tk = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.new_k) + src);
    tv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.new_v) + src);
  }
  auto store_token = [&]() {
    if (token_lane && slot >= 0 && slot < a.num_blocks * a.block_size) {
      const int64_t dst =
          kv_row_offset(slot / a.block_size, h, slot % a.block_size, a.H, a.block_size, D) * ElemT<DT>::bytes +
          lane * 16;
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(const_cast<void*>(a.k_cache)) + dst) = tk;
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(const_cast<void*>(a.v_cache)) + dst) = tv;
    }
  };
  const int ctx = row_ctx(a, row);
  const int nparts = row_parts<MODE>(a, row, ctx).total();
  if (nparts <= 1) {
    store_token();
    return;
  }
  const int64_t prow = ((int64_t)row * a.H + h) * a.ws_parts;
  const float* ml = a.ws + (int64_t)a.num_rows * a.H * a.ws_parts * D + prow * 2;
  const float* acc = a.ws + prow * D;
  constexpr int PER = D / 64;
  // Every load is issued before any result is needed: lane p reads
  // partition p's (m, l) and the first PRE partitions' accumulators are read
  // at once (indices clamped to the row's partitions, weights zero past
  // them), so the merge waits on memory about once instead of once per
  // partition. M and L are reductions across the wave (DPP and row-swap
  // instructions, no LDS round trip); the
  // weighted sum of the accumulators runs in partition order.
  constexpr int PRE = 8;
  float xa[PRE][PER];
#pragma unroll
  for (int p = 0; p < PRE; ++p)
#pragma unroll
    for (int i = 0; i < PER; ++i) xa[p][i] = acc[(int64_t)min(p, nparts - 1) * D + lane + 64 * i];
  const int pl = min(lane, nparts - 1);
  const float m_l = ml[2 * pl];
  const float l_l = ml[2 * pl + 1];
  float M = lane < nparts ? m_l : -INFINITY;
  for (int p = lane + 64; p < nparts; p += 64) M = fmaxf(M, ml[2 * p]);
  M = wave_max_f(M);
  const float w_l = lane < nparts ? fast_exp2(m_l - M) : 0.f;  // weight of partition `lane`
  float Lsum = l_l * w_l;
  for (int p = lane + 64; p < nparts; p += 64) Lsum += ml[2 * p + 1] * fast_exp2(ml[2 * p] - M);
  Lsum = wave_sum_f(Lsum);
  float x[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) x[i] = 0.f;
#pragma unroll
  for (int p = 0; p < PRE; ++p) {
    const float w = p < nparts ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), p))
                               : 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] += xa[p][i] * w;
  }
  for (int p = PRE; p < nparts; ++p) {
    const float w = p < 64 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), p))
                           : fast_exp2(ml[2 * p] - M);
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] += acc[(int64_t)p * D + lane + 64 * i] * w;
  }
  const int64_t orow = ((int64_t)row * a.H + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) store_out<DT>(a.out, orow + lane + 64 * i, x[i] / Lsum, a.out_f32);
  store_token();
}

template <Dt DT, int D, int BS, RowMode MODE>
static hipError_t launch_k2(const DecodeArgs& a, hipStream_t stream) {
  const int64_t n_hg = (a.H + kDecodeHeadsPerGroup - 1) / kDecodeHeadsPerGroup;
  const int64_t grid = (int64_t)a.num_rows * n_hg * a.max_parts;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_partition_kernel<DT, D, BS, kDecodeHeadsPerGroup, MODE>), dim3((unsigned)grid),
                     dim3(kDecodeHeadsPerGroup * 64), 0, stream, a);
  return hipGetLastError();
}

template <Dt DT, int D, RowMode MODE>
static hipError_t dispatch_k2_bs(const DecodeArgs& a, int BS, hipStream_t stream) {
  switch (BS) {
    case 8: return launch_k2<DT, D, 8, MODE>(a, stream);
    case 16: return launch_k2<DT, D, 16, MODE>(a, stream);
    case 32: return launch_k2<DT, D, 32, MODE>(a, stream);
    case 64: return launch_k2<DT, D, 64, MODE>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <Dt DT, RowMode MODE>
static hipError_t dispatch_k2(const DecodeArgs& a, int D, int BS, hipStream_t stream) {
  if (D == 128) return dispatch_k2_bs<DT, 128, MODE>(a, BS, stream);
  if (D == 64) return dispatch_k2_bs<DT, 64, MODE>(a, BS, stream);
  return hipErrorInvalidValue;
}

template <Dt DT>
static hipError_t dispatch_k2_mode(const DecodeArgs& a, int D, int BS, RowMode mode, hipStream_t stream) {
  switch (mode) {
    case RowMode::Decode: return dispatch_k2<DT, RowMode::Decode>(a, D, BS, stream);
    case RowMode::SharedTail: break;  // tails run inside the shared-prefix step kernel only
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_partitions(const DecodeArgs& a, Dt dt, int D, int BS, RowMode mode, hipStream_t stream) {
  switch (dt) {
    case Dt::F32: return dispatch_k2_mode<Dt::F32>(a, D, BS, mode, stream);
    case Dt::F16: return dispatch_k2_mode<Dt::F16>(a, D, BS, mode, stream);
    case Dt::BF16: return dispatch_k2_mode<Dt::BF16>(a, D, BS, mode, stream);
  }
  return hipErrorInvalidValue;
}

template <Dt DT, int D>
static hipError_t launch_k3(const DecodeArgs& a, bool shared, hipStream_t stream) {
  const int64_t grid = (int64_t)a.num_rows * ((a.H + kReduceWaves - 1) / kReduceWaves);
  if (grid == 0) return hipSuccess;
  if (shared)
    hipLaunchKernelGGL((decode_reduce_kernel<DT, D, RowMode::SharedTail>), dim3((unsigned)grid),
                       dim3(64 * kReduceWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<DT, D, RowMode::Decode>), dim3((unsigned)grid), dim3(64 * kReduceWaves),
                       0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeArgs& a, Dt dt, int D, bool shared, hipStream_t stream) {
  switch (dt) {
    case Dt::F32: return D == 128 ? launch_k3<Dt::F32, 128>(a, shared, stream) : launch_k3<Dt::F32, 64>(a, shared, stream);
    case Dt::F16: return D == 128 ? launch_k3<Dt::F16, 128>(a, shared, stream) : launch_k3<Dt::F16, 64>(a, shared, stream);
    case Dt::BF16:
      return D == 128 ? launch_k3<Dt::BF16, 128>(a, shared, stream) : launch_k3<Dt::BF16, 64>(a, shared, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
