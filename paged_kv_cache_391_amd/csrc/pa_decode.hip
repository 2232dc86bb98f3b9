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
#include "pa_internal.h"

namespace pa {

namespace {

template <Dt DT, int D> struct Lane {
  static constexpr int EB = ElemT<DT>::bytes;
  static constexpr int BYTES = D * EB / 16;         // bytes of a row owned by one lane
  static constexpr int WPL = BYTES / 4;             // 32-bit words per lane per row
  static constexpr int VB = BYTES >= 16 ? 16 : 8;   // bytes per load
  static constexpr int NV = BYTES / VB;             // loads per lane per row
  static constexpr int VW = VB / 4;                 // words per load
  static constexpr int EPW = 4 / EB;                // elements per word
  static constexpr int VE = VB / EB;                // elements per load
  static constexpr int EPL = D / 16;                // elements per lane
  static constexpr int ROW_WORDS = D * EB / 4;

  static constexpr int ROW_BYTES = D * EB;

  // element index (within the head's D) of the lane's k-th element
  __device__ static __forceinline__ int elem(int c, int k) { return (k / VE) * 16 * VE + c * VE + (k % VE); }

  // The lane's words of one row. `base` is wave-uniform (scalar registers)
  // and `lane_off` a loop-invariant per-lane byte offset, so the loads use
  // the scalar-base + vector-offset form and every tile's address is formed
  // with scalar arithmetic only. Load j of the lane covers 16*VB contiguous
  // bytes together with the other 15 lanes of its row.
  template <bool NT = false>
  __device__ static __forceinline__ void load(uint32_t (&w)[WPL], const char* base, uint32_t lane_off) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if constexpr (VB == 16) {
        const u32x4 x = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + lane_off + j * 16 * VB))
                           : *reinterpret_cast<const u32x4*>(base + lane_off + j * 16 * VB);
        w[j * 4 + 0] = x[0]; w[j * 4 + 1] = x[1]; w[j * 4 + 2] = x[2]; w[j * 4 + 3] = x[3];
      } else {
        const u32x2 x = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + lane_off + j * 16 * VB))
                           : *reinterpret_cast<const u32x2*>(base + lane_off + j * 16 * VB);
        w[j * 2 + 0] = x[0]; w[j * 2 + 1] = x[1];
      }
    }
  }

  __device__ static __forceinline__ float dot(const uint32_t (&q)[WPL], const uint32_t (&k)[WPL]) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      if constexpr (DT == Dt::F16)
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q[i]), __builtin_bit_cast(half2_t, k[i]), acc,
                                     false);
      else if constexpr (DT == Dt::BF16)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q[i]), __builtin_bit_cast(bf162_t, k[i]),
                                              acc, false);
      else
        acc = fmaf(__uint_as_float(q[i]), __uint_as_float(k[i]), acc);
    }
    return acc;
  }

  // acc[k] += p * v[k]
  __device__ static __forceinline__ void axpy(float (&acc)[EPL], float p, const uint32_t (&v)[WPL]) {
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      if constexpr (EPW == 2) {
        acc[2 * i] = fmaf(p, widen_lo<DT>(v[i]), acc[2 * i]);
        acc[2 * i + 1] = fmaf(p, widen_hi<DT>(v[i]), acc[2 * i + 1]);
      } else {
        acc[i] = fmaf(p, __uint_as_float(v[i]), acc[i]);
      }
    }
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax state of one 16-lane row of a wave.
template <int EPL> struct Soft {
  float m;
  float l;
  float acc[EPL];
};

// Consume one 16-token tile: token 4*j + g of the tile is in K[j]/V[j].
template <Dt DT, int D>
__device__ __forceinline__ void consume_tile(Soft<D / 16>& st, const uint32_t (&qw)[Lane<DT, D>::WPL],
                                             const uint32_t (&kw)[4][Lane<DT, D>::WPL],
                                             const uint32_t (&vw)[4][Lane<DT, D>::WPL], int t0, int ctx, int g,
                                             float scale_log2) {
  using L = Lane<DT, D>;
  float s[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s[j] = row16_sum(L::dot(qw, kw[j])) * scale_log2;
  const bool partial = t0 + 16 > ctx;
  bool valid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    valid[j] = !partial || (t0 + 4 * j + g < ctx);
    s[j] = valid[j] ? s[j] : -INFINITY;
  }
  const float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  const float m_new = fmaxf(st.m, mt);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = fast_exp2(st.m - m_use);
  float p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = fast_exp2(s[j] - m_use);
  st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
  for (int k = 0; k < L::EPL; ++k) st.acc[k] *= alpha;
  // Slots past the context may hold anything (even NaN): select zeros for
  // them instead of multiplying (0 * NaN would poison the sum). Selects on
  // every tile, not a branch for the last one, keep the instruction stream
  // straight so the compiler's load-wait counts stay exact.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t vz[L::WPL];
#pragma unroll
    for (int i = 0; i < L::WPL; ++i) vz[i] = valid[j] ? vw[j][i] : 0u;
    L::axpy(st.acc, p[j], vz);
  }
  st.m = m_new;
}

template <Dt DT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x, int out_f32) {
  if (out_f32 || DT == Dt::F32) {
    reinterpret_cast<float*>(out)[idx] = x;
  } else {
    const uint32_t b = DT == Dt::F16 ? f32_to_f16_bits(x) : f32_to_bf16_bits(x);
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)b;
  }
}

// Row r of the prefill-row mode is query j of chunk s: its causal context is
// ctx[s] - L_s + j + 1 tokens of sequence s.
__device__ __forceinline__ void prefill_row(const int32_t* qsl, const int32_t* ctx_lens, int S, int r, int& seq,
                                            int& ctx) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= r) lo = mid; else hi = mid - 1;
  }
  seq = lo;
  const int L = qsl[lo + 1] - qsl[lo];
  ctx = ctx_lens[lo] - L + (r - qsl[lo]) + 1;
}

// Group g of a prefix-sharing batch is rows group_starts[g] .. group_starts[g+1]-1.
__device__ __forceinline__ int group_of_row(const int32_t* group_starts, int num_groups, int r) {
  int lo = 0, hi = num_groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (group_starts[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Partition layout of one row: own partitions cover tokens [tok0, ctx) in
// part_tiles-tile steps and sit in workspace slots poff, poff+1, ...; a row
// of a prefix-sharing group has ceil(prefix / partition) shared partitions
// (written by the shared-prefix kernel) in slots 0 .. poff-1.
struct RowParts {
  int tok0, own, poff;
  __device__ __forceinline__ int total() const { return poff + own; }
};
template <RowMode MODE>
__device__ __forceinline__ RowParts row_parts(const DecodeArgs& a, int row, int ctx) {
  RowParts rp{0, 0, 0};
  if constexpr (MODE == RowMode::SharedTail) {
    // the prefix is whole tiles inside the row (clamped so that a prefix
    // longer than the row can never send a read past the row's blocks)
    const int p = min(a.prefix_lens[group_of_row(a.group_starts, a.num_groups, row)], ctx) & ~15;
    const int pt = a.part_tiles * 16;
    rp.tok0 = p;
    rp.poff = (p + pt - 1) / pt;
  }
  const int own_tiles = ((ctx + 15) >> 4) - (rp.tok0 >> 4);
  rp.own = (own_tiles + a.part_tiles - 1) / a.part_tiles;
  return rp;
}

}  // namespace

template <Dt DT, int D, int BS, int HG, RowMode MODE>
__global__ __launch_bounds__(HG * 64, PA_DECODE_MIN_WAVES) void decode_partition_kernel(const DecodeArgs a) {
  using L = Lane<DT, D>;
  constexpr int WPL = L::WPL;
  // a 16-token tile lies in one block (BS >= 16) or in two (BS == 8)
  constexpr int TPB = BS >= 16 ? BS / 16 : 1;  // tiles per block

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int g = lane >> 4;
  const int c = lane & 15;

  // grid: partition-major, then row, then head group; wave w takes head hg*HG + w
  const int n_hg = (a.H + HG - 1) / HG;
  int bid = blockIdx.x;
  const int hg = bid % n_hg;
  bid /= n_hg;
  const int row = bid % a.num_rows;
  const int part = bid / a.num_rows;
  const int h = hg * HG + wave;
  if (h >= a.H) return;

  int seq, ctx;
  if constexpr (MODE == RowMode::PrefillRows) {
    prefill_row(a.query_start_loc, a.context_lens, a.num_seqs, row, seq, ctx);
  } else {
    seq = row;
    ctx = a.context_lens[row];
  }
  const int n_tiles = (ctx + 15) >> 4;
  const RowParts rp = row_parts<MODE>(a, row, ctx);
  // partition 0 of an empty row still runs (it writes zeros), except for the
  // tail of a shared prefix that covers the whole row
  if (part >= (rp.own > 0 ? rp.own : (rp.poff > 0 ? 0 : 1))) return;

  const int u0 = (rp.tok0 >> 4) + part * a.part_tiles;
  const int my_tiles = max(0, min(n_tiles, u0 + a.part_tiles) - u0);

  uint32_t qw[WPL];
  L::load(qw, reinterpret_cast<const char*>(a.q) + ((int64_t)row * a.H + h) * L::ROW_BYTES, (uint32_t)(c * L::VB));

  Soft<L::EPL> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int k = 0; k < L::EPL; ++k) st.acc[k] = 0.f;

  const int32_t* bt_row = a.block_tables + (int64_t)seq * a.max_blocks;
  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);
  // row g of a 4-row group, lane chunk c
  const uint32_t lane_off = (uint32_t)(g * L::ROW_BYTES + c * L::VB);

  for (int base = 0; base < my_tiles; base += 64) {
    const int cnt = min(64, my_tiles - base);
    // table entries of tile u0 + base + lane (with 8-token blocks, the
    // second half of the tile is the next entry, read only if the sequence
    // has that block; otherwise its rows are past the context and masked)
    int32_t tb = 0, tb2 = 0;
    if (lane < cnt) {
      const int u = u0 + base + lane;
      if constexpr (BS >= 16) {
        tb = bt_row[u / TPB];
      } else {
        tb = bt_row[2 * u];
        tb2 = 2 * u + 1 < (ctx + 7) / 8 ? bt_row[2 * u + 1] : tb;
      }
    }

    // wave-uniform byte offsets of tile i's rows 0-7 and 8-15 (K and V share them)
    struct TileOff { int64_t lo, hi; };
    auto tile_off = [&](int i, int& t0) -> TileOff {
      const int u = u0 + base + i;
      t0 = u * 16;
      const int64_t lo = kv_row_offset(__builtin_amdgcn_readlane(tb, i), h, (u % TPB) * 16, a.H, BS, D) * L::EB;
      if constexpr (BS >= 16) return {lo, lo + 8 * L::ROW_BYTES};
      else return {lo, kv_row_offset(__builtin_amdgcn_readlane(tb2, i), h, 0, a.H, BS, D) * L::EB};
    };
    auto load_tile = [&](uint32_t (&kw)[4][WPL], uint32_t (&vw)[4][WPL], TileOff off) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        L::template load<true>(kw[j], kc + (j < 2 ? off.lo : off.hi) + (j & 1) * 4 * L::ROW_BYTES, lane_off);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        L::template load<true>(vw[j], vc + (j < 2 ? off.lo : off.hi) + (j & 1) * 4 * L::ROW_BYTES, lane_off);
      // keep the loads issued here, ahead of the other buffer's math
      __builtin_amdgcn_sched_barrier(0);
    };

    // Two register buffers, next tile always in flight. The steady-state
    // loop body has no branch, so the compiler's wait counts stay exact and
    // never drain the load queue; the last one or two tiles are finished
    // after it, so every tile is fetched exactly once.
    uint32_t ka[4][WPL], va[4][WPL], kb[4][WPL], vb[4][WPL];
    int ta, tb0;
    load_tile(ka, va, tile_off(0, ta));
    int i = 0;
    for (; i + 2 < cnt; i += 2) {
      load_tile(kb, vb, tile_off(i + 1, tb0));
      consume_tile<DT, D>(st, qw, ka, va, ta, ctx, g, a.scale_log2);
      load_tile(ka, va, tile_off(i + 2, ta));
      consume_tile<DT, D>(st, qw, kb, vb, tb0, ctx, g, a.scale_log2);
    }
    if (i + 1 < cnt) {
      load_tile(kb, vb, tile_off(i + 1, tb0));
      consume_tile<DT, D>(st, qw, ka, va, ta, ctx, g, a.scale_log2);
      consume_tile<DT, D>(st, qw, kb, vb, tb0, ctx, g, a.scale_log2);
    } else {
      consume_tile<DT, D>(st, qw, ka, va, ta, ctx, g, a.scale_log2);
    }
  }

  // merge the four 16-lane rows of the wave (same lane column c)
  float m_all = fmaxf(st.m, shfl_xor_f(st.m, 16));
  m_all = fmaxf(m_all, shfl_xor_f(m_all, 32));
  {
    const float f = fast_exp2(st.m - (m_all == -INFINITY ? 0.f : m_all));
    float lw = st.l * f;
    lw += shfl_xor_f(lw, 16);
    lw += shfl_xor_f(lw, 32);
    st.l = lw;
#pragma unroll
    for (int k = 0; k < L::EPL; ++k) {
      float x = st.acc[k] * f;
      x += shfl_xor_f(x, 16);
      x += shfl_xor_f(x, 32);
      st.acc[k] = x;
    }
    st.m = m_all;
  }
  if (g != 0) return;

  const int64_t orow = ((int64_t)row * a.H + h) * D;
  if (rp.total() <= 1) {
#pragma unroll
    for (int k = 0; k < L::EPL; ++k) {
      const float o = st.l > 0.f ? st.acc[k] / st.l : 0.f;
      store_out<DT>(a.out, orow + L::elem(c, k), o, a.out_f32);
    }
  } else {
    const int64_t prow = ((int64_t)row * a.H + h) * a.ws_parts + rp.poff + part;
    float* acc_out = a.ws + prow * D;
#pragma unroll
    for (int k = 0; k < L::EPL; ++k) acc_out[L::elem(c, k)] = st.acc[k];
    if (c == 0) {
      float* ml = a.ws + (int64_t)a.num_rows * a.H * a.ws_parts * D + prow * 2;
      ml[0] = st.m;
      ml[1] = st.l;
    }
  }
}

// K3: merge the partitions of rows that have more than one. One wave per
// (row, head); lane e handles elements e, e + 64, ...
template <Dt DT, int D, RowMode MODE>
__global__ __launch_bounds__(64) void decode_reduce_kernel(const DecodeArgs a) {
  const int row = blockIdx.x / a.H;
  const int h = blockIdx.x % a.H;
  const int ctx = a.context_lens[row];
  const int nparts = row_parts<MODE>(a, row, ctx).total();
  if (nparts <= 1) return;
  const int lane = threadIdx.x;
  const int64_t prow = ((int64_t)row * a.H + h) * a.ws_parts;
  const float* ml = a.ws + (int64_t)a.num_rows * a.H * a.ws_parts * D + prow * 2;
  const float* acc = a.ws + prow * D;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  float Lsum = 0.f;
  for (int p = 0; p < nparts; ++p) Lsum += ml[2 * p + 1] * fast_exp2(ml[2 * p] - M);
  constexpr int PER = D / 64;
  float x[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) x[i] = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = fast_exp2(ml[2 * p] - M);
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] += acc[(int64_t)p * D + lane + 64 * i] * w;
  }
  const int64_t orow = ((int64_t)row * a.H + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) store_out<DT>(a.out, orow + lane + 64 * i, x[i] / Lsum, a.out_f32);
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
    case RowMode::PrefillRows: return dispatch_k2<DT, RowMode::PrefillRows>(a, D, BS, stream);
    case RowMode::SharedTail: return dispatch_k2<DT, RowMode::SharedTail>(a, D, BS, stream);
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
  const int64_t grid = (int64_t)a.num_rows * a.H;
  if (grid == 0) return hipSuccess;
  if (shared)
    hipLaunchKernelGGL((decode_reduce_kernel<DT, D, RowMode::SharedTail>), dim3((unsigned)grid), dim3(64), 0, stream,
                       a);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<DT, D, RowMode::Decode>), dim3((unsigned)grid), dim3(64), 0, stream, a);
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
