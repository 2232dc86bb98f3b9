// Device-side building blocks of paged decode, shared by the decode kernels
// (partition, reduction) and the shared-prefix step kernel: the lane
// mapping of a token row onto a 16-lane DPP row, the per-row online
// softmax, row layouts of each row mode and the partition kernel's body.
// Included by pa_decode.hip and pa_shared.hip only.
#pragma once

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

  // the lane's words of one row written back in the layout load() reads
  __device__ static __forceinline__ void store(const uint32_t (&w)[WPL], char* base, uint32_t lane_off) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if constexpr (VB == 16)
        *reinterpret_cast<u32x4*>(base + lane_off + j * 16 * VB) = u32x4{w[j * 4], w[j * 4 + 1], w[j * 4 + 2], w[j * 4 + 3]};
      else
        *reinterpret_cast<u32x2*>(base + lane_off + j * 16 * VB) = u32x2{w[j * 2], w[j * 2 + 1]};
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

// Context length of row r (decode and shared-tail modes), clamped.
__device__ __forceinline__ int row_ctx(const DecodeArgs& a, int r) { return clamp_len(a.context_lens[r], a.max_ctx); }

// Group g of a prefix-sharing batch is rows group_starts[g] .. group_starts[g+1]-1.
// The starts are non-decreasing from group_starts[0] = 0, so the group is
// the number of starts g >= 1 at or before row r. The wave counts them 64 at
// a time (lane i reads start g0 + i, one ballot): one memory round trip for
// up to 65 groups, where a binary search chains log2(groups) loads.
// Called by whole waves (every lane active).
__device__ __forceinline__ int group_of_row(const int32_t* group_starts, int num_groups, int r) {
  const int lane = __lane_id();
  int cnt = 0;
  for (int g0 = 1; g0 < num_groups; g0 += 64) {
    const int g = g0 + lane;
    const bool before = g < num_groups && group_starts[min(g, num_groups - 1)] <= r;
    cnt += __popcll(__ballot(before));
  }
  return cnt;
}

// Shared tokens of group g, the same value in every kernel that walks the
// group: prefix_lens[g], clamped to the shortest member's context (a longer
// prefix breaks the call's precondition; with the clamp every member still
// owns the shared range, reads stay inside the members' blocks and the
// kernels agree on which partitions exist), rounded down to whole 16-token
// tiles. Called by whole waves (every lane active).
__device__ __forceinline__ int group_prefix(const DecodeArgs& a, int g) {
  const int lane = __lane_id();
  const int r0 = min(max(a.group_starts[g], 0), a.num_rows);
  const int r1 = min(max(a.group_starts[g + 1], r0), a.num_rows);
  int p = a.prefix_lens[g];
  for (int r = r0 + lane; r < r1; r += 64) p = min(p, row_ctx(a, r));
  return max(wave_min_i(p), 0) & ~15;
}

// group_prefix(a, group_of_row(...)) for row r in a single dependent
// memory round trip when there are at most 63 groups: lane i reads
// group_starts[i], prefix_lens[i] and the length of row r - 31 + i at once,
// so the group's start, end and requested prefix come out of registers once
// the ballot has found the group, and so do the members' lengths whenever
// the group lies within those 64 rows (always for groups of up to 32 rows);
// otherwise they are read after it. Same result as the general path.
// Called by whole waves (every lane active).
__device__ __forceinline__ int row_group_prefix(const DecodeArgs& a, int r) {
  if (a.num_groups < 1 || a.num_groups > 63) return group_prefix(a, group_of_row(a.group_starts, a.num_groups, r));
  const int lane = __lane_id();
  const int gs = a.group_starts[min(lane, a.num_groups)];
  const int pl = a.prefix_lens[min(lane, a.num_groups - 1)];
  const int w = r - 31 + lane;  // a window of rows around r
  const int cw = w >= 0 && w < a.num_rows ? row_ctx(a, w) : 0;
  const int g = __popcll(__ballot(lane >= 1 && lane < a.num_groups && gs <= r));
  const int r0 = min(max(__builtin_amdgcn_readlane(gs, g), 0), a.num_rows);
  const int r1 = min(max(__builtin_amdgcn_readlane(gs, g + 1), r0), a.num_rows);
  int p = __builtin_amdgcn_readlane(pl, g);
  if (r0 >= r - 31 && r1 <= r + 33) {
    if (w >= r0 && w < r1) p = min(p, cw);
  } else {
    for (int m = r0 + lane; m < r1; m += 64) p = min(p, row_ctx(a, m));
  }
  return max(wave_min_i(p), 0) & ~15;
}

// Partition layout of one row: own partitions cover tokens [tok0, ctx) in
// part_tiles-tile steps and sit in workspace slots poff, poff+1, ...; a row
// of a prefix-sharing group has ceil(prefix / shared partition) shared
// partitions (written by the shared-prefix kernel) in slots 0 .. poff-1.
struct RowParts {
  int tok0, own, poff;
  __device__ __forceinline__ int total() const { return poff + own; }
};
template <RowMode MODE>
__device__ __forceinline__ RowParts row_parts(const DecodeArgs& a, int row, int ctx) {
  RowParts rp{0, 0, 0};
  if constexpr (MODE == RowMode::SharedTail) {
    const int p = row_group_prefix(a, row);
    const int pt = a.shared_part_tiles * 16;
    rp.tok0 = p;
    rp.poff = (p + pt - 1) / pt;
  }
  rp.own = own_partitions(ctx, rp.tok0, a.part_tiles);
  return rp;
}

}  // namespace

// Body of the partition kernel for workgroup `bid` (wave `wave` of HG takes
// head hg*HG + wave); shared by the partition kernel and the shared-prefix
// step kernel.
template <Dt DT, int D, int BS, int HG, RowMode MODE>
__device__ __forceinline__ void decode_partition_body(const DecodeArgs& a, int bid, int wave) {
  using L = Lane<DT, D>;
  constexpr int WPL = L::WPL;
  // a 16-token tile lies in one block (BS >= 16) or in two (BS == 8)
  constexpr int TPB = BS >= 16 ? BS / 16 : 1;  // tiles per block

  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c = lane & 15;

  // grid: partition-major, then row, then head group; wave w takes head hg*HG + w
  const int n_hg = (a.H + HG - 1) / HG;
  const int hg = bid % n_hg;
  bid /= n_hg;
  const int row = bid % a.num_rows;
  const int part = bid / a.num_rows;
  const int h = hg * HG + wave;
  if (h >= a.H) return;

  const int seq = row;
  const int ctx = row_ctx(a, row);
  const int n_tiles = (ctx + 15) >> 4;
  const RowParts rp = row_parts<MODE>(a, row, ctx);
  // partition 0 of an empty row still runs (it writes zeros), except for the
  // tail of a shared prefix that covers the whole row
  if (part >= (rp.own > 0 ? rp.own : (rp.poff > 0 ? 0 : 1))) return;

  const int u0 = (rp.tok0 >> 4) + part * a.part_tiles;
  const int my_tiles = max(0, min(n_tiles, u0 + a.part_tiles) - u0);

  // Fused cache write (decode rows, new_k set): row `row`'s new token sits at
  // position ctx - 1, in the final tile of the row's last partition. That
  // partition's wave fetches the token's K and V rows from new_k/new_v into
  // LDS right behind its first tile (DMA: no registers held across the tile
  // loop, the fetch is long done when the final tile comes, and the slot
  // read that decides it waits behind the table and tile loads, not in front
  // of them) and uses them in place of the final tile's cache row, so no
  // other kernel has to run first. The slot itself (padding slots and slots
  // past the pool are skipped, and the row then reads the cache as it is) is
  // written by the reduction kernel when one follows: a store in this
  // read-bound kernel costs far more than its bytes (an extra 512 B per wave
  // measured ~10 us over 8k waves). Without a reduction the wave stores
  // them itself, after its output.
  // K row at [0, ROW_BYTES), V row at [1024, 1024 + ROW_BYTES) of the wave's
  // 2 KiB; the rest of each KiB takes the DMA's unused lanes
  __shared__ __align__(16) uint8_t ntok[MODE == RowMode::Decode ? HG : 1][2048];
  static_assert(L::ROW_BYTES <= 1024, "a row fits one DMA");
  bool last_part = false;
  if constexpr (MODE == RowMode::Decode) last_part = a.new_k != nullptr && part == max(rp.own, 1) - 1;
  // The slot, read unconditionally (another row-indexed array stands in when
  // there is no slot to read) with a vector load: a scalar load would be
  // waited for together with the kernel arguments, ahead of the table and
  // tile loads; a vector load is done by the time the table entries are.
  int32_t slot_v;
  {
    int32_t zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    slot_v = (last_part ? a.slot_mapping + row : a.context_lens + row)[zero];
  }
  // the slot at the point of use (what is computed from it is not hoisted
  // ahead of the loads issued before that point)
  auto slot_here = [&]() {
    int32_t v = slot_v;
    asm volatile("" : "+v"(v));
    return __builtin_amdgcn_readfirstlane(v);
  };
  auto fused = [&]() {
    const int32_t sl = slot_here();
    return last_part && sl >= 0 && sl < a.num_blocks * BS;
  };
  auto fetch_new_token = [&]() {
    const int64_t new_src = ((int64_t)row * a.H + h) * L::ROW_BYTES;
    const uint32_t voff = (uint32_t)((lane * 16) % L::ROW_BYTES);
    const uint32_t lds = lds_offset(&ntok[wave][0]);
    lds_dma16s(reinterpret_cast<const char*>(a.new_k) + new_src, voff, lds);
    lds_dma16s(reinterpret_cast<const char*>(a.new_v) + new_src, voff, lds + 1024);
  };
  // the lane's words of the new token's K or V row (in the lane layout of a
  // tile row), out of LDS
  auto token_words = [&](uint32_t (&w)[WPL], int kv) {
    const uint8_t* const src = &ntok[wave][kv * 1024];
#pragma unroll
    for (int j = 0; j < L::NV; ++j)
#pragma unroll
      for (int x = 0; x < L::VW; ++x)
        w[j * L::VW + x] = *reinterpret_cast<const uint32_t*>(src + c * L::VB + j * 16 * L::VB + 4 * x);
  };
  // The token's rows, once every earlier load (the DMA among them) is done;
  // the caller needs the last tile's loads next anyway.
  auto new_token = [&](uint32_t (&nk)[WPL], uint32_t (&nv)[WPL]) {
    wait_vmcnt0();
    token_words(nk, 0);
    token_words(nv, 1);
  };
  // Row group 0 stores the token into its slot as the wave's last act: the
  // compiler counts stores with the loads, so a store ahead of the tile
  // math would make the wave wait for its write to complete.
  auto store_new_token = [&]() {
    uint32_t w[WPL];
    const int32_t sl = slot_here();
    const int64_t dst = kv_row_offset(sl / BS, h, sl % BS, a.H, BS, D) * L::EB;
    const uint32_t lo = (uint32_t)(c * L::VB);
    token_words(w, 0);
    L::store(w, const_cast<char*>(reinterpret_cast<const char*>(a.k_cache)) + dst, lo);
    token_words(w, 1);
    L::store(w, const_cast<char*>(reinterpret_cast<const char*>(a.v_cache)) + dst, lo);
  };
  // the final tile's row (ctx - 1) % 16 is held by load j = r / 4 of the
  // lanes of row group r % 4: they take the new token's words instead. The
  // token is read into the first row of the other, already consumed buffer
  // (no registers beyond the two tile buffers).
  auto fuse_tile = [&](uint32_t (&kw)[4][WPL], uint32_t (&vw)[4][WPL], uint32_t (&nk)[WPL], uint32_t (&nv)[WPL]) {
    new_token(nk, nv);
    const int r = (ctx - 1) & 15;
    const bool mine = g == (r & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < WPL; ++w) {
        kw[j][w] = (mine && j == (r >> 2)) ? nk[w] : kw[j][w];
        vw[j][w] = (mine && j == (r >> 2)) ? nv[w] : vw[j][w];
      }
  };
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
        tb = clamp_block(bt_row[u / TPB], a.num_blocks);
      } else {
        tb = clamp_block(bt_row[2 * u], a.num_blocks);
        tb2 = 2 * u + 1 < (ctx + 7) / 8 ? clamp_block(bt_row[2 * u + 1], a.num_blocks) : tb;
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
    if (fused() && base == 0) fetch_new_token();
    int i = 0;
    for (; i + 2 < cnt; i += 2) {
      load_tile(kb, vb, tile_off(i + 1, tb0));
      consume_tile<DT, D>(st, qw, ka, va, ta, ctx, g, a.scale_log2);
      load_tile(ka, va, tile_off(i + 2, ta));
      consume_tile<DT, D>(st, qw, kb, vb, tb0, ctx, g, a.scale_log2);
    }
    const bool fuse_here = fused() && base + 64 >= my_tiles;  // this chunk ends with the row's final tile
    if (i + 1 < cnt) {
      load_tile(kb, vb, tile_off(i + 1, tb0));
      consume_tile<DT, D>(st, qw, ka, va, ta, ctx, g, a.scale_log2);
      if (fuse_here) fuse_tile(kb, vb, ka[0], va[0]);
      consume_tile<DT, D>(st, qw, kb, vb, tb0, ctx, g, a.scale_log2);
    } else {
      if (fuse_here) fuse_tile(ka, va, kb[0], vb[0]);
      consume_tile<DT, D>(st, qw, ka, va, ta, ctx, g, a.scale_log2);
    }
  }
  if (fused() && my_tiles == 0 && !a.write_in_reduce) {  // an empty context still has its token written
    fetch_new_token();
    wait_vmcnt0();
  }

  // merge the four 16-lane rows of the wave (same lane column c) with the
  // row-swap instructions (VALU, no LDS round trip)
  const float m_all = rows4_max(st.m);
  {
    const float f = fast_exp2(st.m - (m_all == -INFINITY ? 0.f : m_all));
    st.l = rows4_sum(st.l * f);
#pragma unroll
    for (int k = 0; k < L::EPL; ++k) st.acc[k] = rows4_sum(st.acc[k] * f);
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
  if (fused() && !a.write_in_reduce) store_new_token();
}

}  // namespace pa
