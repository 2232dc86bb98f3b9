// Causal prefill of multi-token query chunks over the paged cache, on MFMA.
//
// A chunk of L new tokens of a sequence attends to the sequence's cached
// tokens through its block table (devpress.csdn.net page, sections on how
// PagedAttention works and on the paged KV cache; betteryeah.com page,
// section 2.4); the chunk's own K/V are already cached and it is the last L
// of ctx tokens, so query j (position ctx-L+j) sees tokens 0..ctx-L+j.
//
// With many queries per key this is a dense contraction, so it runs on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulate).
// Orientation: the wave computes S^T = K Q^T (keys on the MFMA rows, its
// queries on the columns) and O^T += V^T P^T. In that orientation the
// score accumulator a lane holds (one query, four keys per 16-key subtile)
// is exactly the B operand P^T needs, so P never leaves registers; the V^T
// operand comes from LDS through transposing reads. Per tile of KT keys:
//   * the tile's K and V rows travel from global memory straight into LDS
//     (global_load_lds_dwordx4: each wave moves 1 KiB pieces, lane L's 16
//     bytes landing at the piece base + 16 L), three buffers deep, so tile
//     t+2 is in flight while tile t is computed; one barrier per tile. The
//     rows of a piece lie in one block, so each piece's block id is read
//     with a scalar load (issued before the barrier, whose wait hides its
//     latency) and the source address is that block's row, in SGPRs, plus
//     a fixed per-lane offset; the tile loop is unrolled three times, so
//     every LDS offset is an immediate;
//   * tiles are row-major with the 16-byte chunks XOR-swizzled per row, so
//     the K fragment reads and the V^T reads (ds_read_b64_tr_b16, which
//     turns 4 key rows x 16 dims around per 16 lanes) use every bank once;
//   * only the last tile is clamped (its rows past the context read the
//     last block) and has its V rows past the context zeroed in LDS;
//   * each wave owns NQ groups of 16 queries (two in the standard shape, one
//     in the wide shape, below); every K or V^T fragment read from LDS
//     feeds one MFMA per group;
//   * online softmax per query: the max over the raw scores (the scale is
//     applied once to it, and inside the exponent's FMA), cross-row max on
//     the row-swap instructions (both query groups folded together), P
//     narrowed with the packed converts; each lane sums the rounded P of
//     its own keys into the denominator with packed dot2 against (1, 1),
//     and the four lanes of a query add their sums at the end;
//     only tiles that cross a wave's first query carry the causal mask (the
//     masked scores are set to -inf), tiles past its last query are skipped, and
//     the running max is raised lazily (see compute()) so the accumulators
//     are rescaled, and the cross-row max taken, only on the few tiles that
//     need it.
// P is rounded to the input type for the P.V product; for bf16 it is split
// into a bf16 head and a bf16 remainder (two MFMAs) to keep ~16 bits. A
// negative scale is applied as |scale| on negated queries (exact: a sign
// flip), so the max of the raw scores is the max of the scaled ones.
#include "pa_grid.h"
#include "pa_internal.h"

#include <type_traits>
#include <utility>

namespace pa {

namespace {

#ifndef PA_PREFILL_KT
#define PA_PREFILL_KT 32
#endif
constexpr int KT = PA_PREFILL_KT;  // keys per tile (32 or 64)
// Workgroup shapes: NW waves, NQ 16-query groups per wave, every shape
// covering QT queries per workgroup. The standard shape (4 waves x 32
// queries, three waves per SIMD) reads each K or V^T fragment from LDS once
// for two MFMAs, the best rate when there are more workgroups than the chip
// holds at once. The wide shape (8 waves x 16 queries, head dim 128 only)
// halves each wave's dependent chain per tile (half the MFMAs and
// exponentials, four waves per SIMD) at twice the LDS reads per MFMA; it
// shortens the longest query tiles when every workgroup is resident at once.
template <int D, bool WIDE> struct PfShape {
  static constexpr bool W = WIDE && D == 128;
  static constexpr int NW = W ? 8 : 4;
  static constexpr int NQ = W ? 1 : 2;
  static constexpr int QW = 16 * NQ;  // queries per wave
  static constexpr int QT = NW * QW;  // queries per workgroup
  static constexpr int WAVES = W ? 4 : 3;  // waves per SIMD the registers must allow
};
constexpr int QT = PfShape<128, false>::QT;
static_assert(PfShape<64, false>::QT == QT && PfShape<128, true>::QT == QT, "one query tile for every shape");
#ifndef PA_PREFILL_NBUF
#define PA_PREFILL_NBUF 3
#endif
constexpr int NBUF = PA_PREFILL_NBUF;  // LDS buffers per operand: tile t computed while t+1 .. t+NBUF-1 land
static_assert(NBUF >= 2, "at least one tile in flight");
constexpr float RESCALE_LOG2 = 8.f; // lazy rescale threshold (log2 units): p < 256 between rescales
static_assert(KT == 32, "key tile of 32");

// max without the NaN-quieting the compiler adds around values of unknown
// origin (the scores are never signalling NaNs); the wait states let a
// following v_permlane read the result
__device__ __forceinline__ float vmax_nc(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2\n\ts_nop 1" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Row maxima of two values at once: afterwards every lane holds the max of
// a over the four lanes n16, n16+16, n16+32, n16+48, and the same for b.
// The first swap pairs a's odd rows with b's even rows, so one max folds
// both values' row pairs into one register; the row-pair swap folds the
// halves; the last swap hands a's result to every row of one register and
// b's to the other.
__device__ __forceinline__ void rows4_max2(float& a, float& b) {
  const auto s1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, a), __builtin_bit_cast(int, b), false, false);
  const float x = vmax_nc(__builtin_bit_cast(float, (int)s1[0]), __builtin_bit_cast(float, (int)s1[1]));
  const auto s2 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  const float y = vmax_nc(__builtin_bit_cast(float, (int)s2[0]), __builtin_bit_cast(float, (int)s2[1]));
  const auto s3 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, y), __builtin_bit_cast(int, y), false, false);
  a = __builtin_bit_cast(float, (int)s3[0]);
  b = __builtin_bit_cast(float, (int)s3[1]);
}
// Block ids through the scalar cache, as inline assembly: once the DMA
// assembly is in the kernel the compiler can no longer prove the table
// unchanged and would read it with vector loads, whose waits would drain
// the DMA queue. (Waits on lgkmcnt only: LDS and scalar loads.)
__device__ __forceinline__ void sload2(const int32_t* p0, const int32_t* p1, int32_t& v0, int32_t& v1) {
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(v0), "=&s"(v1) : "s"(p0), "s"(p1) : "memory");
}
// The top of a pipeline step: the scalar loads of the next DMA's block ids
// (PPW of them), the wait until at most VMCNT of this wave's DMA loads are
// outstanding (the tiles still in flight behind the one about to be
// computed), the workgroup barrier, then the wait for the scalar loads,
// whose latency thus hides behind the barrier.
template <int PPW, int VMCNT>
__device__ __forceinline__ void sload_barrier(const int32_t* const (&e)[PPW], int32_t (&v)[PPW]) {
  static_assert(PPW == 1 || PPW == 2, "one or two DMA pieces per wave");
  static_assert(VMCNT >= 0 && VMCNT <= 63, "vmcnt field");
  if constexpr (PPW == 2)
    asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt vmcnt(%4)\n\ts_barrier\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&s"(v[0]), "=&s"(v[1]) : "s"(e[0]), "s"(e[1]), "i"(VMCNT) : "memory");
  else
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt vmcnt(%2)\n\ts_barrier\n\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(v[0]) : "s"(e[0]), "i"(VMCNT) : "memory");
}
// f(integral_constant<int, B>) for B = 0, 1, ..., in order (an unrolled loop
// whose index is a compile-time constant in the body)
template <typename F, int... B>
__device__ __forceinline__ void for_each_const(F&& f, std::integer_sequence<int, B...>) {
  (f(std::integral_constant<int, B>{}), ...);
}
// c + the two 16-bit values of w times those of one2 (packed f16 or bf16)
template <Dt DT> __device__ __forceinline__ float dot2one(uint32_t w, uint32_t one2, float c) {
  if constexpr (DT == Dt::F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w), __builtin_bit_cast(half2_t, one2), c, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, w), __builtin_bit_cast(bf162_t, one2), c, false);
}

// Work item of this workgroup: sequence s, head h, query tile qt (of QT
// queries; key tiles of KTP keys price the items; PER_CU workgroups fit on
// a compute unit at once). False when the workgroup has none (padding of
// the grouped grid).
template <int KTP, int PER_CU>
__device__ __forceinline__ bool prefill_item(const PrefillArgs& a, int lane, int& s, int& h, int& qt) {
  // Work order. With more workgroups than fit on the chip at once: the
  // grouped order of pa_grid.h (every query tile of a pair on one XCD
  // together in the first round, the heaviest remaining tiles first after
  // it). Otherwise every workgroup is resident at once; the (sequence, query
  // tile) items are then taken heaviest first (priced from the lengths on
  // the device), and the rounds in which the workgroups reach the compute
  // units alternate direction, so heavy and light items share units.
  if (a.grouped) {
    const int pairs_p = (int)gridDim.x / a.q_tiles;  // pairs, padded to a multiple of 8
    int pair, qi;
    grouped_item(blockIdx.x, a.q_tiles, pairs_p, grouped_first_round_pairs(a.cus * PER_CU, a.q_tiles, pairs_p), pair,
                 qi);
    if (pair >= a.num_seqs * a.H) return false;
    h = pair % a.H;
    s = pair / a.H;
    qt = a.q_tiles - 1 - qi;
  } else {
    // Workgroups are handed to compute units in order, one per unit per
    // round (workgroup x, x + CUs, x + 2 CUs, ... share a unit). Every
    // other round runs backwards, so the unit that holds one of the
    // heaviest query tiles of the first round gets one of the lightest of
    // the second.
    int pos = blockIdx.x;
    if (a.cus > 0) {
      const int round = pos / a.cus, c = pos % a.cus;
      if ((round & 1) && (round + 1) * a.cus <= (int)gridDim.x) pos = round * a.cus + (a.cus - 1 - c);
    }
    const int rank = pos / a.H;
    h = pos % a.H;
    const int n_items = a.num_seqs * a.q_tiles;
    if (n_items <= 64) {
      // Lane i prices work item i (sequence i / q_tiles, query tile
      // i % q_tiles) at the key tiles its workgroup walks (0 when the chunk
      // has no such query tile); the grid takes items by decreasing price,
      // ties in index order, so the heaviest query tiles start first, one
      // per compute unit. (More items than lanes: the fixed order, latest
      // query tiles first.)
      int price = -1;
      if (lane < n_items) {
        const int si = lane / a.q_tiles, qi = lane % a.q_tiles;
        const ChunkRows r = chunk_rows(a.query_start_loc[si], a.query_start_loc[si + 1], a.context_lens[si],
                                       a.total_q, a.max_context_len);
        price = qi * QT < r.L ? (r.ctx - r.L + min((qi + 1) * QT, r.L) + KTP - 1) / KTP : 0;
      }
      int ahead = 0;  // items taken before item `lane`
      for (int j = 0; j < n_items; ++j) {
        const int pj = __builtin_amdgcn_readlane(price, j);
        ahead += (pj > price || (pj == price && j < lane)) ? 1 : 0;
      }
      const uint64_t hit = __ballot(lane < n_items && ahead == rank);
      const int item = hit ? (int)__builtin_ctzll(hit) : 0;  // exactly one lane holds each rank
      s = item / a.q_tiles;
      qt = item % a.q_tiles;
    } else {
      s = rank % a.num_seqs;
      qt = a.q_tiles - 1 - rank / a.num_seqs;
    }
  }
  return true;
}

}  // namespace

template <Dt DT, int D, int BS, bool WIDE>
__global__ __launch_bounds__((PfShape<D, WIDE>::NW * 64))
    __attribute__((amdgpu_waves_per_eu(PfShape<D, WIDE>::WAVES))) void prefill_mfma_kernel(const PrefillArgs a) {
  using Shape = PfShape<D, WIDE>;
  constexpr int NW = Shape::NW, NQ = Shape::NQ, QW = Shape::QW;
  constexpr int KS = D / 32;     // MFMA k-steps over head_dim for Q.K
  constexpr int NDT = D / 16;    // 16-row tiles of O^T
  constexpr int NSUB = KT / 16;  // 16-key subtiles of S^T
  constexpr int NKST = KT / 32;  // MFMA k-steps over keys for P.V
  constexpr int CPR = D / 8;     // 16-byte chunks per K/V row
  constexpr int ROWB = D * 2;    // bytes per K/V row
  constexpr int TILEB = KT * ROWB;       // bytes of one K (or V) tile in LDS
  constexpr int PR = 1024 / ROWB;        // rows per 1 KiB DMA piece (one wave-wide load)
  constexpr int PPW = TILEB / 1024 / NW;  // pieces per wave, per operand and tile
  static_assert(PR <= BS && BS % PR == 0, "the rows of one DMA piece lie in one block");
  static_assert(PPW >= 1, "every wave loads a piece of each tile");

  // K and V tiles row-major in LDS, unpadded; 16-byte chunk c of row r sits
  // at chunk position c ^ f(r), which spreads the MFMA operand reads over
  // all banks: K is read 16 rows at one chunk (f = r mod 16, or (r/2) mod 8
  // for 8-chunk rows), V^T by transposing reads of 4 rows x 2 chunks per
  // 16 lanes (f = 2r mod 16, or r & 6).
  __shared__ __align__(1024) uint8_t sk[NBUF][TILEB];
  __shared__ __align__(1024) uint8_t sv[NBUF][TILEB];
  auto fk = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto fv = [](int r) { return D == 128 ? ((2 * r) & 15) : (r & 6); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15;
  const int g4 = lane >> 4;

  int h, s, qt;
  if (!prefill_item<KT, kPrefillWorkgroupsPerCU>(a, lane, s, h, qt)) return;
  // lengths and row ranges clamped to what the host validated (in-range
  // values are unchanged): no read or write leaves the caller's buffers
  const ChunkRows cr =
      chunk_rows(a.query_start_loc[s], a.query_start_loc[s + 1], a.context_lens[s], a.total_q, a.max_context_len);
  const int ctx = cr.ctx, q_beg = cr.q_beg, L = cr.L;
  const int j0 = qt * QT;
  if (j0 >= L) return;
  const int c0 = ctx - L;                          // position of the chunk's first query
  const int kv_end = c0 + min(j0 + QT, L);         // keys this workgroup needs: [0, kv_end)
  const int n_tiles = (kv_end + KT - 1) / KT;
  const int wq0 = j0 + wave * QW;                  // the wave's first query (chunk-relative)
  const bool wave_active = wq0 < L;
  const int wave_last_pos = c0 + min(wq0 + QW, L) - 1;

  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks;
  const int nb = (kv_end + BS - 1) / BS;           // blocks this workgroup reads
  const uint32_t blk_bytes = (uint32_t)a.H * BS * ROWB;   // one block of every head (< 2^32)
  const uint32_t head_bytes = (uint32_t)h * BS * ROWB;

  // Q^T fragments (B operand of S^T = K Q^T): query n16 of group g, d = 32*ks + 8*g4 .. +7
  u32x4 qf[NQ][KS];
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    const int jq = wq0 + g * 16 + n16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (jq < L) {
        const char* p = reinterpret_cast<const char*>(a.q) + (((int64_t)(q_beg + jq) * a.H + h) * D + ks * 32 + 8 * g4) * 2;
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        qf[g][ks] = u32x4{v[0] ^ a.q_sign, v[1] ^ a.q_sign, v[2] ^ a.q_sign, v[3] ^ a.q_sign};
      } else {
        qf[g][ks] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // o: O^T of the wave's queries; lsum: this lane's share of the softmax
  // denominators (the sum of the rounded P of its keys, the same P the
  // numerator uses), added over the query's four lanes at the end
  f32x4 o[NQ][NDT];
  float m[NQ], lsum[NQ];
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    m[g] = -INFINITY;
    lsum[g] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[g][dt] = zero4();
  }
  constexpr uint32_t ONE2 = ones2<DT>();

  // DMA of one tile into LDS buffer b: piece p holds rows p*PR .. p*PR+PR-1
  // and wave w loads pieces w, w+4, ...; lane L of a piece fills chunk
  // position L % CPR of row L / CPR, i.e. source chunk (L % CPR) ^ f(row).
  // The swizzle terms repeat every 16 rows, so the per-lane source offsets
  // are the same for every piece and tile.
  const int prow = lane / CPR;
  const int pcol = lane % CPR;
  const uint32_t k_src = prow * ROWB + ((pcol ^ fk(wave * PR + prow)) * 16);
  const uint32_t v_src = prow * ROWB + ((pcol ^ fv(wave * PR + prow)) * 16);
  const uint32_t sk0 = lds_offset(&sk[0][0]);
  const uint32_t sv0 = lds_offset(&sv[0][0]);
  // block-table entry of piece i of tile t (clamped to the blocks read)
  auto entry = [&](int t, int i) {
    const uint32_t k = (uint32_t)(t * KT + (wave + NW * i) * PR);
    return bt_row + min(k / BS, (uint32_t)(nb - 1));
  };
  // DMA of tile t into buffer b given its pieces' block ids
  auto dma_ids = [&](int t, int b, const int (&phys)[PPW]) {
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int p = wave + NW * i;
      const uint32_t key = (uint32_t)(t * KT + p * PR);
      const uint64_t row =
          (uint64_t)(uint32_t)clamp_block(phys[i], a.num_blocks) * blk_bytes + (head_bytes + (key % BS) * ROWB);
      lds_dma16s(kc + row, k_src, sk0 + b * TILEB + p * 1024);
      lds_dma16s(vc + row, v_src, sv0 + b * TILEB + p * 1024);
    }
  };
  // rows at or past kv_end of the last tile: V rows become zeros (their
  // weights are zero, but the slots may hold anything, NaN included)
  auto zero_tail = [&](int t, int b) {
    const int r0 = kv_end - t * KT;
    for (int i = tid; i < (KT - r0) * CPR; i += NW * 64)
      *reinterpret_cast<u32x4*>(&sv[b][(r0 + i / CPR) * ROWB + (i % CPR) * 16]) = u32x4{0u, 0u, 0u, 0u};
  };
  // MFMA operand offsets (bytes inside a buffer): K fragment of k-step ks is
  // chunk 4 ks + g4 of row n16 (+16 rows per subtile); V^T fragment rows
  // come from keys 4 g4 + n16/4 (+16), dims 16 dt + 4 (n16 % 4).
  uint32_t k_rd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_rd[ks] = n16 * ROWB + (((4 * ks + g4) ^ fk(n16)) * 16);
  const int vkey = 4 * g4 + (n16 >> 2);
  // chunk 2 dt + (n16 % 4) / 2 of row vkey sits at (2 dt + a) ^ fv = 2 (dt ^ fv/2) + a: the dt term
  // enters by an XOR of dt << 5 into bits that are zero in the rest of the offset
  const uint32_t v_rd = vkey * ROWB + (((n16 & 3) >> 1) * 16) + 8 * (n16 & 1) + ((fv(vkey) >> 1) << 5);

  const float c = fmaxf(a.scale_log2, 1.17549435e-38f);
  // S^T = K Q^T of the tile in buffer b over NSUB key subtiles of 16
  auto qk = [&](auto bc, f32x4 (&sacc)[NQ][NSUB]) {
    constexpr int b = decltype(bc)::value;
#pragma unroll
    for (int g = 0; g < NQ; ++g)
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) sacc[g][sub] = zero4();
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(&sk[b][sub * 16 * ROWB + k_rd[ks]]);
#pragma unroll
        for (int g = 0; g < NQ; ++g) sacc[g][sub] = mfma16<DT>(ka, qf[g][ks], sacc[g][sub]);
      }
    }
  };
  // online softmax of the scores of keys kv0 .. kv0+KT-1 into the P^T
  // operands (pb, and the bf16 remainders pbl); lane holds query n16, keys
  // kv0 + 16*sub + 4*g4 + i.
  auto softmax = [&](f32x4 (&sacc)[NQ][NSUB], int kv0, u32x4 (&pb)[NQ][NKST], u32x4 (&pbl)[NQ][NKST]) {
    // Only tiles that reach past the wave's first query need the causal
    // mask (wave-uniform test). The running max is raised lazily: a row
    // keeps its reference max until a tile's max exceeds it by more than
    // 2^RESCALE_LOG2, so p = 2^(s - m) stays below 2^RESCALE_LOG2 and the
    // accumulators are rescaled only on the (rare) tiles where some row
    // needs it; the final O / l is the same softmax.
    const bool masked = kv0 + KT - 1 > c0 + wq0;
    if (masked) {  // keys past a query's position score -inf
#pragma unroll
      for (int g = 0; g < NQ; ++g) {
        const int last_key = min(c0 + wq0 + g * 16 + n16, kv_end - 1);
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kv0 + 16 * sub + 4 * g4 + i > last_key) sacc[g][sub][i] = -INFINITY;
      }
    }
    static_assert(NQ == 1 || NQ == 2, "one or two query groups per wave");
    float mrow[NQ];  // max of the raw scores (c > 0: the scaled max is mr * c)
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
      float mr = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) mr = fmaxf(mr, sacc[g][sub][i]);
      mrow[g] = mr;
    }
    // A row's max exceeds its reference by more than 2^RESCALE_LOG2 exactly
    // when one of its four lanes' maxima does (the row's lanes share m, and
    // x -> x * c is monotonic), so a lane-local test decides; the cross-row
    // max runs only on the tiles that raise some row (the first one, m =
    // -inf, and the rare jumps), and those take the same decisions as before.
    bool jump = false;
#pragma unroll
    for (int g = 0; g < NQ; ++g) jump |= mrow[g] * c > m[g] + RESCALE_LOG2;
    if (__any(jump)) {
      if constexpr (NQ == 2) rows4_max2(mrow[0], mrow[1]);
      else mrow[0] = rows4_max(mrow[0]);
#pragma unroll
      for (int g = 0; g < NQ; ++g) {
        const float mt = mrow[g] * c;
        const bool grow = mt > m[g] + RESCALE_LOG2;
        if (__any(grow)) {
          const float m_new = grow ? mt : m[g];
          const float alpha = __builtin_amdgcn_exp2f(m[g] - m_new);
          lsum[g] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[g][dt] *= alpha;
          m[g] = m_new;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
      const float neg_m = m[g] == -INFINITY ? 0.f : -m[g];
      float p[4 * NSUB];
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[4 * sub + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[g][sub][i], c, neg_m));
      // B operand of O^T += V^T P^T for key step kst: elements 0..3 from
      // subtile 2*kst, 4..7 from subtile 2*kst+1
#pragma unroll
      for (int kst = 0; kst < NKST; ++kst) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack2<DT>(p[8 * kst + 2 * j], p[8 * kst + 2 * j + 1]);
        pb[g][kst] = u32x4{w[0], w[1], w[2], w[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) lsum[g] = dot2one<DT>(w[j], ONE2, lsum[g]);
        if constexpr (DT == Dt::BF16) {
          uint32_t r[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            r[j] = pack2<DT>(p[8 * kst + 2 * j] - __uint_as_float(w[j] << 16),
                             p[8 * kst + 2 * j + 1] - __uint_as_float(w[j] & 0xffff0000u));
          pbl[g][kst] = u32x4{r[0], r[1], r[2], r[3]};
#pragma unroll
          for (int j = 0; j < 4; ++j) lsum[g] = dot2one<DT>(r[j], ONE2, lsum[g]);
        }
      }
    }
  };
  // O^T += V^T P^T with the V tile in buffer b: A = V^T rows d = 16*dt + n16, keys 4*g4 + {0..3} and
  // 16 + 4*g4 + {0..3}, two transposing 8-byte LDS reads (each 16 lanes turn 4 key rows x 16 dims around)
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  auto vt_frag = [&](auto bc, int dt) -> u32x4 {
    constexpr int b = decltype(bc)::value;
    const uint8_t* vb = &sv[b][0];
    const uint32_t off = v_rd ^ (dt << 5);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) void*)(vb + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) void*)(vb + off + 16 * ROWB));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };
  auto pv = [&](auto bc, const u32x4 (&pb)[NQ][NKST], const u32x4 (&pbl)[NQ][NKST], const u32x4 va0) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x4 va = dt == 0 ? va0 : vt_frag(bc, dt);
#pragma unroll
      for (int g = 0; g < NQ; ++g) {
        o[g][dt] = mfma16<DT>(va, pb[g][0], o[g][dt]);
        if constexpr (DT == Dt::BF16) o[g][dt] = mfma16<DT>(va, pbl[g][0], o[g][dt]);
      }
    }
  };
  auto compute = [&](auto bc, int kv0) {
    f32x4 sacc[NQ][NSUB];
    u32x4 pb[NQ][NKST], pbl[NQ][NKST];
    qk(bc, sacc);
    const u32x4 va0 = vt_frag(bc, 0);  // read ahead: its LDS latency hides under the softmax
    softmax(sacc, kv0, pb, pbl);
    pv(bc, pb, pbl, va0);
  };

  // Pipeline over tiles with three LDS buffers: tile t+2's DMA is issued
  // while tile t is computed (tile t+1's is in flight). Each iteration waits
  // until this wave's loads of tile t have landed (the DMA loads of t+1 may
  // stay outstanding), then a barrier makes every wave's share visible and
  // guarantees that all waves are done with tile t-1, whose buffer the DMA
  // of t+2 reuses. DMAs past the last tile re-read it (never used).
  // The Q loads must be complete before the first DMA: otherwise the wait
  // the compiler places at their first use, inside the loop, would drain
  // the DMA queue on every iteration.
#pragma unroll
  for (int g = 0; g < NQ; ++g)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[g][ks]));
  const int last = n_tiles - 1;
  // prologue: tiles 0 .. NBUF-2 into buffers 0 .. NBUF-2 (clamped to the
  // last tile; a buffer past it holds a copy that is never read)
#pragma unroll
  for (int i = 0; i + 1 < NBUF; i += 2) {
    int pa_ids[PPW], pb_ids[PPW];
    const int ta = min(i, last), tb = min(i + 1, last);
    if constexpr (PPW == 2) {
      sload2(entry(ta, 0), entry(ta, 1), pa_ids[0], pa_ids[1]);
      if (i + 2 < NBUF) sload2(entry(tb, 0), entry(tb, 1), pb_ids[0], pb_ids[1]);
    } else {
      sload2(entry(ta, 0), entry(tb, 0), pa_ids[0], pb_ids[0]);
    }
    dma_ids(ta, i, pa_ids);
    if (i + 2 < NBUF) dma_ids(tb, i + 1, pb_ids);
  }
  // One iteration, buffer b = t mod NBUF known at compile time (the loop is
  // unrolled NBUF times), so LDS offsets are immediates. Tile t+NBUF-1 goes
  // into the buffer of tile t-1, which every wave has finished once past
  // this iteration's barrier; clamped re-reads of the last tile land in
  // buffers no later iteration reads.
  auto iter = [&](int t, auto bc) {
    constexpr int b = decltype(bc)::value;
    const int tn = min(t + NBUF - 1, last);
    const int32_t* e[PPW];
    int ids[PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) e[i] = entry(tn, i);
    sload_barrier<PPW, 2 * PPW * (NBUF - 2)>(e, ids);
    if ((t + 1) * KT > kv_end) {
      zero_tail(t, b);
      __syncthreads();
    }
    dma_ids(tn, (b + NBUF - 1) % NBUF, ids);
    if (wave_active && t * KT <= wave_last_pos) compute(bc, t * KT);
  };
  for (int t = 0; t < n_tiles; t += NBUF)
    for_each_const(
        [&](auto bc) {
          if (t + decltype(bc)::value < n_tiles) iter(t + decltype(bc)::value, bc);
        },
        std::make_integer_sequence<int, NBUF>{});
  wait_vmcnt0();  // no DMA may still be writing this workgroup's LDS when it ends

  if (!wave_active) return;
  // finish: the query's denominator is the sum over its four lanes
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    const float l2 = lsum[g] + __shfl_xor(lsum[g], 16);
    const float lt = l2 + __shfl_xor(l2, 32);
    const int jq = wq0 + g * 16 + n16;
    if (jq >= L) continue;
    const int64_t orow = ((int64_t)(q_beg + jq) * a.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d0 = dt * 16 + 4 * g4;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = o[g][dt][i] / lt;
      if (a.out_f32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + orow + d0) = f32x4{v[0], v[1], v[2], v[3]};
      } else {
        const uint32_t w0 = to_bits<DT>(v[0]) | (to_bits<DT>(v[1]) << 16);
        const uint32_t w1 = to_bits<DT>(v[2]) | (to_bits<DT>(v[3]) << 16);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + orow + d0) = u32x2{w0, w1};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// f32 causal prefill on the matrix cores. v_mfma_f32_16x16x4_f32 takes fp32
// operands and accumulates in fp32 (no rounding of q, K, V or P), at the
// chip's fp32 rate; what it adds over the vector ALUs is that each K/V tile
// is staged in LDS once and shared by the workgroup's 128 queries (8 waves x
// 16), instead of every query row walking its own causal prefix.
// Same orientation as the f16/bf16 kernel: S^T = K Q^T, O^T += V^T P^T, with
// the score accumulator a lane holds (query n16, keys 4 g4 + r) used as the
// P^T operand of the k-steps that walk those keys, so P stays in registers
// at full precision. Each MFMA contracts 4 values, so the operands are
// read 4 k-steps at a time with one 16-byte LDS read per lane: Q.K steps
// (t, u) take dims 16 t + 4 g4 + u, and the P.V product is cut into output
// blocks (bb, u) whose row i is dim 64 bb + 4 i + u. A tile is 8 KiB of K
// and 8 KiB of V (16 keys at head dim 128, 32 at 64), three tiles deep in
// LDS by the LDS DMA; rows are XOR-swizzled by 16-byte chunk (chunk c of
// row r at c ^ (r mod 16)), so both the K reads (16 rows, one chunk) and the
// V reads (one row, 16 chunks) use every bank once.
namespace {
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
}  // namespace

template <int D, int BS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void prefill_f32_kernel(const PrefillArgs a) {
  constexpr int NW = 8;              // waves per workgroup, 16 queries each
  constexpr int KTF = 2048 / D;      // keys per tile: 8 KiB of K and of V
  constexpr int NSUB = KTF / 16;     // 16-key subtiles
  constexpr int NT = D / 16;         // groups of 4 Q.K k-steps (16 dims)
  constexpr int NBB = D / 64;        // 64-dim blocks of O^T (4 MFMA outputs each)
  constexpr int NCH = 4;             // Q.K accumulation chains
  constexpr int CPR = D / 4;         // 16-byte chunks per row
  constexpr int ROWB = D * 4;        // bytes per K/V row
  constexpr int TILEB = KTF * ROWB;  // 8 KiB
  constexpr int PR = 1024 / ROWB;    // rows per 1 KiB DMA piece (one per wave)
  static_assert(TILEB == 1024 * NW && CPR >= 16, "one DMA piece per wave; rows of at least 16 chunks");
  static_assert(PR <= BS && BS % PR == 0, "the rows of one DMA piece lie in one block");
  static_assert(NW * 16 == QT, "the query tile of the f16/bf16 kernel");

  __shared__ __align__(1024) uint8_t sk[NBUF][TILEB];
  __shared__ __align__(1024) uint8_t sv[NBUF][TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15;
  const int g4 = lane >> 4;

  int h, s, qt;
  if (!prefill_item<KTF, kPrefillF32WorkgroupsPerCU>(a, lane, s, h, qt)) return;
  const ChunkRows cr =
      chunk_rows(a.query_start_loc[s], a.query_start_loc[s + 1], a.context_lens[s], a.total_q, a.max_context_len);
  const int ctx = cr.ctx, q_beg = cr.q_beg, L = cr.L;
  const int j0 = qt * QT;
  if (j0 >= L) return;
  const int c0 = ctx - L;                          // position of the chunk's first query
  const int kv_end = c0 + min(j0 + QT, L);         // keys this workgroup needs: [0, kv_end)
  const int n_tiles = (kv_end + KTF - 1) / KTF;
  const int wq0 = j0 + wave * 16;                  // the wave's first query (chunk-relative)
  const bool wave_active = wq0 < L;
  const int wave_last_pos = c0 + min(wq0 + 16, L) - 1;

  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks;
  const int nb = (kv_end + BS - 1) / BS;           // blocks this workgroup reads
  const uint32_t blk_bytes = (uint32_t)a.H * BS * ROWB;   // one block of every head (< 2^32)
  const uint32_t head_bytes = (uint32_t)h * BS * ROWB;

  // Q^T operand of k-step (t, u): query n16, dim 16 t + 4 g4 + u
  const int jq = wq0 + n16;
  const uint32_t qsign = a.q_sign ? 0x80000000u : 0u;
  f32x4 qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (jq < L) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(a.q) +
                                                       ((int64_t)(q_beg + jq) * a.H + h) * D + 16 * t + 4 * g4);
      qf[t] = __builtin_bit_cast(f32x4, u32x4{v[0] ^ qsign, v[1] ^ qsign, v[2] ^ qsign, v[3] ^ qsign});
    } else {
      qf[t] = zero4();
    }
  }
  // o[bb][u]: O^T rows d = 64 bb + 4 i + u (i = 4 g4 + r), query n16;
  // lsum: this lane's share of the softmax denominator (its keys' P)
  f32x4 o[NBB][4];
#pragma unroll
  for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
    for (int u = 0; u < 4; ++u) o[bb][u] = zero4();
  float m = -INFINITY, lsum = 0.f;

  // DMA: wave w moves rows w*PR .. w*PR+PR-1 of each tile; lane L fills
  // chunk position L % CPR of row L / CPR from source chunk (L % CPR) ^ sw
  const int prow = lane / CPR;
  const int pcol = lane % CPR;
  const uint32_t src = prow * ROWB + ((pcol ^ ((wave * PR + prow) & 15)) * 16);
  const uint32_t sk0 = lds_offset(&sk[0][0]);
  const uint32_t sv0 = lds_offset(&sv[0][0]);
  auto entry = [&](int t) {
    const uint32_t k = (uint32_t)(t * KTF + wave * PR);
    return bt_row + min(k / BS, (uint32_t)(nb - 1));
  };
  auto dma_id = [&](int t, int b, int phys) {
    const uint32_t key = (uint32_t)(t * KTF + wave * PR);
    const uint64_t row = (uint64_t)(uint32_t)clamp_block(phys, a.num_blocks) * blk_bytes + (head_bytes + (key % BS) * ROWB);
    lds_dma16s(kc + row, src, sk0 + b * TILEB + wave * 1024);
    lds_dma16s(vc + row, src, sv0 + b * TILEB + wave * 1024);
  };
  auto zero_tail = [&](int t, int b) {
    const int r0 = kv_end - t * KTF;
    for (int i = tid; i < (KTF - r0) * CPR; i += NW * 64)
      *reinterpret_cast<u32x4*>(&sv[b][(r0 + i / CPR) * ROWB + (i % CPR) * 16]) = u32x4{0u, 0u, 0u, 0u};
  };
  // LDS offsets of the operand reads: K row 16 sub + n16, chunk 4 t + g4;
  // V row 16 sub + 4 g4 + j, chunk 16 bb + n16 (the swizzle of both rows is
  // their row index mod 16: n16, and 4 g4 + j)
  const uint32_t k_rd = n16 * ROWB + ((g4 ^ n16) * 16);  // t enters as an XOR of 4 t into the chunk index
  const float c = fmaxf(a.scale_log2, 1.17549435e-38f);

  auto compute = [&](auto bc, int kv0) {
    constexpr int b = decltype(bc)::value;
    // Four independent accumulation chains over the dims (k-step (t, u) goes
    // to chain u), added pairwise at the end: fp32 chains of a quarter of the
    // steps over smaller partial sums round about as little as a per-lane
    // dot product finished by a butterfly (a single chain's rounding error
    // of the scores, amplified by the exponent at large scales, would exceed
    // 1e-5 on the outputs), and consecutive MFMAs do not wait on each other
    f32x4 sacc[NSUB];
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      f32x4 ch[NCH];
#pragma unroll
      for (int i = 0; i < NCH; ++i) ch[i] = zero4();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 ka = *reinterpret_cast<const f32x4*>(&sk[b][sub * 16 * ROWB + (k_rd ^ (t << 6))]);
#pragma unroll
        for (int u = 0; u < 4; ++u) ch[u % NCH] = mfma4(ka[u], qf[t][u], ch[u % NCH]);
      }
#pragma unroll
      for (int w = NCH / 2; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) ch[i] += ch[i + w];
      sacc[sub] = ch[0];
    }
    if (kv0 + KTF - 1 > c0 + wq0) {  // keys past a query's position score -inf
      const int last_key = min(c0 + jq, kv_end - 1);
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kv0 + 16 * sub + 4 * g4 + r > last_key) sacc[sub][r] = -INFINITY;
    }
    // online softmax with the lazy max of the f16/bf16 kernel
    float mr = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) mr = fmaxf(mr, sacc[sub][r]);
    if (__any(mr * c > m + RESCALE_LOG2)) {
      const float mt = rows4_max(mr) * c;
      const bool grow = mt > m + RESCALE_LOG2;
      if (__any(grow)) {
        const float m_new = grow ? mt : m;
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        lsum *= alpha;
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
          for (int u = 0; u < 4; ++u) o[bb][u] *= alpha;
        m = m_new;
      }
    }
    const float neg_m = m == -INFINITY ? 0.f : -m;
    f32x4 p[NSUB];
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[sub][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sub][r], c, neg_m));
        lsum += p[sub][r];
      }
    // O^T += V^T P^T: k-step (sub, j) takes keys 16 sub + 4 k + j, whose P
    // lane (k, n16) already holds in p[sub][j]
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb) {
          const int vr = 16 * sub + 4 * g4 + j;
          const f32x4 va = *reinterpret_cast<const f32x4*>(
              &sv[b][vr * ROWB + (((16 * bb + n16) ^ (4 * g4 + j)) * 16)]);
#pragma unroll
          for (int u = 0; u < 4; ++u) o[bb][u] = mfma4(va[u], p[sub][j], o[bb][u]);
        }
  };

  // The pipeline of the f16/bf16 kernel with one DMA piece per wave: tile
  // t+2 in flight while tile t is computed; one barrier per tile. The Q
  // loads complete before the first DMA, so no wait inside the loop drains
  // the DMA queue for them.
#pragma unroll
  for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(qf[t]));
  const int last = n_tiles - 1;
  {
    int ida, idb;
    sload2(entry(0), entry(min(1, last)), ida, idb);
    dma_id(0, 0, ida);
    dma_id(min(1, last), 1, idb);
  }
  static_assert(NBUF == 3, "three LDS buffers");
  auto iter = [&](int t, auto bc) {
    constexpr int b = decltype(bc)::value;
    const int tn = min(t + NBUF - 1, last);
    const int32_t* e[1] = {entry(tn)};
    int ids[1];
    sload_barrier<1, 2 * (NBUF - 2)>(e, ids);
    if ((t + 1) * KTF > kv_end) {
      zero_tail(t, b);
      __syncthreads();
    }
    dma_id(tn, (b + NBUF - 1) % NBUF, ids[0]);
    if (wave_active && t * KTF <= wave_last_pos) compute(bc, t * KTF);
  };
  for (int t = 0; t < n_tiles; t += NBUF)
    for_each_const(
        [&](auto bc) {
          if (t + decltype(bc)::value < n_tiles) iter(t + decltype(bc)::value, bc);
        },
        std::make_integer_sequence<int, NBUF>{});
  wait_vmcnt0();  // no DMA may still be writing this workgroup's LDS when it ends

  if (!wave_active) return;
  const float l2 = lsum + __shfl_xor(lsum, 16);
  const float lt = l2 + __shfl_xor(l2, 32);
  if (jq >= L) return;
  float* orow = reinterpret_cast<float*>(a.out) + ((int64_t)(q_beg + jq) * a.H + h) * D;
#pragma unroll
  for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<f32x4*>(orow + 64 * bb + 16 * g4 + 4 * r) =
          f32x4{o[bb][0][r] / lt, o[bb][1][r] / lt, o[bb][2][r] / lt, o[bb][3][r] / lt};
}

template <int D, int BS>
static hipError_t launch_f32(const PrefillArgs& a, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.num_seqs * a.H;
  const int64_t grid = (int64_t)a.q_tiles * (a.grouped ? (pairs + 7) / 8 * 8 : pairs);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_f32_kernel<D, BS>), dim3((unsigned)grid), dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_f32_bs(const PrefillArgs& a, int BS, hipStream_t stream) {
  switch (BS) {
    case 8: return launch_f32<D, 8>(a, stream);
    case 16: return launch_f32<D, 16>(a, stream);
    case 32: return launch_f32<D, 32>(a, stream);
    case 64: return launch_f32<D, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_f32(const PrefillArgs& a, int D, int BS, hipStream_t stream) {
  if (D == 128) return dispatch_f32_bs<128>(a, BS, stream);
  if (D == 64) return dispatch_f32_bs<64>(a, BS, stream);
  return hipErrorInvalidValue;
}

int prefill_mfma_q_tile() { return QT; }

template <Dt DT, int D, int BS>
static hipError_t launch_k4(const PrefillArgs& a, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.num_seqs * a.H;
  const int64_t grid = (int64_t)a.q_tiles * (a.grouped ? (pairs + 7) / 8 * 8 : pairs);
  if (grid == 0) return hipSuccess;
  // every workgroup resident at once: the wide shape (head dim 128)
  if constexpr (D == 128) {
    if (a.wide) {
      hipLaunchKernelGGL((prefill_mfma_kernel<DT, D, BS, true>), dim3((unsigned)grid), dim3(PfShape<D, true>::NW * 64),
                         0, stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_mfma_kernel<DT, D, BS, false>), dim3((unsigned)grid), dim3(PfShape<D, false>::NW * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <Dt DT, int D>
static hipError_t dispatch_k4_bs(const PrefillArgs& a, int BS, hipStream_t stream) {
  switch (BS) {
    case 8: return launch_k4<DT, D, 8>(a, stream);
    case 16: return launch_k4<DT, D, 16>(a, stream);
    case 32: return launch_k4<DT, D, 32>(a, stream);
    case 64: return launch_k4<DT, D, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <Dt DT>
static hipError_t dispatch_k4(const PrefillArgs& a, int D, int BS, hipStream_t stream) {
  if (D == 128) return dispatch_k4_bs<DT, 128>(a, BS, stream);
  if (D == 64) return dispatch_k4_bs<DT, 64>(a, BS, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, Dt dt, int D, int BS, hipStream_t stream) {
  if (dt == Dt::F16) return dispatch_k4<Dt::F16>(a, D, BS, stream);
  if (dt == Dt::BF16) return dispatch_k4<Dt::BF16>(a, D, BS, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
