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
// is exactly the B operand P^T needs, so P never leaves registers; the
// price is a transposed V tile, which the workgroup writes into LDS while
// staging it. Per tile of KT keys:
//   * addressing is scalar: every global load of a wave covers a few
//     consecutive keys that lie in one block, so the wave reads the block's
//     id with a scalar load (the scalar cache keeps the table row), forms
//     the row address in scalar registers and adds only a fixed per-lane
//     offset;
//   * 256 threads gather each K tile (row-major) and V tile (transposed,
//     key pairs packed with v_perm) into one of two LDS buffers; tile t+R's
//     global loads are in flight while tile t is computed and tile t+1 is
//     staged, one barrier per tile; only the last tile clamps and zeroes;
//   * each wave owns NQ groups of 16 queries; every K or V^T fragment read
//     from LDS feeds one MFMA per group;
//   * online softmax per query: the max over the raw scores (the scale is
//     applied once to it, and inside the exponent's FMA), cross-row max on
//     the row-swap instructions, P narrowed with the packed converts; the
//     denominator is summed on the matrix cores (a block of ones in V^T);
//     only tiles that cross a wave's first query carry the causal mask (the
//     masked scores are set to -inf), tiles past its last query are skipped, and
//     the running max is raised lazily (see compute()) so the accumulators
//     are rescaled only on the few tiles that need it.
// P is rounded to the input type for the P.V product; for bf16 it is split
// into a bf16 head and a bf16 remainder (two MFMAs) to keep ~16 bits. A
// negative scale is applied as |scale| on negated queries (exact: a sign
// flip), so the max of the raw scores is the max of the scaled ones.
#include "pa_internal.h"

namespace pa {

namespace {

#ifndef PA_PREFILL_KT
#define PA_PREFILL_KT 32
#endif
#ifndef PA_PREFILL_NQ
#define PA_PREFILL_NQ 2
#endif
#ifndef PA_PREFILL_R
#define PA_PREFILL_R 2
#endif
constexpr int KT = PA_PREFILL_KT;  // keys per tile (32 or 64)
constexpr int NQ = PA_PREFILL_NQ;  // 16-query groups per wave
constexpr int QW = 16 * NQ;        // queries per wave
constexpr int QT = 4 * QW;         // queries per workgroup
constexpr int R = PA_PREFILL_R;    // register sets: tile t+R is fetched while tile t is computed
constexpr int UNR = R % 2 == 0 ? R : 2 * R;  // loop unroll: a multiple of R and of the two LDS buffers
constexpr float RESCALE_LOG2 = 8.f; // lazy rescale threshold (log2 units): p < 256 between rescales
static_assert(KT == 32 || KT == 64, "key tile must be 32 or 64");

}  // namespace

template <Dt DT, int D, int BS>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(const PrefillArgs a) {
  constexpr int KS = D / 32;     // MFMA k-steps over head_dim for Q.K
  constexpr int NDT = D / 16;    // 16-row tiles of O^T
  constexpr int NSUB = KT / 16;  // 16-key subtiles of S^T
  constexpr int NKST = KT / 32;  // MFMA k-steps over keys for P.V
  constexpr int CPR = D / 8;     // 16-byte chunks per K/V row
  constexpr int ROWB = D * 2;    // bytes per K/V row
  constexpr int KROW = D + 8;    // K tile row stride in LDS (halves), padded against bank conflicts
  constexpr int VROW = KT + 4;   // V^T tile row stride in LDS (halves)
  constexpr int NKC = KT * CPR;          // K chunks per tile
  constexpr int NVP = (KT / 2) * CPR;    // V (key pair, chunk) items per tile
  constexpr int KCH = NKC / 256;
  constexpr int VPR = (NVP + 255) / 256;
  // one load of a wave covers KW consecutive keys of K, VW of V (in pairs)
  constexpr int KW = 64 / CPR;
  constexpr int VW = 2 * 64 / CPR;
  constexpr bool V_ONE_BLOCK = VW <= BS;
  static_assert(NKC % 256 == 0, "whole K chunks per thread");
  static_assert(KW <= BS && BS % KW == 0, "a wave's K rows of one load lie in one block");
  static_assert(V_ONE_BLOCK || VW == 2 * BS, "a wave's V rows of one load span at most two blocks");

  __shared__ __align__(16) uint16_t sk[2][KT * KROW];
  __shared__ __align__(16) uint16_t sv[2][D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15;
  const int g4 = lane >> 4;

  int bid = blockIdx.x;
  const int h = bid % a.H;
  bid /= a.H;
  const int s = bid % a.num_seqs;
  bid /= a.num_seqs;
  const int qt = a.q_tiles - 1 - bid;  // latest (heaviest) query tiles are dispatched first
  const int q_beg = a.query_start_loc[s];
  const int L = a.query_start_loc[s + 1] - q_beg;
  const int j0 = qt * QT;
  if (j0 >= L) return;
  const int ctx = a.context_lens[s];
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

  // o: O^T of the wave's queries; lacc: the softmax denominators, summed on
  // the matrix cores as a 17th row block of ones in V^T (every row of lacc
  // holds the sum of the query's rounded P, the same P the numerator uses)
  f32x4 o[NQ][NDT], lacc[NQ];
  float m[NQ];
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    m[g] = -INFINITY;
    lacc[g] = zero4();
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[g][dt] = zero4();
  }
  constexpr uint32_t ONE2 = ones2<DT>();
  const u32x4 ones = u32x4{ONE2, ONE2, ONE2, ONE2};

  // wave-uniform address of row `key` (tile-absolute) of head h, its block
  // id read through the scalar cache; keys past the sequence's blocks read
  // the last block's rows (zeroed when staged)
  auto row_base = [&](const char* cache, int key) -> const char* {
    const uint32_t k = (uint32_t)key;
    const uint32_t blk = min(k / BS, (uint32_t)(nb - 1));
    const uint32_t phys = (uint32_t)bt_row[blk];
    return cache + ((uint64_t)phys * blk_bytes + (head_bytes + (k % BS) * ROWB));
  };
  // per-lane byte offsets inside a wave's rows of one load
  const uint32_t k_lane = lane * 16;
  uint32_t v_lane[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    v_lane[e] = ((2 * (lane / CPR) + e) % (V_ONE_BLOCK ? VW : BS)) * ROWB + (lane % CPR) * 16;

  // ---- global -> registers for one tile. Every load is issued
  // unconditionally, so all of a tile's loads are in flight together.
  u32x4 kreg[R][KCH], vreg[R][2 * VPR];
  auto fetch = [&](u32x4 (&kr)[KCH], u32x4 (&vr)[2 * VPR], int t) {
    const int kv0 = t * KT;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int key = kv0 + (wave * 64 + 256 * r) / CPR;
      kr[r] = *reinterpret_cast<const u32x4*>(row_base(kc, key) + k_lane);
    }
#pragma unroll
    for (int r = 0; r < VPR; ++r) {
      const int pw = min(wave * 64 + 256 * r, NVP - 64);  // waves past the tile's pairs repeat the last ones
      const int key = kv0 + 2 * (pw / CPR);
      if constexpr (V_ONE_BLOCK) {
        const char* base = row_base(vc, key);
#pragma unroll
        for (int e = 0; e < 2; ++e) vr[2 * r + e] = *reinterpret_cast<const u32x4*>(base + v_lane[e]);
      } else {  // lanes 0..31 read the first block, 32..63 the next
        const char* b0 = row_base(vc, key);
        const char* b1 = row_base(vc, key + BS);
        const char* base = lane < 32 ? b0 : b1;
#pragma unroll
        for (int e = 0; e < 2; ++e) vr[2 * r + e] = *reinterpret_cast<const u32x4*>(base + v_lane[e]);
      }
    }
  };
  // ---- registers -> LDS buffer b: K row-major, V transposed (two keys
  // packed per word); rows at or past kv_end (last tile only) become zeros
  auto stage = [&](int b, int t, const u32x4 (&kr)[KCH], const u32x4 (&vr)[2 * VPR]) {
    const int kv0 = t * KT;
    auto put = [&](bool tail) {
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < KCH; ++r) {
        const int key = (wave * 64 + 256 * r) / CPR + lane / CPR;
        const int dc = lane % CPR;
        *reinterpret_cast<u32x4*>(&sk[b][key * KROW + dc * 8]) = (tail && kv0 + key >= kv_end) ? z : kr[r];
      }
#pragma unroll
      for (int r = 0; r < VPR; ++r) {
        const int pw = wave * 64 + 256 * r;
        if (NVP % 256 == 0 || pw < NVP) {
          const int kp = pw / CPR + lane / CPR;
          const int dc = lane % CPR;
          const u32x4 v0 = (tail && kv0 + 2 * kp >= kv_end) ? z : vr[2 * r];
          const u32x4 v1 = (tail && kv0 + 2 * kp + 1 >= kv_end) ? z : vr[2 * r + 1];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            // element 2w of keys 2kp, 2kp+1 (low halves), then element 2w+1 (high halves)
            const uint32_t lo = __builtin_amdgcn_perm(v1[w], v0[w], 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(v1[w], v0[w], 0x07060302u);
            *reinterpret_cast<uint32_t*>(&sv[b][(dc * 8 + 2 * w) * VROW + 2 * kp]) = lo;
            *reinterpret_cast<uint32_t*>(&sv[b][(dc * 8 + 2 * w + 1) * VROW + 2 * kp]) = hi;
          }
        }
      }
    };
    if (kv0 + KT > kv_end) put(true);
    else put(false);
  };

  // |scale| * log2(e), floored at the smallest normal float so that a
  // masked score (-inf) times c stays -inf: a zero scale then weighs every
  // allowed key equally to within 1e-26
  const float c = fmaxf(a.scale_log2, 1.17549435e-38f);
  auto compute = [&](int b, int kv0) {
    // S^T = K Q^T over NSUB key subtiles of 16
    f32x4 sacc[NQ][NSUB];
#pragma unroll
    for (int g = 0; g < NQ; ++g)
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) sacc[g][sub] = zero4();
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(&sk[b][(sub * 16 + n16) * KROW + ks * 32 + 8 * g4]);
#pragma unroll
        for (int g = 0; g < NQ; ++g) sacc[g][sub] = mfma16<DT>(ka, qf[g][ks], sacc[g][sub]);
      }
    }
    // online softmax; lane holds query n16, keys kv0 + 16*sub + 4*g4 + i.
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
    u32x4 pb[NQ][NKST];
    u32x4 pbl[NQ][NKST];  // bf16 remainders
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
      float mr = -INFINITY;  // max of the raw scores (c > 0: the scaled max is mr * c)
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) mr = fmaxf(mr, sacc[g][sub][i]);
      const float mt = rows4_max(mr) * c;
      const bool grow = mt > m[g] + RESCALE_LOG2;  // also true for the first tile (m = -inf)
      if (__any(grow)) {
        const float m_new = grow ? mt : m[g];
        const float alpha = __builtin_amdgcn_exp2f(m[g] - m_new);
        lacc[g] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[g][dt] *= alpha;
        m[g] = m_new;
      }
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
        if constexpr (DT == Dt::BF16) {
          uint32_t r[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            r[j] = pack2<DT>(p[8 * kst + 2 * j] - __uint_as_float(w[j] << 16),
                             p[8 * kst + 2 * j + 1] - __uint_as_float(w[j] & 0xffff0000u));
          pbl[g][kst] = u32x4{r[0], r[1], r[2], r[3]};
        }
      }
    }
    // O^T += V^T P^T: A = V^T rows d = 16*dt + n16, keys 32*kst + 4*g4 + {0..3} and +16
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int kst = 0; kst < NKST; ++kst) {
        const uint16_t* row = &sv[b][(dt * 16 + n16) * VROW + kst * 32 + 4 * g4];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(row);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 16);
        const u32x4 va = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int g = 0; g < NQ; ++g) {
          o[g][dt] = mfma16<DT>(va, pb[g][kst], o[g][dt]);
          if constexpr (DT == Dt::BF16) o[g][dt] = mfma16<DT>(va, pbl[g][kst], o[g][dt]);
        }
      }
    }
#pragma unroll
    for (int kst = 0; kst < NKST; ++kst)
#pragma unroll
      for (int g = 0; g < NQ; ++g) {
        lacc[g] = mfma16<DT>(ones, pb[g][kst], lacc[g]);
        if constexpr (DT == Dt::BF16) lacc[g] = mfma16<DT>(ones, pbl[g][kst], lacc[g]);
      }
  };

  // R register sets in a ring and two LDS buffers: while tile t is
  // computed, tile t+R travels global -> registers (set t % R) and tile t+1,
  // fetched R-1 tiles earlier, is staged into the other LDS buffer; one
  // barrier per tile. Fetches and stages are unconditional (past the end
  // they re-read the last tile, an L2 hit, and stage zeros that are never
  // read) so the compiler can prove each set's loads were consumed before it
  // is refilled and never drains the load queue early.
#pragma unroll
  for (int r = 0; r < R; ++r) fetch(kreg[r], vreg[r], min(r, n_tiles - 1));
  stage(0, 0, kreg[0], vreg[0]);
  __syncthreads();
  for (int t0 = 0; t0 < n_tiles; t0 += UNR) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = t0 + u;
      fetch(kreg[u % R], vreg[u % R], min(t + R, n_tiles - 1));
      if (wave_active && t < n_tiles && t * KT <= wave_last_pos) compute(u & 1, t * KT);
      stage((u + 1) & 1, t + 1, kreg[(u + 1) % R], vreg[(u + 1) % R]);
      __syncthreads();
    }
  }

  if (!wave_active) return;
  // finish: every row of lacc holds the query's denominator
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    const float lt = lacc[g][0];
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

int prefill_mfma_q_tile() { return QT; }

template <Dt DT, int D, int BS>
static hipError_t launch_k4(const PrefillArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.q_tiles * a.num_seqs * a.H;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_mfma_kernel<DT, D, BS>), dim3((unsigned)grid), dim3(256), 0, stream, a);
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
