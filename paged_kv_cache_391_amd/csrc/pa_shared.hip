// Shared-prefix partitions on the matrix cores.
//
// Parallel samples of one prompt list the same physical blocks for the
// prompt (aidocs.cortexgrid.cn page, FAQ answer on parallel sampling;
// devpress.csdn.net page, "实际收益远超预期"), so the prompt's K/V only has to
// be streamed once for all of them. With up to 16 samples' queries against
// one K/V tile the work is a small dense contraction, so a wave runs it on
// v_mfma_f32_16x16x32_{f16,bf16} in the same orientation as the causal
// prefill kernel: S^T = K Q^T (keys on the MFMA rows, the group's members on
// the columns) and O^T += V^T P^T, where the score accumulator a lane holds
// (one member, 4 keys per 16-key subtile) is exactly the B operand P^T needs.
//
// One wave per (group, head, partition of the shared prefix, chunk of 16
// members). Per step of 32 keys:
//   * K is loaded straight into MFMA A fragments (lane: one key, 8 dims);
//   * V is loaded two keys per lane, packed pairwise and written transposed
//     into the wave's own LDS buffer, from which the V^T fragments are read;
//   * the next step's loads are in flight while the current step computes;
//   * the running max of a member is raised lazily (by more than 2^8 at a
//     time, wave-uniform), so the accumulators are rescaled on few steps.
// The prefix is whole 16-token tiles, so only a half-filled last step
// masks. Each member gets (m, l, acc[D]) for this partition in the split-K
// workspace (or its final output when the partition is all it has); its
// private tail and the merge run in the partition and reduction kernels.
#include "pa_decode_device.h"

namespace pa {

namespace {
constexpr float kRescaleLog2 = 8.f;  // p = 2^(s - m) stays below 2^8 between rescales
}

template <Dt DT, int D, int BS>
__device__ __forceinline__ void shared_prefix_body(const DecodeArgs& a, int bid) {
  constexpr int KS = D / 32;      // MFMA k-steps over head_dim for S^T = K Q^T
  constexpr int NDT = D / 16;     // 16-row blocks of O^T
  constexpr int ROWB = D * 2;     // bytes of one K/V row (16-bit elements)
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int VCH = CPR / 4;    // V chunks per lane per key
  constexpr int VROW = 32 + 4;    // V^T row stride in LDS (halves): 32 keys, padded

  __shared__ __align__(16) uint16_t sv[2][D * VROW];

  const int lane = threadIdx.x;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;

  // grid: partition-major, then group, member chunk, head
  const int h = bid % a.H;
  bid /= a.H;
  const int mc = bid % a.member_chunks;
  bid /= a.member_chunks;
  const int grp = bid % a.num_groups;
  const int part = bid / a.num_groups;

  const int r_begin = min(max(a.group_starts[grp], 0), a.num_rows);
  const int m0 = r_begin + 16 * mc;
  const int nm = min(16, min(max(a.group_starts[grp + 1], r_begin), a.num_rows) - m0);
  if (nm <= 0) return;
  const int pt = a.shared_part_tiles * 16;
  const int prefix = group_prefix(a, grp);  // whole tiles every member holds
  const int ns = (prefix + pt - 1) / pt;
  if (part >= ns) return;
  const int k_begin = part * pt;
  const int k_end = min(prefix, k_begin + pt);
  const int nsteps = (k_end - k_begin + 31) >> 5;

  // Q^T fragments (B of S^T = K Q^T): member n16, dims 32*ks + 8*g4 .. +7
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = u32x4{0u, 0u, 0u, 0u};
    if (n16 < nm)
      qf[ks] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.q) +
                                               (((int64_t)(m0 + n16) * a.H + h) * D + ks * 32 + 8 * g4) * 2);
  }

  // table entries of the partition's blocks (at most 64), read out with readlane
  const int32_t* bt_row = a.block_tables + (int64_t)r_begin * a.max_blocks + k_begin / BS;
  const int nblk = (k_end - k_begin + BS - 1) / BS;
  const int32_t tb = lane < nblk ? clamp_block(bt_row[lane], a.num_blocks) : 0;
  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);
  // byte offset of partition-relative key `key` (wave-uniform); a 16-key
  // subtile lies in one block, or in two when blocks hold 8 tokens
  auto row_off = [&](int key) -> int64_t {
    const int32_t phys = __builtin_amdgcn_readlane(tb, key / BS);
    return kv_row_offset(phys, h, key % BS, a.H, BS, D) * 2;
  };

  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = zero4();
  float m = -INFINITY, l = 0.f;

  // ---- loads of step s: K fragments (subtile sb, k-step ks) and V rows of
  // keys 2*n16 and 2*n16+1, chunks g4 + 4*j. A subtile past k_end re-reads
  // subtile 0 (its scores are masked and its V rows zeroed).
  auto load_k = [&](u32x4 (&kf)[2][KS], int s) {
    const int rel = 32 * s;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int sub = k_begin + rel + 16 * sb < k_end ? rel + 16 * sb : rel;
      int64_t row;
      if constexpr (BS >= 16) {
        row = row_off(sub) + n16 * ROWB;
      } else {
        const int64_t r0 = row_off(sub), r1 = row_off(sub + 8);
        row = (n16 < 8 ? r0 : r1) + (n16 & 7) * ROWB;
      }
      const char* base = kc + row + g4 * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[sb][ks] = *reinterpret_cast<const u32x4*>(base + ks * 64);
    }
  };
  auto load_v = [&](u32x4 (&vr)[VCH][2], int s) {
    const int rel = 32 * s;
    const int off1 = k_begin + rel + 16 < k_end ? rel + 16 : rel;
    int64_t base;
    if constexpr (BS >= 16) {
      const int64_t b0 = row_off(rel), b1 = row_off(off1);
      base = (n16 < 8 ? b0 : b1) + (2 * (n16 & 7)) * ROWB;
    } else {  // keys 2*n16 and 2*n16+1 lie in block n16 / 4 of the step
      const int64_t c0 = row_off(rel), c1 = row_off(rel + 8), c2 = row_off(off1), c3 = row_off(off1 + 8);
      const int q4 = n16 >> 2;
      base = (q4 == 0 ? c0 : q4 == 1 ? c1 : q4 == 2 ? c2 : c3) + (2 * (n16 & 3)) * ROWB;
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        vr[j][e] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(vc + base + e * ROWB + (g4 + 4 * j) * 16));
  };
  // V rows -> V^T in LDS buffer b, two keys packed per 32-bit word
  auto stage_v = [&](int b, const u32x4 (&vr)[VCH][2], int s) {
    const int key0 = k_begin + 32 * s + 2 * n16;
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
      const int c = g4 + 4 * j;
      const u32x4 v0 = key0 < k_end ? vr[j][0] : z;
      const u32x4 v1 = key0 + 1 < k_end ? vr[j][1] : z;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = (v0[w] & 0xffffu) | (v1[w] << 16);      // dim 8c+2w of keys 2n16, 2n16+1
        const uint32_t hi = (v0[w] >> 16) | (v1[w] & 0xffff0000u);  // dim 8c+2w+1
        *reinterpret_cast<uint32_t*>(&sv[b][(8 * c + 2 * w) * VROW + 2 * n16]) = lo;
        *reinterpret_cast<uint32_t*>(&sv[b][(8 * c + 2 * w + 1) * VROW + 2 * n16]) = hi;
      }
    }
  };

  auto compute = [&](int b, const u32x4 (&kf)[2][KS], int s) {
    f32x4 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      sacc[sb] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc[sb] = mfma16<DT>(kf[sb][ks], qf[ks], sacc[sb]);
    }
    // lane: member n16, keys 32s + 16sb + 4g4 + i
    const bool partial = k_begin + 32 * s + 32 > k_end;
    float x[8];
    float mt = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k_begin + 32 * s + 16 * sb + 4 * g4 + i;
        const float v = sacc[sb][i] * a.scale_log2;
        x[4 * sb + i] = (!partial || key < k_end) ? v : -INFINITY;
        mt = fmaxf(mt, x[4 * sb + i]);
      }
    mt = rows4_max(mt);
    const bool grow = mt > m + kRescaleLog2;  // true on the first step (m = -inf)
    if (__any(grow)) {
      const float m_new = grow ? mt : m;
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      m = m_new;
    }
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(x[i] - m);
      l += p;
      ph[i] = to_bits<DT>(p);
      pl[i] = DT == Dt::BF16 ? to_bits<DT>(p - from_bits<DT>(ph[i])) : 0u;
    }
    // B operand P^T: k-order = keys [4g4 .. 4g4+3] then [16+4g4 .. 16+4g4+3]
    const u32x4 pb = u32x4{ph[0] | (ph[1] << 16), ph[2] | (ph[3] << 16), ph[4] | (ph[5] << 16), ph[6] | (ph[7] << 16)};
    const u32x4 pbl = u32x4{pl[0] | (pl[1] << 16), pl[2] | (pl[3] << 16), pl[4] | (pl[5] << 16), pl[6] | (pl[7] << 16)};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint16_t* row = &sv[b][(dt * 16 + n16) * VROW + 4 * g4];
      const u32x2 lo = *reinterpret_cast<const u32x2*>(row);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 16);
      const u32x4 va = u32x4{lo[0], lo[1], hi[0], hi[1]};
      o[dt] = mfma16<DT>(va, pb, o[dt]);
      if constexpr (DT == Dt::BF16) o[dt] = mfma16<DT>(va, pbl, o[dt]);
    }
  };

  // Step s uses K set (s even: a, odd: b) and LDS buffer s & 1; the loads of
  // step s+1 are in flight while step s computes, then its V is staged.
  // Loads and stages are unconditional (clamped past the end) so the
  // compiler's wait counts stay exact.
  u32x4 ka[2][KS], kb[2][KS];
  u32x4 vr[VCH][2];
  load_k(ka, 0);
  load_v(vr, 0);
  stage_v(0, vr, 0);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    load_k(kb, min(s + 1, nsteps - 1));
    load_v(vr, min(s + 1, nsteps - 1));
    compute(0, ka, s);
    stage_v(1, vr, s + 1);
    __syncthreads();
    load_k(ka, min(s + 2, nsteps - 1));
    load_v(vr, min(s + 2, nsteps - 1));
    if (s + 1 < nsteps) compute(1, kb, s + 1);
    stage_v(0, vr, s + 2);
    __syncthreads();
  }

  // merge the four lane rows of each member; write the partial or output
  const float lt = rows4_sum(l);
  if (n16 >= nm) return;
  const int row = m0 + n16;
  const int ctx = row_ctx(a, row);
  const int total = ns + own_partitions(ctx, prefix, a.part_tiles);
  if (total <= 1) {
    const int64_t orow = ((int64_t)row * a.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d0 = dt * 16 + 4 * g4;
      if (a.out_f32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + orow + d0) = o[dt] / lt;
      } else {
        const f32x4 v = o[dt] / lt;
        const uint32_t w0 = to_bits<DT>(v[0]) | (to_bits<DT>(v[1]) << 16);
        const uint32_t w1 = to_bits<DT>(v[2]) | (to_bits<DT>(v[3]) << 16);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + orow + d0) = u32x2{w0, w1};
      }
    }
  } else {
    const int64_t prow = ((int64_t)row * a.H + h) * a.ws_parts + part;
    float* acc_out = a.ws + prow * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(acc_out + dt * 16 + 4 * g4) = o[dt];
    if (g4 == 0) {
      float* ml = a.ws + (int64_t)a.num_rows * a.H * a.ws_parts * D + prow * 2;
      ml[0] = m;
      ml[1] = lt;
    }
  }
}

// One launch for the whole shared-prefix decode (before the reduction):
// workgroups [0, n_shared) run the shared prefixes on the matrix cores,
// the rest run the members' private tails as partition-kernel waves (one
// head per workgroup), so the two kinds of work overlap on the chip instead
// of running one after the other.
template <Dt DT, int D, int BS>
__global__ __launch_bounds__(64) void shared_prefix_step_kernel(const DecodeArgs a, int n_shared) {
  if ((int)blockIdx.x < n_shared)
    shared_prefix_body<DT, D, BS>(a, blockIdx.x);
  else
    decode_partition_body<DT, D, BS, 1, RowMode::SharedTail>(a, blockIdx.x - n_shared, 0);
}

template <Dt DT, int D, int BS>
static hipError_t launch_step(const DecodeArgs& a, int shared_parts, int tail_parts, hipStream_t stream) {
  const int64_t n_shared = (int64_t)a.num_groups * a.member_chunks * a.H * shared_parts;
  const int64_t grid = n_shared + (int64_t)a.num_rows * a.H * tail_parts;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((shared_prefix_step_kernel<DT, D, BS>), dim3((unsigned)grid), dim3(64), 0, stream, a,
                     (int)n_shared);
  return hipGetLastError();
}

template <Dt DT, int D>
static hipError_t dispatch_step_bs(const DecodeArgs& a, int BS, int sp, int tp, hipStream_t stream) {
  switch (BS) {
    case 8: return launch_step<DT, D, 8>(a, sp, tp, stream);
    case 16: return launch_step<DT, D, 16>(a, sp, tp, stream);
    case 32: return launch_step<DT, D, 32>(a, sp, tp, stream);
    case 64: return launch_step<DT, D, 64>(a, sp, tp, stream);
  }
  return hipErrorInvalidValue;
}

template <Dt DT>
static hipError_t dispatch_step(const DecodeArgs& a, int D, int BS, int sp, int tp, hipStream_t stream) {
  if (D == 128) return dispatch_step_bs<DT, 128>(a, BS, sp, tp, stream);
  if (D == 64) return dispatch_step_bs<DT, 64>(a, BS, sp, tp, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_shared_prefix_step(const DecodeArgs& a, Dt dt, int D, int BS, int shared_parts, int tail_parts,
                                     hipStream_t stream) {
  if (dt == Dt::F16) return dispatch_step<Dt::F16>(a, D, BS, shared_parts, tail_parts, stream);
  if (dt == Dt::BF16) return dispatch_step<Dt::BF16>(a, D, BS, shared_parts, tail_parts, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
