// The library driven through its C ABI alone (no Python, no torch): device
// buffers from hipMalloc, the new tokens written with pa_reshape_and_cache,
// a split-K pa_paged_attention_decode and a causal pa_paged_attention_prefill
// whose fp32 outputs are copied back and compared with the fp64 oracle
// (linked from oracle/liboracle.so; test code only), then the same three
// parts as one pa_attention_step (the pa_step_args struct filled from C), in
// order and with the prefill on a side stream, each equal bit for bit to
// the separate calls and within tolerance of the oracle. Prints
// "max_abs_err <x>", "prefill_max_abs_err <y>", "step_bit_identical <0|1>",
// "step_max_abs_err <z>" and "step_prefill_max_abs_err <w>"; exits 0 when
// x, y, z, w <= 2e-3 and the step results are identical.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "pagedattn.h"

extern "C" int oracle_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                        const int32_t* slot_mapping, int num_tokens, int H, int d, int bs,
                                        int num_blocks, int dtype);
extern "C" int oracle_decode(double* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* bt, const int32_t* ctx, int S, int H, int d, int bs, int num_blocks,
                             int max_blocks, double scale, int dtype, const int32_t* pairs, int npairs,
                             int nthreads);
extern "C" int oracle_prefill(double* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* bt, const int32_t* ctx, const int32_t* qsl, int S, int H, int d,
                              int bs, int num_blocks, int max_blocks, double scale, int dtype, const int32_t* rows,
                              int nrows, int nthreads);

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::printf("%s: %s\n", #x, hipGetErrorString(e_));                      \
      return 2;                                                                \
    }                                                                          \
  } while (0)
#define PA_OK_(x)                                                              \
  do {                                                                         \
    pa_status s_ = (x);                                                        \
    if (s_ != PA_OK) {                                                         \
      std::printf("%s: %s\n", #x, pa_status_string(s_));                       \
      return 3;                                                                \
    }                                                                          \
  } while (0)

// IEEE binary16 bits of a float of magnitude below 2 (round to nearest even)
static uint16_t to_half_bits(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const int32_t exp = (int32_t)((x >> 23) & 0xffu) - 127 + 15;
  uint32_t mant = x & 0x7fffffu;
  if (exp <= 0) {  // subnormal half (or zero)
    if (exp < -10) return (uint16_t)sign;
    mant |= 0x800000u;
    const int shift = 14 - exp;
    uint32_t h = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (h & 1u))) ++h;
    return (uint16_t)(sign | h);
  }
  uint32_t h = ((uint32_t)exp << 10) | (mant >> 13);
  const uint32_t rem = mant & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
  return (uint16_t)(sign | h);
}

// f16 bits of a value in [-1, 1) drawn from a 64-bit LCG (test data only)
static uint16_t next_half(uint64_t& st) {
  st = st * 6364136223846793005ull + 1442695040888963407ull;
  return to_half_bits((float)((st >> 40) & 0xffffff) / 8388608.0f - 1.0f);
}

int main() {
  const int H = 4, D = 128, BS = 16, S = 3, NB = 80;
  const int ctx[S] = {1, 300, 700};  // the last one spans two 512-token partitions
  const int max_blocks = 44;
  const float scale = 1.0f / std::sqrt((float)D);
  const int64_t cache_elems = (int64_t)NB * H * BS * D;

  // block tables: consecutive slices of a fixed shuffle of the pool
  std::vector<int32_t> perm(NB);
  for (int i = 0; i < NB; ++i) perm[i] = (i * 37 + 11) % NB;  // 37 is coprime with 80
  std::vector<int32_t> bt((size_t)S * max_blocks, -1);
  int used = 0;
  for (int s = 0; s < S; ++s)
    for (int b = 0; b < (ctx[s] + BS - 1) / BS; ++b) bt[(size_t)s * max_blocks + b] = perm[used++];

  // cache contents of the first ctx-1 tokens, then one new token per sequence
  uint64_t st = 391;
  std::vector<uint16_t> kc(cache_elems), vc(cache_elems), q((size_t)S * H * D), nk((size_t)S * H * D),
      nv((size_t)S * H * D);
  for (auto& x : kc) x = next_half(st);
  for (auto& x : vc) x = next_half(st);
  for (auto& x : q) x = next_half(st);
  for (auto& x : nk) x = next_half(st);
  for (auto& x : nv) x = next_half(st);
  std::vector<int32_t> slots(S);
  for (int s = 0; s < S; ++s) {
    const int t = ctx[s] - 1;
    slots[s] = bt[(size_t)s * max_blocks + t / BS] * BS + t % BS;
  }

  void *dkc, *dvc, *dq, *dnk, *dnv, *dout, *dws;
  int32_t *dbt, *dctx, *dslots;
  HIP_OK(hipMalloc(&dkc, cache_elems * 2));
  HIP_OK(hipMalloc(&dvc, cache_elems * 2));
  HIP_OK(hipMalloc(&dq, q.size() * 2));
  HIP_OK(hipMalloc(&dnk, nk.size() * 2));
  HIP_OK(hipMalloc(&dnv, nv.size() * 2));
  HIP_OK(hipMalloc(&dout, (size_t)S * H * D * 4));
  HIP_OK(hipMalloc(&dbt, bt.size() * 4));
  HIP_OK(hipMalloc(&dctx, S * 4));
  HIP_OK(hipMalloc(&dslots, S * 4));
  const size_t ws_bytes = pa_decode_workspace_bytes(S, H, D, 700);
  HIP_OK(hipMalloc(&dws, ws_bytes));
  HIP_OK(hipMemcpy(dkc, kc.data(), cache_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dvc, vc.data(), cache_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dq, q.data(), q.size() * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dnk, nk.data(), nk.size() * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dnv, nv.data(), nv.size() * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dbt, bt.data(), bt.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dctx, ctx, S * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dslots, slots.data(), S * 4, hipMemcpyHostToDevice));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  PA_OK_(pa_reshape_and_cache(dnk, dnv, dkc, dvc, dslots, S, H, D, BS, NB, PA_F16, stream));
  PA_OK_(pa_paged_attention_decode(dout, PA_F32, dq, dkc, dvc, dbt, dctx, S, H, H, D, BS, NB, max_blocks, 700, scale,
                                   PA_F16, dws, ws_bytes, stream));
  // an unsupported head dim is refused before anything is launched
  if (pa_paged_attention_decode(dout, PA_F32, dq, dkc, dvc, dbt, dctx, S, H, H, 96, BS, NB, max_blocks, 700, scale,
                                PA_F16, dws, ws_bytes, stream) != PA_ERR_UNSUPPORTED) {
    std::printf("head dim 96 was not refused\n");
    return 4;
  }
  std::vector<float> out((size_t)S * H * D);
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(out.data(), dout, out.size() * 4, hipMemcpyDeviceToHost));

  // the oracle on the host copies
  if (oracle_reshape_and_cache(nk.data(), nv.data(), kc.data(), vc.data(), slots.data(), S, H, D, BS, NB, 1) != 0) {
    std::printf("oracle cache write failed\n");
    return 5;
  }
  std::vector<int32_t> pairs;
  for (int s = 0; s < S; ++s)
    for (int h = 0; h < H; ++h) pairs.insert(pairs.end(), {s, h});
  std::vector<double> ref((size_t)S * H * D);
  if (oracle_decode(ref.data(), q.data(), kc.data(), vc.data(), bt.data(), ctx, S, H, D, BS, NB, max_blocks, scale, 1,
                    pairs.data(), S * H, 1) != 0) {
    std::printf("oracle decode failed\n");
    return 5;
  }
  double err = 0.0;
  for (size_t i = 0; i < out.size(); ++i) err = std::fmax(err, std::fabs((double)out[i] - ref[i]));
  std::printf("max_abs_err %.3e\n", err);

  // ---- causal prefill: the last 40 tokens of sequence 1 and the last 100 of
  // sequence 2 as query chunks over the same cache
  const int PS = 2, TQ = 140;
  const int32_t qsl[PS + 1] = {0, 40, 140};
  const int32_t pctx[PS] = {ctx[1], ctx[2]};
  std::vector<int32_t> pbt(bt.begin() + max_blocks, bt.end());
  std::vector<uint16_t> pq((size_t)TQ * H * D);
  for (auto& x : pq) x = next_half(st);
  void *dpq, *dpout;
  int32_t *dpbt, *dpctx, *dqsl;
  HIP_OK(hipMalloc(&dpq, pq.size() * 2));
  HIP_OK(hipMalloc(&dpout, (size_t)TQ * H * D * 4));
  HIP_OK(hipMalloc(&dpbt, pbt.size() * 4));
  HIP_OK(hipMalloc(&dpctx, PS * 4));
  HIP_OK(hipMalloc(&dqsl, (PS + 1) * 4));
  HIP_OK(hipMemcpy(dpq, pq.data(), pq.size() * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dpbt, pbt.data(), pbt.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dpctx, pctx, PS * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dqsl, qsl, (PS + 1) * 4, hipMemcpyHostToDevice));
  PA_OK_(pa_paged_attention_prefill(dpout, PA_F32, dpq, dkc, dvc, dpbt, dpctx, dqsl, PS, TQ, 100, H, H, D, BS, NB,
                                    max_blocks, 700, scale, PA_F16, stream));
  std::vector<float> pout((size_t)TQ * H * D);
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(pout.data(), dpout, pout.size() * 4, hipMemcpyDeviceToHost));
  std::vector<int32_t> rows;
  for (int r = 0; r < TQ; ++r)
    for (int h = 0; h < H; ++h) rows.insert(rows.end(), {r, h});
  std::vector<double> pref((size_t)TQ * H * D);
  if (oracle_prefill(pref.data(), pq.data(), kc.data(), vc.data(), pbt.data(), pctx, qsl, PS, H, D, BS, NB,
                     max_blocks, scale, 1, rows.data(), TQ * H, 1) != 0) {
    std::printf("oracle prefill failed\n");
    return 5;
  }
  double perr = 0.0;
  for (size_t i = 0; i < pout.size(); ++i) perr = std::fmax(perr, std::fabs((double)pout[i] - pref[i]));
  std::printf("prefill_max_abs_err %.3e\n", perr);

  // ---- the same work as one scheduler step: the cache write (the same rows
  // into the same slots again), the prefill and the decode
  void *dsdec, *dspf;
  HIP_OK(hipMalloc(&dsdec, (size_t)S * H * D * 4));
  HIP_OK(hipMalloc(&dspf, (size_t)TQ * H * D * 4));
  pa_step_args a;
  std::memset(&a, 0, sizeof(a));
  a.k_cache = dkc;
  a.v_cache = dvc;
  a.num_blocks = NB;
  a.num_heads = H;
  a.head_dim = D;
  a.block_size = BS;
  a.dtype = PA_F16;
  a.scale = scale;
  a.new_k = dnk;
  a.new_v = dnv;
  a.slot_mapping = dslots;
  a.num_new_tokens = S;
  a.prefill_out = dspf;
  a.prefill_out_dtype = PA_F32;
  a.prefill_q = dpq;
  a.prefill_block_tables = dpbt;
  a.prefill_context_lens = dpctx;
  a.prefill_query_start_loc = dqsl;
  a.num_prefill_seqs = PS;
  a.prefill_total_q = TQ;
  a.prefill_max_q_len = 100;
  a.prefill_max_blocks_per_seq = max_blocks;
  a.prefill_max_context_len = 700;
  a.decode_out = dsdec;
  a.decode_out_dtype = PA_F32;
  a.decode_q = dq;
  a.decode_block_tables = dbt;
  a.decode_context_lens = dctx;
  a.num_decode_seqs = S;
  a.decode_max_blocks_per_seq = max_blocks;
  a.decode_max_context_len = 700;
  a.workspace = dws;
  a.workspace_bytes = ws_bytes;
  hipStream_t side;
  hipEvent_t fork, join;
  HIP_OK(hipStreamCreate(&side));
  HIP_OK(hipEventCreateWithFlags(&fork, hipEventDisableTiming));
  HIP_OK(hipEventCreateWithFlags(&join, hipEventDisableTiming));
  int identical = 1;
  double step_err = 0.0, step_perr = 0.0;  // the step's outputs against the oracle, worst of both modes
  for (int mode = 0; mode < 2; ++mode) {
    HIP_OK(hipMemsetAsync(dsdec, 0xff, (size_t)S * H * D * 4, stream));
    HIP_OK(hipMemsetAsync(dspf, 0xff, (size_t)TQ * H * D * 4, stream));
    PA_OK_(pa_attention_step(&a, stream, mode ? side : nullptr, mode ? fork : nullptr, mode ? join : nullptr));
    HIP_OK(hipStreamSynchronize(stream));
    std::vector<float> sdec(out.size()), spf(pout.size());
    HIP_OK(hipMemcpy(sdec.data(), dsdec, sdec.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(spf.data(), dspf, spf.size() * 4, hipMemcpyDeviceToHost));
    if (std::memcmp(sdec.data(), out.data(), out.size() * 4) != 0 ||
        std::memcmp(spf.data(), pout.data(), pout.size() * 4) != 0)
      identical = 0;
    for (size_t i = 0; i < sdec.size(); ++i) step_err = std::fmax(step_err, std::fabs((double)sdec[i] - ref[i]));
    for (size_t i = 0; i < spf.size(); ++i) step_perr = std::fmax(step_perr, std::fabs((double)spf[i] - pref[i]));
  }
  // a side stream equal to the main stream is refused before anything runs
  if (pa_attention_step(&a, stream, stream, fork, join) != PA_ERR_INVALID_ARG) {
    std::printf("side stream == stream was not refused\n");
    return 4;
  }
  std::printf("step_bit_identical %d\n", identical);
  std::printf("step_max_abs_err %.3e\n", step_err);
  std::printf("step_prefill_max_abs_err %.3e\n", step_perr);
  return (err <= 2e-3 && perr <= 2e-3 && identical && step_err <= 2e-3 && step_perr <= 2e-3) ? 0 : 1;
}
