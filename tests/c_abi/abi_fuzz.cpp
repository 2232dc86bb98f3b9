// The host side of the C ABI (argument validation, launch plans, sizing,
// status strings) driven with bad and extreme arguments, for a build whose
// host code carries AddressSanitizer and UndefinedBehaviorSanitizer. It
// passes fake device pointers, so it runs only where no GPU is visible (the
// launches that pass validation then fail in the runtime, and nothing is
// executed); elsewhere it prints "skip: ..." and exits 0. Prints
// "abi_fuzz ok <calls>" and exits 0 when every call returned a known status
// without a sanitizer report.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "pagedattn.h"

#define CHECK(c)                                                \
  do {                                                          \
    if (!(c)) {                                                 \
      std::printf("FAIL line %d: %s\n", __LINE__, #c);          \
      std::exit(1);                                             \
    }                                                           \
  } while (0)

static uint64_t st = 0x391;
static uint32_t rnd(uint32_t n) {  // xorshift64*, test data only
  st ^= st >> 12;
  st ^= st << 25;
  st ^= st >> 27;
  return (uint32_t)((st * 2685821657736338717ull) >> 33) % n;
}
static const int32_t kVals[] = {INT_MIN, -7, -1, 0, 1, 2, 8, 16, 32, 64, 96, 128, 512, 4096, 65536, INT_MAX};
static int32_t v() { return kVals[rnd(sizeof(kVals) / sizeof(kVals[0]))]; }
static void* const kFake = (void*)0x1000;
static void* p() { return rnd(4) == 0 ? nullptr : kFake; }
// every value an enum of these enumerators can hold in C++ (0..3 and -8..7):
// 3 is no dtype, 1..7 and -8 are no status
static pa_dtype dt() { return (pa_dtype)rnd(4); }
static float f() {
  const float s[] = {0.f, -1.f, 0.088f, 1e30f, __builtin_inff(), __builtin_nanf("")};
  return s[rnd(6)];
}
static bool known(pa_status s) { return s <= PA_OK && s >= PA_ERR_SCRATCH_LIMIT; }

int main() {
  int n = 0;
  const hipError_t e = hipGetDeviceCount(&n);
  (void)hipGetLastError();
  if (e == hipSuccess && n > 0) {
    std::printf("skip: a GPU is visible and this program passes fake device pointers\n");
    return 0;
  }
  long calls = 0;
  for (int c = -8; c <= 7; ++c, ++calls) CHECK(pa_status_string((pa_status)c) != nullptr);
  // sizing: pure functions of their arguments, 0 for non-positive sizes
  for (int32_t a : kVals)
    for (int32_t b : kVals)
      for (int32_t d : kVals)
        for (int32_t m : kVals) {
          const size_t w = pa_decode_workspace_bytes(a, b, d, m);
          const size_t ws = pa_decode_shared_workspace_bytes(a, b, d, m);
          if (a <= 0 || b <= 0 || d <= 0 || m <= 0) CHECK(w == 0 && ws == 0);
          if (w != 0 && w != SIZE_MAX) CHECK(ws > w);
          calls += 2;
        }
  CHECK(pa_decode_partition_tokens() > 0 && pa_decode_noalloc_scratch_bytes() > 0);
  for (int it = 0; it < 20000; ++it) {
    pa_status s = PA_OK;
    switch (rnd(12)) {
      case 0:
        s = pa_reshape_and_cache(p(), p(), p(), p(), (const int32_t*)p(), v(), v(), v(), v(), v(), dt(), nullptr);
        break;
      case 1:
        s = pa_copy_blocks(p(), p(), (const int32_t*)p(), v(), v(), v(), v(), v(), dt(), nullptr);
        break;
      case 2:
        s = pa_gather_kv(p(), p(), p(), p(), (const int32_t*)p(), (const int32_t*)p(), (const int32_t*)p(), v(), v(),
                         v(), v(), v(), v(), v(), dt(), nullptr);
        break;
      case 3:
        s = pa_paged_attention_decode(p(), dt(), p(), p(), p(), (const int32_t*)p(), (const int32_t*)p(), v(), v(),
                                      v(), v(), v(), v(), v(), v(), f(), dt(), p(), (size_t)(uint32_t)v(), nullptr);
        break;
      case 4:
        s = pa_paged_attention_decode_noalloc(p(), dt(), p(), p(), p(), (const int32_t*)p(), (const int32_t*)p(), v(),
                                              v(), v(), v(), v(), v(), v(), v(), f(), dt(), nullptr);
        break;
      case 5:
        s = pa_paged_attention_decode_reduce(p(), dt(), (const int32_t*)p(), v(), v(), v(), v(), dt(), p(),
                                             (size_t)(uint32_t)v(), nullptr);
        break;
      case 6:
        s = pa_paged_attention_decode_shared_prefix(p(), dt(), p(), p(), p(), (const int32_t*)p(), (const int32_t*)p(),
                                                    (const int32_t*)p(), (const int32_t*)p(), v(), v(), v(), v(), v(),
                                                    v(), v(), v(), v(), v(), v(), f(), dt(), p(),
                                                    (size_t)(uint32_t)v(), nullptr);
        break;
      case 8:
        s = pa_paged_attention_decode_with_cache_write(p(), dt(), p(), p(), p(), p(), p(), (const int32_t*)p(),
                                                       (const int32_t*)p(), (const int32_t*)p(), v(), v(), v(), v(),
                                                       v(), v(), v(), v(), f(), dt(), p(), (size_t)(uint32_t)v(),
                                                       nullptr);
        break;
      case 10:
        s = pa_paged_attention_decode_with_cache_write_reduce(
            p(), dt(), p(), p(), p(), p(), p(), (const int32_t*)p(), (const int32_t*)p(), (const int32_t*)p(), v(),
            v(), v(), v(), v(), v(), v(), v(), f(), dt(), p(), (size_t)(uint32_t)v(), nullptr);
        break;
      case 9:
        s = pa_paged_attention_decode_with_cache_write_partitions(
            p(), dt(), p(), p(), p(), p(), p(), (const int32_t*)p(), (const int32_t*)p(), (const int32_t*)p(), v(),
            v(), v(), v(), v(), v(), v(), v(), f(), dt(), p(), (size_t)(uint32_t)v(), nullptr);
        break;
      case 7:
        s = pa_paged_attention_prefill(p(), dt(), p(), p(), p(), (const int32_t*)p(), (const int32_t*)p(),
                                       (const int32_t*)p(), v(), v(), v(), v(), v(), v(), v(), v(), v(), v(), f(), dt(),
                                       nullptr);
        break;
      default: {
        pa_step_args a;
        a.k_cache = p(); a.v_cache = p();
        a.num_blocks = v(); a.num_heads = v(); a.head_dim = v(); a.block_size = v();
        a.dtype = dt(); a.scale = f();
        a.new_k = p(); a.new_v = p(); a.slot_mapping = (const int32_t*)p(); a.num_new_tokens = v();
        a.prefill_out = p(); a.prefill_out_dtype = dt(); a.prefill_q = p();
        a.prefill_block_tables = (const int32_t*)p(); a.prefill_context_lens = (const int32_t*)p();
        a.prefill_query_start_loc = (const int32_t*)p();
        a.num_prefill_seqs = v(); a.prefill_total_q = v(); a.prefill_max_q_len = v();
        a.prefill_max_blocks_per_seq = v(); a.prefill_max_context_len = v();
        a.decode_out = p(); a.decode_out_dtype = dt(); a.decode_q = p();
        a.decode_block_tables = (const int32_t*)p(); a.decode_context_lens = (const int32_t*)p();
        a.num_decode_seqs = v(); a.decode_max_blocks_per_seq = v(); a.decode_max_context_len = v();
        a.workspace = p(); a.workspace_bytes = (size_t)(uint32_t)v();
        // a fake side stream comes without events, so the call refuses the
        // fork before touching either (a call without a fork never uses it)
        const bool side = rnd(2) != 0;
        s = pa_attention_step(rnd(8) ? &a : nullptr, nullptr, side ? (hipStream_t)kFake : nullptr, nullptr,
                              nullptr);
        break;
      }
    }
    CHECK(known(s));
    ++calls;
  }
  std::printf("abi_fuzz ok %ld\n", calls);
  return 0;
}
