// C ABI: host-side validation and kernel dispatch. No allocation, no device
// reads; the only state kept between calls is each device's compute-unit
// count, read once.
#include <limits.h>
#include <math.h>

#include <atomic>

#include "../../include/pagedattn.h"
#include "pa_internal.h"

namespace {

using pa::Dt;

bool dtype_ok(pa_dtype d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }
int elt_bytes(pa_dtype d) { return d == PA_F32 ? 4 : 2; }
bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }
bool block_size_ok(int32_t b) { return b == 8 || b == 16 || b == 32 || b == 64; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

pa_status hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

pa_status check_cache_shape(int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            pa_dtype dtype) {
  if (num_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if ((int64_t)num_blocks * block_size > INT32_MAX) return PA_ERR_INVALID_ARG;  // slots are int32
  return PA_OK;
}

// Bytes of fp32 split-K partials (acc[head_dim], m, l) for rows x heads x
// slots, all positive; SIZE_MAX when the product does not fit in size_t
// (no launch of that size can pass validation anyway). The factors are
// below 2^31 (slots below 2^23), so the product fits 128 bits.
size_t partial_bytes(int64_t rows, int64_t heads, int64_t slots, int64_t head_dim) {
  const unsigned __int128 b = (unsigned __int128)rows * (uint64_t)heads * (uint64_t)slots *
                              (uint64_t)(head_dim + 2) * sizeof(float);
  return b > (unsigned __int128)SIZE_MAX ? SIZE_MAX : (size_t)b;
}

int64_t max_parts_for(int32_t max_context_len) { return pa::partitions_for(max_context_len, pa::kPartitionTokens); }

// Compute units of the current device (0 if it cannot be read: the caller
// then keeps its default, and the launch reports the device error). The
// count is read once per device and kept: it is a fixed property of the
// hardware, and the attribute query costs host time on every call.
int device_compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> known[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = known[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev >= 0 && dev < kMaxDevices) known[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Split-K scratch of pa_paged_attention_decode_noalloc: a file-scope device
// array, so that call allocates nothing. Every device the library runs on
// holds its own copy from module load until the process ends. In host code
// the array's name is not a device address: its device address comes from
// hipGetSymbolAddress, fetched once per device (scratch_on_device) and used
// wherever host code hands the memory to a kernel. All calls on a device
// share its copy; the partials it holds are written before they are read
// within one call, so nothing in it needs to start at zero, and calls that
// overlap on one device (different streams, no ordering) race.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

// Device address of this device's scratch (nullptr if the runtime cannot
// give it; the call then reports PA_ERR_HIP).
float* scratch_on_device() {
  constexpr int kMaxDevices = 64;
  static std::atomic<float*> known[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  float* p = known[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* sym = nullptr;
  if (hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch)) != hipSuccess || !sym) {
    (void)hipGetLastError();
    return nullptr;
  }
  p = static_cast<float*>(sym);
  known[dev].store(p, std::memory_order_release);  // racing first calls store the same address
  return p;
}

struct DecodeCall {
  pa::DecodeArgs args{};
  Dt dt;
  int D, BS;
  bool split;
};

pa_status prepare_decode(DecodeCall& call, void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
                         size_t workspace_bytes) {
  pa_status st = check_cache_shape(num_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
  if (num_kv_heads != num_heads) return PA_ERR_UNSUPPORTED;
  if (out_dtype != PA_F32 && out_dtype != dtype) return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens))
    return PA_ERR_INVALID_ARG;
  const int64_t parts = max_parts_for(max_context_len);
  bool split = parts > 1 && workspace != nullptr;
  if (split && workspace_bytes < pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len))
    return PA_ERR_WORKSPACE;
  if (split && ((uintptr_t)workspace % 16) != 0) return PA_ERR_WORKSPACE;
  const int64_t grid_parts = split ? parts : 1;
  if ((int64_t)num_seqs * num_heads * grid_parts > INT32_MAX) return PA_ERR_INVALID_ARG;
  pa::DecodeArgs& a = call.args;
  a.out = out;
  a.ws = split ? static_cast<float*>(workspace) : nullptr;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_rows = num_seqs;
  a.num_seqs = num_seqs;
  a.H = num_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.max_parts = (int)grid_parts;
  a.ws_parts = (int)grid_parts;
  // without split-K one partition spans the longest context
  a.part_tiles = split ? pa::kPartitionTokens / 16 : pa::single_partition_tiles(max_context_len);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_f32 = out_dtype == PA_F32 ? 1 : 0;
  call.dt = static_cast<Dt>(dtype);
  call.D = head_dim;
  call.BS = block_size;
  call.split = split;
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "split-K workspace missing, misaligned or too small";
    case PA_ERR_HIP: return "HIP launch failure";
    case PA_ERR_NO_BLOCKS: return "no free KV block left in the pool";
    case PA_ERR_NO_MEMORY: return "host memory allocation failed";
    case PA_ERR_PENDING_WRITES: return "copy source still has writes in the open batch: take_copies first";
    case PA_ERR_SCRATCH_LIMIT: return "request needs more split-K scratch than the allocation-free call holds (64 MiB)";
  }
  return "unknown status";
}

pa_status pa_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                               const int32_t* slot_mapping, int32_t num_tokens, int32_t num_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                               hipStream_t stream) {
  pa_status st = check_cache_shape(num_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_heads,
                                                 head_dim, block_size, num_blocks, elt_bytes(dtype), stream));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping, int32_t num_pairs,
                         int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         pa_dtype dtype, hipStream_t stream) {
  pa_status st = check_cache_shape(num_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_INVALID_ARG;
  const int64_t wgs = ((int64_t)num_heads * block_size * head_dim * elt_bytes(dtype) / 16 + 1023) / 1024;
  if ((int64_t)num_pairs * wgs > INT32_MAX) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_copy_blocks(k_cache, v_cache, block_mapping, num_pairs, num_heads, head_dim,
                                           block_size, num_blocks, elt_bytes(dtype), stream));
}

pa_status pa_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* cu_context_lens, int32_t num_seqs, int32_t max_context_len,
                       int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       int32_t max_blocks_per_seq, pa_dtype dtype, hipStream_t stream) {
  pa_status st = check_cache_shape(num_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_seqs > 65535 || max_context_len < 0 || max_blocks_per_seq <= 0)
    return PA_ERR_INVALID_ARG;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_context_len == 0) return PA_OK;
  if (!k_out || !v_out || !k_cache || !v_cache || !block_tables || !context_lens || !cu_context_lens)
    return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_gather_kv(k_out, v_out, k_cache, v_cache, block_tables, context_lens,
                                         cu_context_lens, num_seqs, max_context_len, num_heads, head_dim,
                                         block_size, max_blocks_per_seq, num_blocks, elt_bytes(dtype), stream));
}

int32_t pa_decode_partition_tokens(void) { return pa::kPartitionTokens; }

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const int64_t parts = max_parts_for(max_context_len);
  if (parts <= 1) return 0;
  return partial_bytes(num_seqs, num_heads, parts, head_dim);
}

pa_status pa_paged_attention_decode_partitions(void* out, pa_dtype out_dtype, const void* q,
                                               const void* k_cache, const void* v_cache,
                                               const int32_t* block_tables, const int32_t* context_lens,
                                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                               int32_t max_blocks_per_seq, int32_t max_context_len,
                                               float scale, pa_dtype dtype, void* workspace,
                                               size_t workspace_bytes, hipStream_t stream) {
  DecodeCall call;
  pa_status st = prepare_decode(call, out, out_dtype, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                                num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                max_context_len, scale, dtype, workspace, workspace_bytes);
  if (st != PA_OK || num_seqs == 0) return st;
  return hip_status(pa::launch_decode_partitions(call.args, call.dt, call.D, call.BS, pa::RowMode::Decode, stream));
}

pa_status pa_paged_attention_decode_reduce(void* out, pa_dtype out_dtype, const int32_t* context_lens,
                                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                           int32_t max_context_len, pa_dtype dtype, const void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  if (num_seqs < 0 || num_heads <= 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || !head_dim_ok(head_dim)) return PA_ERR_UNSUPPORTED;
  if (out_dtype != PA_F32 && out_dtype != dtype) return PA_ERR_UNSUPPORTED;
  const int64_t parts = max_parts_for(max_context_len);
  if (num_seqs == 0 || parts <= 1 || workspace == nullptr) return PA_OK;  // nothing was split
  if (workspace_bytes < pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len))
    return PA_ERR_WORKSPACE;
  if (!out || !context_lens) return PA_ERR_INVALID_ARG;
  pa::DecodeArgs a{};
  a.out = out;
  a.ws = static_cast<float*>(const_cast<void*>(workspace));
  a.context_lens = context_lens;
  a.num_rows = num_seqs;
  a.num_seqs = num_seqs;
  a.H = num_heads;
  a.max_ctx = max_context_len;
  a.num_blocks = 1;  // reads no blocks
  a.max_parts = (int)parts;
  a.ws_parts = (int)parts;
  a.part_tiles = pa::kPartitionTokens / 16;
  a.out_f32 = out_dtype == PA_F32 ? 1 : 0;
  return hip_status(pa::launch_decode_reduce(a, static_cast<Dt>(dtype), head_dim, false, stream));
}

pa_status pa_paged_attention_decode(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                    float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  DecodeCall call;
  pa_status st = prepare_decode(call, out, out_dtype, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                                num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                max_context_len, scale, dtype, workspace, workspace_bytes);
  if (st != PA_OK || num_seqs == 0) return st;
  hipError_t e = pa::launch_decode_partitions(call.args, call.dt, call.D, call.BS, pa::RowMode::Decode, stream);
  if (e == hipSuccess && call.split) e = pa::launch_decode_reduce(call.args, call.dt, call.D, false, stream);
  return hip_status(e);
}

namespace {
// The decode call of pa_paged_attention_decode_with_cache_write: a plain
// decode call that also carries the new tokens.
pa_status prepare_decode_with_cache_write(DecodeCall& call, void* out, pa_dtype out_dtype, const void* q,
                                          void* k_cache, void* v_cache, const void* new_k, const void* new_v,
                                          const int32_t* slot_mapping, const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                          int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                          float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes) {
  pa_status st = prepare_decode(call, out, out_dtype, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                                num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                max_context_len, scale, dtype, workspace, workspace_bytes);
  if (st != PA_OK || num_seqs == 0) return st;
  if (!new_k || !new_v || !slot_mapping) return PA_ERR_INVALID_ARG;
  call.args.new_k = new_k;
  call.args.new_v = new_v;
  call.args.slot_mapping = slot_mapping;
  call.args.write_in_reduce = call.split ? 1 : 0;  // K3 stores the tokens when it runs; K2 otherwise
  return PA_OK;
}
}  // namespace

pa_status pa_paged_attention_decode_with_cache_write(
    void* out, pa_dtype out_dtype, const void* q, void* k_cache, void* v_cache, const void* new_k, const void* new_v,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  DecodeCall call;
  pa_status st = prepare_decode_with_cache_write(call, out, out_dtype, q, k_cache, v_cache, new_k, new_v,
                                                 slot_mapping, block_tables, context_lens, num_seqs, num_heads,
                                                 num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                                 max_context_len, scale, dtype, workspace, workspace_bytes);
  if (st != PA_OK || num_seqs == 0) return st;
  hipError_t e = pa::launch_decode_partitions(call.args, call.dt, call.D, call.BS, pa::RowMode::Decode, stream);
  if (e == hipSuccess && call.split) e = pa::launch_decode_reduce(call.args, call.dt, call.D, false, stream);
  return hip_status(e);
}

pa_status pa_paged_attention_decode_with_cache_write_partitions(
    void* out, pa_dtype out_dtype, const void* q, void* k_cache, void* v_cache, const void* new_k, const void* new_v,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  DecodeCall call;
  pa_status st = prepare_decode_with_cache_write(call, out, out_dtype, q, k_cache, v_cache, new_k, new_v,
                                                 slot_mapping, block_tables, context_lens, num_seqs, num_heads,
                                                 num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                                 max_context_len, scale, dtype, workspace, workspace_bytes);
  if (st != PA_OK || num_seqs == 0) return st;
  return hip_status(pa::launch_decode_partitions(call.args, call.dt, call.D, call.BS, pa::RowMode::Decode, stream));
}

pa_status pa_paged_attention_decode_with_cache_write_reduce(
    void* out, pa_dtype out_dtype, const void* q, void* k_cache, void* v_cache, const void* new_k, const void* new_v,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  DecodeCall call;
  pa_status st = prepare_decode_with_cache_write(call, out, out_dtype, q, k_cache, v_cache, new_k, new_v,
                                                 slot_mapping, block_tables, context_lens, num_seqs, num_heads,
                                                 num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                                 max_context_len, scale, dtype, workspace, workspace_bytes);
  if (st != PA_OK || num_seqs == 0 || !call.split) return st;
  return hip_status(pa::launch_decode_reduce(call.args, call.dt, call.D, false, stream));
}

size_t pa_decode_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

pa_status pa_paged_attention_decode_noalloc(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                                            const void* v_cache, const int32_t* block_tables,
                                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                            int32_t num_blocks, int32_t max_blocks_per_seq,
                                            int32_t max_context_len, float scale, pa_dtype dtype,
                                            hipStream_t stream) {
  // the scratch a split-K launch of this size needs must fit the built-in array
  const size_t need = pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len);
  if (need > kNoAllocScratchBytes) return PA_ERR_SCRATCH_LIMIT;
  float* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_device();
    if (!ws) return PA_ERR_HIP;
  }
  DecodeCall call;
  pa_status st = prepare_decode(call, out, out_dtype, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                                num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                max_context_len, scale, dtype, ws, need);
  if (st != PA_OK || num_seqs == 0) return st;
  hipError_t e = pa::launch_decode_partitions(call.args, call.dt, call.D, call.BS, pa::RowMode::Decode, stream);
  if (e == hipSuccess && call.split) e = pa::launch_decode_reduce(call.args, call.dt, call.D, false, stream);
  return hip_status(e);
}

size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t max_context_len) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  // shared + own partitions of one row: ceil(p / shared) + ceil((ctx - p) / own) for a prefix of p
  // tokens, at most ceil(ctx / own) + 1 as shared partitions are no shorter than own ones
  const int64_t slots = max_parts_for(max_context_len) + 1;
  return partial_bytes(num_seqs, num_heads, slots, head_dim);
}

pa_status pa_paged_attention_decode_shared_prefix(
    void* out, pa_dtype out_dtype, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_starts,
    const int32_t* prefix_lens, int32_t num_groups, int32_t max_group_size, int32_t max_prefix_len,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pa_status st = check_cache_shape(num_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_groups < 0 || max_group_size < 0 ||
      max_prefix_len < 0 || max_prefix_len > max_context_len)
    return PA_ERR_INVALID_ARG;
  if (num_kv_heads != num_heads) return PA_ERR_UNSUPPORTED;
  if (out_dtype != PA_F32 && out_dtype != dtype) return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (num_groups < 1 || num_groups > num_seqs || max_group_size < 1 || max_group_size > num_seqs)
    return PA_ERR_INVALID_ARG;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !group_starts || !prefix_lens)
    return PA_ERR_INVALID_ARG;
  const size_t need = pa_decode_shared_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 16) != 0) return PA_ERR_WORKSPACE;
  const int64_t parts = max_parts_for(max_context_len);
  if ((int64_t)num_seqs * num_heads * parts > INT32_MAX) return PA_ERR_INVALID_ARG;
  pa::DecodeArgs a{};
  a.out = out;
  a.ws = static_cast<float*>(workspace);
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_rows = num_seqs;
  a.num_seqs = num_seqs;
  a.H = num_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.num_blocks = num_blocks;
  a.ws_parts = (int)parts + 1;
  a.part_tiles = pa::kPartitionTokens / 16;
  a.shared_part_tiles = pa::shared_partition_tokens(block_size) / 16;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_f32 = out_dtype == PA_F32 ? 1 : 0;
  a.group_starts = group_starts;
  a.prefix_lens = prefix_lens;
  a.num_groups = num_groups;
  const Dt dt = static_cast<Dt>(dtype);
  hipError_t e = hipSuccess;
  if (dtype != PA_F32 && max_prefix_len > 0) {
    a.member_chunks = (int)ceil_div(max_group_size, pa::kSharedMembersPerWave);
    const int64_t shared_parts = ceil_div(max_prefix_len, pa::shared_partition_tokens(block_size));
    if ((int64_t)num_groups * a.member_chunks * num_heads * shared_parts + (int64_t)num_seqs * num_heads * parts >
        INT32_MAX)
      return PA_ERR_INVALID_ARG;
    a.max_parts = (int)parts;
    e = pa::launch_shared_prefix_step(a, dt, head_dim, block_size, (int)shared_parts, (int)parts, stream);
    if (e == hipSuccess) e = pa::launch_decode_reduce(a, dt, head_dim, true, stream);
  } else {
    // nothing shared to exploit (or f32): the ordinary split-K decode
    a.max_parts = (int)parts;
    e = pa::launch_decode_partitions(a, dt, head_dim, block_size, pa::RowMode::Decode, stream);
    if (e == hipSuccess) e = pa::launch_decode_reduce(a, dt, head_dim, false, stream);
  }
  return hip_status(e);
}

// Validated launch plan of one prefill call: the MFMA kernel of its dtype.
struct PrefillCall {
  bool empty = true;
  pa::PrefillArgs pf{};
  Dt dt = Dt::F16;
  int D = 0, BS = 0;
};

static pa_status prepare_prefill(PrefillCall& call, void* out, pa_dtype out_dtype, const void* q,
                                 const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_seqs,
                                 int32_t total_q, int32_t max_q_len, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype) {
  pa_status st = check_cache_shape(num_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_kv_heads != num_heads) return PA_ERR_UNSUPPORTED;
  if (out_dtype != PA_F32 && out_dtype != dtype) return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_INVALID_ARG;
  if (max_q_len > max_context_len || (num_seqs > 0 && total_q > (int64_t)num_seqs * max_q_len))
    return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  call.empty = num_seqs == 0 || total_q == 0;
  if (call.empty) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return PA_ERR_INVALID_ARG;
  call.dt = static_cast<Dt>(dtype);
  call.D = head_dim;
  call.BS = block_size;
  pa::PrefillArgs& a = call.pf;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.H = num_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_blocks = num_blocks;
  a.q_tiles = (int)ceil_div(max_q_len, pa::prefill_mfma_q_tile());
  // a negative scale runs as |scale| on negated queries (a sign flip, exact)
  a.scale_log2 = std::fabs(scale) * 1.4426950408889634f;
  a.q_sign = std::signbit(scale) ? 0x80008000u : 0u;
  a.out_f32 = out_dtype == PA_F32 ? 1 : 0;
  if ((int64_t)a.q_tiles * num_heads * (num_seqs + 7) > INT32_MAX) return PA_ERR_INVALID_ARG;
  // more workgroups than the chip holds at once: group each pair's query
  // tiles for L2 reuse (the kernel's work-order note)
  const int cus = device_compute_units();
  a.cus = cus;
  const int per_cu = dtype == PA_F32 ? pa::kPrefillF32WorkgroupsPerCU : pa::kPrefillWorkgroupsPerCU;
  a.grouped = cus > 0 && (int64_t)a.q_tiles * num_heads * num_seqs > (int64_t)cus * per_cu;
  a.wide = !a.grouped;  // every workgroup resident at once
  return PA_OK;
}

static hipError_t launch_prefill(const PrefillCall& call, hipStream_t stream) {
  if (call.empty) return hipSuccess;
  if (call.dt == Dt::F32) return pa::launch_prefill_f32(call.pf, call.D, call.BS, stream);
  return pa::launch_prefill_mfma(call.pf, call.dt, call.D, call.BS, stream);
}

pa_status pa_paged_attention_prefill(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, const int32_t* query_start_loc,
                                     int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t num_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                     float scale, pa_dtype dtype, hipStream_t stream) {
  PrefillCall call;
  pa_status st = prepare_prefill(call, out, out_dtype, q, k_cache, v_cache, block_tables, context_lens,
                                 query_start_loc, num_seqs, total_q, max_q_len, num_heads, num_kv_heads, head_dim,
                                 block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype);
  if (st != PA_OK) return st;
  return hip_status(launch_prefill(call, stream));
}

pa_status pa_attention_step(const pa_step_args* s, hipStream_t stream, hipStream_t side_stream,
                            hipEvent_t fork_event, hipEvent_t join_event) {
  if (!s) return PA_ERR_INVALID_ARG;
  // validate every part before anything is launched
  pa_status st = check_cache_shape(s->num_heads, s->head_dim, s->block_size, s->num_blocks, s->dtype);
  if (st != PA_OK) return st;
  if (s->num_new_tokens < 0 || s->num_prefill_seqs < 0 || s->num_decode_seqs < 0) return PA_ERR_INVALID_ARG;
  if (s->num_new_tokens > 0 && (!s->new_k || !s->new_v || !s->k_cache || !s->v_cache || !s->slot_mapping))
    return PA_ERR_INVALID_ARG;
  PrefillCall pf;
  if (s->num_prefill_seqs > 0) {
    st = prepare_prefill(pf, s->prefill_out, s->prefill_out_dtype, s->prefill_q, s->k_cache, s->v_cache,
                         s->prefill_block_tables, s->prefill_context_lens, s->prefill_query_start_loc,
                         s->num_prefill_seqs, s->prefill_total_q, s->prefill_max_q_len, s->num_heads, s->num_heads,
                         s->head_dim, s->block_size, s->num_blocks, s->prefill_max_blocks_per_seq,
                         s->prefill_max_context_len, s->scale, s->dtype);
    if (st != PA_OK) return st;
  }
  DecodeCall dc;
  const bool decode = s->num_decode_seqs > 0;
  if (decode) {
    st = prepare_decode(dc, s->decode_out, s->decode_out_dtype, s->decode_q, s->k_cache, s->v_cache,
                        s->decode_block_tables, s->decode_context_lens, s->num_decode_seqs, s->num_heads,
                        s->num_heads, s->head_dim, s->block_size, s->num_blocks, s->decode_max_blocks_per_seq,
                        s->decode_max_context_len, s->scale, s->dtype, s->workspace, s->workspace_bytes);
    if (st != PA_OK) return st;
  }
  const bool prefill = !pf.empty;
  const bool fork = prefill && decode && side_stream != nullptr;
  if (fork && (side_stream == stream || !fork_event || !join_event)) return PA_ERR_INVALID_ARG;

  hipError_t e = hipSuccess;
  if (s->num_new_tokens > 0)
    e = pa::launch_reshape_and_cache(s->new_k, s->new_v, s->k_cache, s->v_cache, s->slot_mapping, s->num_new_tokens,
                                     s->num_heads, s->head_dim, s->block_size, s->num_blocks, elt_bytes(s->dtype),
                                     stream);
  if (e != hipSuccess) return hip_status(e);
  if (fork) {
    // the prefill runs on the side stream next to the decode: both only read
    // the cache the write above produced. Next to the decode's waves the
    // prefill's 4-wave workgroups find room sooner than 8-wave ones (the
    // mixed step: 742 against 772 us), so it keeps its standard shape.
    pf.pf.wide = 0;
    e = hipEventRecord(fork_event, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(side_stream, fork_event, 0);
    if (e == hipSuccess) e = launch_prefill(pf, side_stream);
    if (e == hipSuccess) e = pa::launch_decode_partitions(dc.args, dc.dt, dc.D, dc.BS, pa::RowMode::Decode, stream);
    if (e == hipSuccess && dc.split) e = pa::launch_decode_reduce(dc.args, dc.dt, dc.D, false, stream);
    if (e == hipSuccess) e = hipEventRecord(join_event, side_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, join_event, 0);
    return hip_status(e);
  }
  if (prefill) e = launch_prefill(pf, stream);
  if (e == hipSuccess && decode) {
    e = pa::launch_decode_partitions(dc.args, dc.dt, dc.D, dc.BS, pa::RowMode::Decode, stream);
    if (e == hipSuccess && dc.split) e = pa::launch_decode_reduce(dc.args, dc.dt, dc.D, false, stream);
  }
  return hip_status(e);
}

}  // extern "C"
