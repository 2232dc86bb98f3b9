/*
 * pagedattn.h -- C ABI of a gfx950 (MI355X) library for attention over a
 * paged KV cache.
 *
 * The method (devpress.csdn.net page, sections "PagedAttention 是如何工作的"
 * and "分页式KV缓存"; aidocs.cortexgrid.cn page, intro bullets and FAQ;
 * betteryeah.com page, sections 2.2 and 2.4): the KV cache of every sequence
 * is cut into fixed-size blocks of block_size tokens (16 or 32) that may sit
 * anywhere in one pool; a per-sequence block table maps logical block i to a
 * physical block; attention follows the table across the scattered blocks.
 * Sequences that share a prefix (parallel sampling) list the same physical
 * blocks in their tables; the kernels only read them.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller. The kernel
 *    calls allocate nothing, keep no pointer after returning and are safe
 *    to call from several host threads; the only state they keep is each
 *    device's compute-unit count, read once (atomically) on first use. The
 *    block allocator (pa_allocator_*) keeps its host-side state in a handle
 *    the caller creates and destroys.
 *  - Work is queued on `stream` and never synchronised; the library never
 *    reads device memory on the host.
 *  - Validation is host-side on scalars and pointer nullness only; a failed
 *    check returns an error before anything is launched. Data preconditions
 *    (listed per call) are the caller's duty and are not checked on device.
 *  - Layouts (row-major, contiguous):
 *      k_cache, v_cache  [num_blocks][num_heads][block_size][head_dim]
 *      block_tables      int32 [num_seqs][max_blocks_per_seq]
 *      q, out            [rows][num_heads][head_dim]
 *    A slot is block * block_size + offset.
 *  - Supported: head_dim 64 or 128, block_size 8, 16, 32 or 64 (the pages
 *    use 16 or 32 and advise against more than 64), num_kv_heads ==
 *    num_heads, dtype f32/f16/bf16; out_dtype is PA_F32 or equal to dtype.
 *    Accumulation is fp32; a narrower output is rounded to nearest even from
 *    the fp32 result.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, inconsistent sizes */
  PA_ERR_UNSUPPORTED = -2, /* head_dim, block_size, dtype or head layout not built */
  PA_ERR_WORKSPACE = -3,   /* split-K workspace missing or too small */
  PA_ERR_HIP = -4,         /* a launch failed; hipGetLastError() was cleared */
  PA_ERR_NO_BLOCKS = -5,   /* block allocator: not enough free blocks (nothing was changed) */
  PA_ERR_NO_MEMORY = -6,   /* block allocator: host memory allocation failed */
  PA_ERR_PENDING_WRITES = -7, /* block allocator: the copy source still has writes in the open batch */
  PA_ERR_SCRATCH_LIMIT = -8   /* allocation-free decode: the request needs more than its built-in scratch */
} pa_status;

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* Human-readable name of a status code (static storage). */
const char* pa_status_string(pa_status status);

/*
 * reshape_and_cache -- write this step's new tokens into their cache slots.
 * New tokens get slots in blocks handed out on demand (devpress page,
 * "实际收益远超预期" and workflow step "分页加载"; betteryeah page, section
 * 2.2). For every n < num_tokens with slot_mapping[n] >= 0 and every head h:
 *   k_cache[slot/bs][h][slot%bs][:] = k[n][h][:]   (same for v)
 * bit for bit. Rows with a negative slot are skipped; every other cache slot
 * is left untouched.
 *   k, v          [num_tokens][num_heads][head_dim], dtype
 *   slot_mapping  int32 [num_tokens]
 * Preconditions: non-negative slots are distinct and < num_blocks*block_size
 * (a slot past the pool is skipped on the device). num_tokens == 0 is a
 * no-op. Errors: INVALID_ARG (null pointer, sizes,
 * num_blocks*block_size > INT32_MAX), UNSUPPORTED, HIP.
 */
pa_status pa_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                               const int32_t* slot_mapping, int32_t num_tokens, int32_t num_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                               hipStream_t stream);

/*
 * copy_blocks -- the copy half of copy-on-write. Parallel samples share the
 * prompt's blocks through their block tables, each block carrying a
 * reference count; before a sharer writes into a shared block it gets a
 * private copy (aidocs.cortexgrid.cn page, FAQ answer on parallel
 * sampling). For every pair i < num_pairs:
 *   k_cache[map[i][1]] = k_cache[map[i][0]]   (all heads and offsets; same for v)
 * bit for bit.
 *   block_mapping  int32 [num_pairs][2] (src, dst), device memory
 * Preconditions: destinations are distinct and none is also a source (the
 * copies run concurrently). Pairs naming a block outside [0, num_blocks)
 * are skipped on the device. num_pairs == 0 is a no-op.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping, int32_t num_pairs,
                         int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         pa_dtype dtype, hipStream_t stream);

/*
 * Block allocator -- host-side bookkeeping of the physical blocks (no device
 * memory is touched). Blocks are handed out on demand as sequences grow and
 * returned when they finish (devpress page, workflow step on memory
 * reclamation; betteryeah page, section 2.2); a fork shares every block of
 * its parent and raises their reference counts; appending to a sequence
 * whose partly filled last block is shared first moves it to a fresh block
 * and queues the (old, fresh) pair for pa_copy_blocks (aidocs page, FAQ on
 * parallel sampling). Free blocks form a LIFO stack that starts with block 0.
 * The handle is owned by the caller; one host thread at a time per handle.
 *
 *   create        num_blocks, block_size > 0, num_blocks*block_size <= INT32_MAX
 *   new_sequence  returns an empty sequence id (ids are never reused)
 *   fork          child shares all of parent's blocks (refcount + 1 each)
 *   append        reserves num_tokens slots at the end of seq and writes their
 *                 slot ids (block * block_size + offset) to slots (NULL: don't);
 *                 NO_BLOCKS, with no state changed, if the pool is too small
 *   free_sequence releases seq's blocks (a block returns to the pool when its
 *                 count reaches 0); the id becomes invalid
 *   block_table   copies seq's table into table[capacity] and sets
 *                 *num_blocks; capacity 0 only queries the size; a smaller
 *                 non-zero capacity is INVALID_ARG
 *   take_copies   moves up to capacity pending (src, dst) pairs into
 *                 pairs[capacity][2], oldest first, and sets *num_pairs;
 *                 capacity 0 only queries how many are pending. A call
 *                 with capacity > 0 that leaves nothing pending closes the
 *                 open batch (below).
 *   num_free / refcount / sequence_length return -1 for a bad handle, block or id.
 *
 * Batches: the calls of one scheduler step form a batch. Close it with
 * take_copies (capacity > 0, even when nothing is pending), then queue on
 * one stream, in this order: pa_copy_blocks of the pairs it returned, then
 * pa_reshape_and_cache of every slot the batch's appends handed out. The
 * allocator guarantees that the pairs of one batch have distinct
 * destinations, that no destination is also a source, and that no source
 * receives slots in the same batch (so the copies see its final contents):
 *   - append returns PA_ERR_PENDING_WRITES, changing nothing, when it would
 *     copy a shared last block that received slots in the open batch (its
 *     new tokens are not written yet); close the batch and append again;
 *   - a block whose count drops to 0 while it received slots or is a copy
 *     source in the open batch returns to the pool when the batch closes
 *     (num_free counts it from then on).
 * Errors: INVALID_ARG (null pointer, bad id, size), NO_BLOCKS, NO_MEMORY,
 * PENDING_WRITES.
 */
typedef struct pa_allocator pa_allocator;
pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size, pa_allocator** out);
void pa_allocator_destroy(pa_allocator* a);
int32_t pa_allocator_num_free(const pa_allocator* a);
int32_t pa_allocator_refcount(const pa_allocator* a, int32_t block);
pa_status pa_allocator_new_sequence(pa_allocator* a, int32_t* seq);
pa_status pa_allocator_fork(pa_allocator* a, int32_t parent, int32_t* child);
pa_status pa_allocator_append(pa_allocator* a, int32_t seq, int32_t num_tokens, int32_t* slots);
pa_status pa_allocator_free_sequence(pa_allocator* a, int32_t seq);
int32_t pa_allocator_sequence_length(const pa_allocator* a, int32_t seq);
pa_status pa_allocator_block_table(const pa_allocator* a, int32_t seq, int32_t* table, int32_t capacity,
                                   int32_t* num_blocks);
pa_status pa_allocator_take_copies(pa_allocator* a, int32_t* pairs, int32_t capacity, int32_t* num_pairs);

/*
 * gather_kv -- materialise each sequence's logical K and V contiguously
 * through its block table (the translation every attention kernel uses).
 * The pages define the translation: each logical page of a sequence maps to
 * a physical block through a page table, and the kernel stitches the
 * scattered blocks into the stream attention reads (devpress page, section
 * "分页式KV缓存：让显存利用接近理论极限"; betteryeah page, section 2.2, pages
 * stored anywhere and reached through the table). This call performs only
 * that stitching:
 *   k_out[cu_context_lens[s] + t][h][:] = k_cache[bt[s][t/bs]][h][t%bs][:]
 * for t < context_lens[s]; same for v. Bit-exact copy, for checking the
 * table translation and for debugging.
 *   cu_context_lens  int32 [num_seqs+1], exclusive prefix sum of context_lens
 *   max_context_len  >= every context_lens[s] (sizes the grid)
 * Preconditions: table entries below ceil(ctx/bs) are valid block ids.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
pa_status pa_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* cu_context_lens, int32_t num_seqs, int32_t max_context_len,
                       int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       int32_t max_blocks_per_seq, pa_dtype dtype, hipStream_t stream);

/*
 * Split-K sizing for decode. The pages do not describe splitting one
 * sequence's attention: they only say that long contexts (4K tokens and
 * more) are where paging pays most (betteryeah page, section 3.3, long
 * sequences) and configure contexts of up to 4096 tokens (devpress page,
 * the max_model_len setting in the example after "实际收益远超预期"). Cutting
 * such contexts into partitions that run in parallel and are merged by a
 * separate reduction is this library's design for keeping every compute
 * unit busy when a batch holds few long sequences.
 * Contexts are cut into partitions of pa_decode_partition_tokens() tokens
 * (a whole number of blocks). The workspace holds fp32 partials (m, l,
 * acc[head_dim]) for every (sequence, head, partition):
 * pa_decode_workspace_bytes() bytes, or 0 when max_context_len fits one
 * partition (then no workspace is needed). Both are pure functions of their
 * arguments; pa_decode_workspace_bytes returns 0 for non-positive sizes and
 * SIZE_MAX for sizes whose partials would not fit in size_t.
 */
int32_t pa_decode_partition_tokens(void);
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len);

/*
 * paged_attention_decode -- one step of autoregressive decoding: the new
 * token of each sequence attends to the K/V cached for every earlier token
 * (devpress page, "PagedAttention 是如何工作的": decoding reuses the cached
 * Key/Value vectors), read from blocks scattered through the pool by
 * following the sequence's page table (devpress page, "分页式KV缓存"; betteryeah
 * page, section 2.4, attention across pages; section 2.1, L x d values per
 * head and sequence). The pages do not write the attention formula; the
 * reading used is scaled dot-product softmax attention over all of its
 * context_lens[s] cached tokens (the current token included: it is written by
 * pa_reshape_and_cache first):
 *   out[s][h] = softmax_t(scale * <q[s][h], K_t>) . V_t,  t < context_lens[s]
 * with K_t, V_t read through block_tables[s].
 *   q           [num_seqs][num_heads][head_dim], dtype
 *   out         [num_seqs][num_heads][head_dim], out_dtype
 *   workspace   NULL disables split-K (one partition per sequence); otherwise
 *               at least pa_decode_workspace_bytes(...) bytes, fp32-aligned.
 * context_lens[s] == 0 gives a zero output row.
 * Preconditions: context_lens[s] <= max_context_len <= max_blocks_per_seq *
 * block_size; table entries below ceil(ctx/bs) are valid block ids; entries
 * past them, and cache slots past a context, are never read.
 * Launches K2 (partitions) and, when any partial exists, K3 (reduction).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
pa_status pa_paged_attention_decode(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                    float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * paged_attention_decode_with_cache_write -- a decode step's cache write and
 * attention in one launch. A decode step appends each sequence's new token
 * to its last block and then attends over everything cached (devpress page,
 * workflow steps "分页加载" and the PagedAttention section; betteryeah page,
 * section 2.2 for the on-demand blocks, 2.4 for attention across pages).
 * Here the wave of the partition kernel that holds position
 * context_lens[s] - 1 takes row s's new token from new_k / new_v instead of
 * the cache, so no cache-write launch has to finish first, and the call
 * writes new_k[s] and new_v[s] into slot slot_mapping[s] exactly as
 * pa_reshape_and_cache puts them (negative slots and slots past the pool
 * are skipped): the reduction kernel does, when the call is split, else
 * the partition kernel.
 *   new_k, new_v   [num_seqs][num_heads][head_dim], dtype
 *   slot_mapping   int32 [num_seqs]
 *   k_cache, v_cache are written (the new tokens' slots only).
 * Other arguments, layouts and errors as for pa_paged_attention_decode; also
 * INVALID_ARG for a null new_k, new_v or slot_mapping.
 * Precondition beyond those of pa_paged_attention_decode: a non-negative
 * slot_mapping[s] is the slot of position context_lens[s] - 1 in row s's
 * table, read by no other row, and no two rows share a slot (as in a decode
 * step; a negative one means the row has no new token and reads the cache
 * as it is). Then out and the caches equal, bit for bit, those of
 * pa_reshape_and_cache(new_k, new_v, ..., slot_mapping, num_seqs) followed
 * by pa_paged_attention_decode.
 */
pa_status pa_paged_attention_decode_with_cache_write(
    void* out, pa_dtype out_dtype, const void* q, void* k_cache, void* v_cache, const void* new_k, const void* new_v,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_noalloc -- pa_paged_attention_decode with split-K
 * always on and no workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The split-K partials live in a scratch
 * array built into the library: pa_decode_noalloc_scratch_bytes() bytes
 * (64 MiB) per device, held from the library's load until the process ends.
 * The call allocates nothing and gives the same result, bit for bit, as
 * pa_paged_attention_decode with a workspace. Every call on a device shares
 * that device's array: calls that may overlap on one device (different
 * streams with no ordering between them) race and must not be issued.
 * Arguments as for pa_paged_attention_decode, without workspace and
 * workspace_bytes. Errors: those of pa_paged_attention_decode except
 * WORKSPACE, and SCRATCH_LIMIT when pa_decode_workspace_bytes(num_seqs,
 * num_heads, head_dim, max_context_len) exceeds the scratch (nothing is
 * launched); HIP if the scratch's device address cannot be obtained.
 */
size_t pa_decode_noalloc_scratch_bytes(void);
pa_status pa_paged_attention_decode_noalloc(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                                            const void* v_cache, const int32_t* block_tables,
                                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                            int32_t num_blocks, int32_t max_blocks_per_seq,
                                            int32_t max_context_len, float scale, pa_dtype dtype,
                                            hipStream_t stream);

/*
 * The two stages of pa_paged_attention_decode, for callers that schedule or
 * time them separately (the split-K design described above; not from the
 * pages). _partitions takes the same arguments and launches K2 only; _reduce
 * then merges the partials of rows with more than one partition, with
 * log-sum-exp weights: M = max_p m_p, out = sum_p acc_p 2^(m_p - M) /
 * sum_p l_p 2^(m_p - M). Together they equal pa_paged_attention_decode bit
 * for bit. _reduce needs the same workspace, context_lens and
 * max_context_len as the _partitions call it follows; it returns PA_OK
 * without launching when nothing was split (no workspace, or one partition).
 */
pa_status pa_paged_attention_decode_partitions(void* out, pa_dtype out_dtype, const void* q,
                                               const void* k_cache, const void* v_cache,
                                               const int32_t* block_tables, const int32_t* context_lens,
                                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                               int32_t max_blocks_per_seq, int32_t max_context_len,
                                               float scale, pa_dtype dtype, void* workspace,
                                               size_t workspace_bytes, hipStream_t stream);
pa_status pa_paged_attention_decode_reduce(void* out, pa_dtype out_dtype, const int32_t* context_lens,
                                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                           int32_t max_context_len, pa_dtype dtype, const void* workspace,
                                           size_t workspace_bytes, hipStream_t stream);
/*
 * The two stages of pa_paged_attention_decode_with_cache_write, both with
 * its arguments: _partitions launches K2 (which uses the new tokens, and
 * writes them into their slots itself when no reduction follows), _reduce
 * launches K3 (which merges the partials and writes the new tokens) when the
 * call is split, and returns PA_OK without launching otherwise. Together they
 * equal pa_paged_attention_decode_with_cache_write bit for bit, outputs and
 * caches; pa_paged_attention_decode_reduce does not write the tokens and is
 * no substitute for _reduce here.
 */
pa_status pa_paged_attention_decode_with_cache_write_partitions(
    void* out, pa_dtype out_dtype, const void* q, void* k_cache, void* v_cache, const void* new_k, const void* new_v,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
    size_t workspace_bytes, hipStream_t stream);
pa_status pa_paged_attention_decode_with_cache_write_reduce(
    void* out, pa_dtype out_dtype, const void* q, void* k_cache, void* v_cache, const void* new_k, const void* new_v,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_shared_prefix -- decode for batches in which groups
 * of sequences share a prefix through aliased blocks, as the samples of one
 * prompt do in parallel sampling (aidocs.cortexgrid.cn page, intro bullets
 * and FAQ answer on parallel sampling; devpress page, "实际收益远超预期").
 * Computes exactly what pa_paged_attention_decode computes, but reads each
 * shared K/V tile once per group instead of once per sequence: one wave
 * scores the queries of up to 16 group members against every shared tile
 * on the matrix cores, each member's private tail runs as ordinary split-K
 * partitions, and the reduction merges both.
 *   group_starts  int32 [num_groups+1], device: rows group_starts[g] ..
 *                 group_starts[g+1]-1 form group g; group_starts[0] == 0,
 *                 non-decreasing, group_starts[num_groups] == num_seqs
 *   prefix_lens   int32 [num_groups], device: tokens every member of group
 *                 g holds in the same physical blocks (identical first
 *                 prefix_lens[g]/block_size table entries); a multiple of
 *                 block_size, <= every member's context length; 0 = nothing
 *                 shared (a group of one sequence)
 *   max_group_size >= every group's size; max_prefix_len >= every prefix
 *   workspace     required: >= pa_decode_shared_workspace_bytes(...) bytes,
 *                 16-byte aligned (fp32 partials of the shared and private
 *                 partitions)
 * Other arguments and layouts as for pa_paged_attention_decode. f32 caches
 * run the ordinary decode (same result). A prefix longer than some member's
 * context breaks the precondition; the device then clamps the group's
 * prefix to its shortest member's context for every member alike, so reads
 * stay inside the members' blocks and each output row has one writer (the
 * result is then that of the shorter prefix, still the members' attention
 * as long as the clamped prefix's blocks are shared).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t max_context_len);
pa_status pa_paged_attention_decode_shared_prefix(
    void* out, pa_dtype out_dtype, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_starts,
    const int32_t* prefix_lens, int32_t num_groups, int32_t max_group_size, int32_t max_prefix_len,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_prefill -- causal attention of multi-token query chunks
 * over the paged cache. The pages let one sequence run in segments across
 * several batches under a per-step token budget (devpress page, continuous
 * batching workflow, step 4, and the max_num_batched_tokens setting), so a
 * prompt is processed as chunks of consecutive tokens, each attending
 * causally to everything cached before it; attention follows the page table
 * as in decode (devpress page, "分页式KV缓存"; betteryeah page, section 2.4).
 * Neither the chunk layout nor the causal alignment is written on the pages;
 * the reading used is the standard one below. Sequence s owns query rows query_start_loc[s] ..
 * query_start_loc[s+1]-1 (L_s >= 0 of them); its context context_lens[s]
 * INCLUDES the chunk, whose K/V are already cached, so the chunk is the last
 * L_s tokens: row query_start_loc[s] + j sits at position ctx - L_s + j and
 * attends to tokens 0 .. ctx - L_s + j.
 *   q, out           [total_q][num_heads][head_dim]
 *   query_start_loc  int32 [num_seqs+1], query_start_loc[0] == 0,
 *                    query_start_loc[num_seqs] == total_q
 *   max_q_len        >= every L_s (sizes the grid)
 * All dtypes run on matrix cores with fp32 accumulation: f16/bf16 round P
 * to the input dtype before the P.V product; f32 keeps every operand in
 * fp32.
 * Preconditions: non-decreasing query_start_loc, L_s <= context_lens[s] <=
 * max_context_len <= max_blocks_per_seq * block_size, valid table entries.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
pa_status pa_paged_attention_prefill(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, const int32_t* query_start_loc,
                                     int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t num_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                     float scale, pa_dtype dtype, hipStream_t stream);

/*
 * attention_step -- one scheduler iteration as a single call: the pages'
 * continuous batching re-forms the batch every iteration, so one step mixes
 * prompts being prefilled and sequences being decoded under a per-step
 * token budget (devpress page, sections on continuous batching and
 * max_num_batched_tokens; aidocs page, static vs continuous batching
 * table). The call writes the step's new tokens (pa_reshape_and_cache),
 * then runs the causal prefill of the chunks and the split-K decode of the
 * decoding sequences, all against the same cache.
 *   num_new_tokens == 0, num_prefill_seqs == 0 or num_decode_seqs == 0
 *   skips that part. Field meanings and layouts are those of the three
 *   single calls; the caches, heads, head_dim, block size, dtype and scale
 *   are shared. workspace is the decode's split-K workspace.
 *   side_stream  NULL: everything is queued on stream in order. Otherwise
 *                (a different stream on the same device, with fork_event
 *                and join_event created by the caller) the prefill runs on
 *                side_stream concurrently with the decode on stream: the
 *                call records fork_event on stream after the cache write,
 *                makes side_stream wait for it, and makes stream wait for
 *                join_event recorded on side_stream after the prefill, so
 *                on return all work is ordered before anything queued
 *                later on stream. Safe inside stream capture (fork/join).
 * Every part is validated before anything is queued; an error leaves the
 * streams untouched. Errors: those of the three calls, and INVALID_ARG for
 * a side stream equal to stream or missing events.
 */
typedef struct {
  void* k_cache;
  void* v_cache;
  int32_t num_blocks, num_heads, head_dim, block_size;
  pa_dtype dtype;
  float scale;
  const void* new_k; /* [num_new_tokens][H][D] */
  const void* new_v;
  const int32_t* slot_mapping;
  int32_t num_new_tokens;
  void* prefill_out; /* [prefill_total_q][H][D] */
  pa_dtype prefill_out_dtype;
  const void* prefill_q;
  const int32_t* prefill_block_tables;
  const int32_t* prefill_context_lens;
  const int32_t* prefill_query_start_loc;
  int32_t num_prefill_seqs, prefill_total_q, prefill_max_q_len, prefill_max_blocks_per_seq,
      prefill_max_context_len;
  void* decode_out; /* [num_decode_seqs][H][D] */
  pa_dtype decode_out_dtype;
  const void* decode_q;
  const int32_t* decode_block_tables;
  const int32_t* decode_context_lens;
  int32_t num_decode_seqs, decode_max_blocks_per_seq, decode_max_context_len;
  void* workspace;
  size_t workspace_bytes;
} pa_step_args;

pa_status pa_attention_step(const pa_step_args* step, hipStream_t stream, hipStream_t side_stream,
                            hipEvent_t fork_event, hipEvent_t join_event);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
