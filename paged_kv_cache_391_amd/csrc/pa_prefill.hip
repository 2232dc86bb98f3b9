// Causal prefill of query chunks (placeholder: vector path per query row).
#include "pa_internal.h"

namespace pa {

int prefill_mfma_q_tile() { return 128; }

hipError_t launch_prefill_mfma(const PrefillArgs& p, Dt dt, int D, int BS, hipStream_t stream) {
  DecodeArgs a{};
  a.out = p.out;
  a.q = p.q;
  a.k_cache = p.k_cache;
  a.v_cache = p.v_cache;
  a.block_tables = p.block_tables;
  a.context_lens = p.context_lens;
  a.query_start_loc = p.query_start_loc;
  a.num_seqs = p.num_seqs;
  a.num_rows = p.total_q;
  a.H = p.H;
  a.max_blocks = p.max_blocks;
  a.max_parts = 1;
  a.part_tiles = (p.max_context_len + 15) / 16;
  a.scale_log2 = p.scale_log2;
  a.out_f32 = p.out_f32;
  return launch_decode_partitions(a, dt, D, BS, true, stream);
}

}  // namespace pa
