"""Seeded synthetic inputs for paged-KV attention (shared by the oracle side
and the HIP side; holds no attention arithmetic)."""
from .allocator import AllocatorError, BlockAllocator, Sequence
from .configs import (BASE_SEED, CONFIG_NAMES, DTYPES, ELT_BYTES, POISON_BITS, STORAGE, DecodeBatch,
                      NewTokens, PrefillBatch, Workload, bits, config1, config2, config3, config4, config5,
                      contiguous_utilisation, decode_workload, f32_to_storage, lognormal_lengths, make_config,
                      normal, paged_slots, paged_utilisation, poison_array, prefill_workload, storage_to_f32)
