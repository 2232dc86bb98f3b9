"""Generator and allocator checks: the memory accounting the pages print, the
block-table invariants of paging, and determinism of the seeded inputs."""
import json
import math
import os

import numpy as np
import pytest

from workloads import (POISON_BITS, AllocatorError, BlockAllocator, bits, config1, config4, config5,
                       contiguous_utilisation, decode_workload, lognormal_lengths, paged_slots, paged_utilisation)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_printed_memory_accounting():
    g = json.load(open(os.path.join(GOLDEN, "memory_accounting.json")))
    c = g["contiguous_reservation"]
    wasted = c["reserve"] - c["length"]
    assert wasted == c["wasted_exact"] and wasted > c["wasted_more_than"]
    t = g["three_sequences"]
    assert contiguous_utilisation(t["lengths"]) == pytest.approx(t["contiguous_utilisation"])
    p = g["paged_utilisation"]
    assert paged_slots(p["lengths"], p["block_size"]) == p["paged_slots"]
    u = paged_utilisation(p["lengths"], p["block_size"])
    assert u >= p["utilisation_at_least"] and 1 - u < p["waste_below"]


def _check_tables(wl, batch):
    bs = wl.block_size
    for s, c in enumerate(batch.context_lens):
        n = math.ceil(c / bs)
        row = batch.block_tables[s]
        assert np.all((row[:n] >= 0) & (row[:n] < wl.num_blocks))
        assert np.all(row[n:] == -1)


def test_tiny_config_shape():
    wl = config1()
    d = wl.decode
    assert wl.num_blocks == 64 and wl.k_cache.shape == (64, 2, 16, 64) and wl.dtype == "f32"
    assert d.context_lens.tolist() == [1, 17, 33, 100]
    _check_tables(wl, d)
    used = {int(b) for b in d.block_tables.ravel() if b >= 0}
    assert len(used) == 13  # 1 + 2 + 3 + 7 blocks, no sharing
    # unused blocks are all poison; the new tokens' slots are poison too before the write
    unused = sorted(set(range(64)) - used)
    assert np.all(bits(wl.k_cache[unused], "f32") == POISON_BITS["f32"])
    sm = wl.new.slot_mapping
    assert np.all(bits(wl.k_cache[sm // 16, :, sm % 16], "f32") == POISON_BITS["f32"])


def test_only_the_last_block_of_a_sequence_is_partial_and_waste_is_small():
    wl = decode_workload("acct", 31, "f16", 1, 64, 16, np.arange(128, 2049, 61), maxb=128)
    ctx = wl.decode.context_lens
    blocks = np.ceil(ctx / 16).astype(int)
    assert wl.num_blocks == blocks.sum()  # pool sized to fit exactly
    waste = (blocks * 16 - ctx) / (blocks * 16)
    assert np.all(blocks * 16 - ctx < 16)
    assert waste.max() < 0.04 * (2048 / 128)  # at most bs-1 slots of the last block
    assert 1 - ctx.sum() / (blocks.sum() * 16) < 0.04
    _check_tables(wl, wl.decode)
    # tables are slices of one permutation: every block used exactly once
    flat = wl.decode.block_tables[wl.decode.block_tables >= 0]
    assert np.array_equal(np.sort(flat), np.arange(wl.num_blocks))


def test_prefix_sharing_refcounts_and_conservation():
    wl = config4(prompts=4, samples=8, prompt_len=64, max_tail=40, H=2, D=64)
    d = wl.decode
    _check_tables(wl, d)
    refs = wl.notes["refcount"]
    # sum of refcounts equals the number of table entries of live sequences
    assert refs.sum() == (d.block_tables >= 0).sum()
    for p in range(4):
        rows = d.block_tables[p * 8:(p + 1) * 8, :4]  # 64-token prompt = 4 shared blocks
        assert np.all(rows == rows[0])
        assert np.all(refs[rows[0]] == 8)
    assert wl.notes["cow_copies"] == 0


def test_copy_on_write_of_a_partial_shared_block():
    wl = config4(prompts=3, samples=4, prompt_len=64, max_tail=20, H=2, D=64, cow=True)
    d = wl.decode
    _check_tables(wl, d)
    assert wl.notes["cow_copies"] > 0
    plens = wl.notes["prompt_lens"]
    for p in range(3):
        last = (plens[p] - 1) // 16
        rows = d.block_tables[p * 4:(p + 1) * 4]
        tails = wl.notes["tails"][p]
        extended = [i for i in range(4) if tails[i] > 0]
        # the full prompt blocks stay shared
        assert np.all(rows[:, :last] == rows[0, :last])
        # no two writers share the partially filled block after copy-on-write
        owners = [rows[i, last] for i in extended]
        assert len(set(owners)) == len(owners)
        # the copied blocks hold the prompt's tokens bit for bit
        r0 = plens[p] - 16 * last
        src = rows[[i for i in range(4) if tails[i] == 0][0], last] if len(extended) < 4 else None
        if src is not None:
            for b in owners:
                assert np.array_equal(bits(wl.k_cache[b, :, :r0], "f16"), bits(wl.k_cache[src, :, :r0], "f16"))


def test_mixed_step_budget_and_slots():
    wl = config5(H=2, D=64)
    sm = wl.new.slot_mapping
    assert sm.shape == (2048,) and len(set(sm.tolist())) == 2048 and sm.min() >= 0
    L = np.diff(wl.prefill.query_start_loc)
    assert L.sum() + 96 + wl.notes["n_fill"] == 2048
    assert np.all((L >= 256) & (L <= 512))
    prior = wl.prefill.context_lens - L
    assert np.all((prior >= 0) & (prior <= 1024))
    assert np.all((wl.decode.context_lens >= 256) & (wl.decode.context_lens <= 4096))
    _check_tables(wl, wl.prefill)
    _check_tables(wl, wl.decode)
    # filler slots are referenced by no sequence
    ref = set()
    for batch in (wl.prefill, wl.decode):
        for s, c in enumerate(batch.context_lens):
            t = np.arange(c)
            ref.update((batch.block_tables[s, t // 16] * 16 + t % 16).tolist())
    assert not set(sm[-wl.notes["n_fill"]:].tolist()) & ref


def test_lognormal_lengths_mean_and_clip():
    x = lognormal_lengths(np.random.default_rng(0), 200000)
    assert x.min() >= 1 and x.max() <= 4096
    assert 570 < x.mean() < 600


def test_generation_is_deterministic():
    a, b = config1(), config1()
    assert np.array_equal(bits(a.k_cache, "f32"), bits(b.k_cache, "f32"))
    assert np.array_equal(a.decode.block_tables, b.decode.block_tables)
    assert np.array_equal(bits(a.new.v, "f32"), bits(b.new.v, "f32"))


def test_allocator_alloc_fork_free_and_errors():
    al = BlockAllocator(4, 16)
    s = al.new_sequence()
    al.append(s, 20)
    assert len(s.table) == 2 and al.num_free == 2
    f = al.fork(s)
    assert all(al.refcount[b] == 2 for b in s.table)
    slots = al.append(f, 1)  # writes into the shared partial block -> copy-on-write
    assert al.copies and f.table[-1] != s.table[-1] and slots[0] // 16 == f.table[-1]
    al.free(s)
    al.free(f)
    assert al.num_free == 4 and al.refcount.sum() == 0
    with pytest.raises(AllocatorError):
        al.release(0)
    s = al.new_sequence()
    with pytest.raises(AllocatorError):
        al.append(s, 5 * 16)
