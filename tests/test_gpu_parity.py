"""GPU parity of the HIP library against the fp64 oracle, through the C ABI.

Bars: bit-exact for the cache write and the block-table gather; for
attention, max-abs error of the fp32 output <= 2e-3 (f16/bf16 inputs) or
1e-5 (f32 inputs), and a narrowed output equal bit for bit to the
round-to-nearest-even of the same kernel's fp32 output."""
import functools
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_391_amd as pa
from tests._gpu import ATOL, TORCH_DT, OnDevice, bits, dev, host, rne
from workloads import config4, decode_workload, make_config, prefill_workload

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def _config(cid, dtype=None):
    wl = make_config(cid) if dtype is None else make_config(cid, dtype=dtype)
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping,
                                      wl.block_size, wl.dtype)
    return wl, kc, vc


@functools.lru_cache(maxsize=None)
def _oracle_decode(cid, dtype=None):
    wl, kc, vc = _config(cid, dtype)
    d = wl.decode
    return oracle.decode(d.q, kc, vc, d.block_tables, d.context_lens, wl.scale, wl.dtype)


@functools.lru_cache(maxsize=None)
def _oracle_prefill(cid, dtype=None):
    wl, kc, vc = _config(cid, dtype)
    p = wl.prefill
    return oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, wl.dtype)


def _on_device_written(wl):
    od = OnDevice(wl)
    od.write_new_tokens()
    return od


def _check_attention(got_f32: torch.Tensor, ref: np.ndarray, dtype: str):
    got = host(got_f32).astype(np.float64)
    assert got.shape == ref.shape
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max() if got.size else 0.0
    assert err <= ATOL[dtype], f"max abs error {err:.3e} > {ATOL[dtype]}"
    return err


# ------------------------------------------------------------ cache writes

@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_reshape_and_cache_bit_exact(cid):
    wl, kc_ref, vc_ref = _config(cid)
    od = _on_device_written(wl)
    assert np.array_equal(bits(host(od.k_cache)), bits(kc_ref))
    assert np.array_equal(bits(host(od.v_cache)), bits(vc_ref))


@pytest.mark.parametrize("dtype,H,D,bs", [("f16", 4, 128, 16), ("bf16", 2, 64, 32), ("f32", 3, 128, 8),
                                          ("f16", 5, 64, 64)])
def test_reshape_and_cache_padding_and_slots_past_the_pool(dtype, H, D, bs):
    """Rows with a negative slot (padding) and rows whose slot lies past the
    pool are skipped; every other row lands bit-exactly in its slot, and every
    slot no row names keeps its poison bits."""
    from workloads import normal, poison_array
    rng = np.random.default_rng(17 + bs)
    T = 200
    nb = -(-T // bs) + 8  # room for every row, and slots no row names
    slots = rng.permutation(nb * bs)[:T].astype(np.int32)
    slots[rng.random(T) < 0.2] = -1
    past = rng.choice(T, 5, replace=False)
    slots[past] = nb * bs + rng.integers(0, 1000, 5)
    k, v = normal(rng, (T, H, D), dtype), normal(rng, (T, H, D), dtype)
    kc, vc = poison_array((nb, H, bs, D), dtype), poison_array((nb, H, bs, D), dtype)
    dk, dv = dev(kc, dtype), dev(vc, dtype)
    pa.reshape_and_cache(dev(k, dtype), dev(v, dtype), dk, dv, dev(slots))
    valid = slots.copy()
    valid[past] = -1
    kr, vr = oracle.reshape_and_cache(k, v, kc, vc, valid, bs, dtype)
    assert np.array_equal(bits(host(dk)), bits(kr))
    assert np.array_equal(bits(host(dv)), bits(vr))


@pytest.mark.parametrize("dtype,H,D,bs", [("f16", 40, 128, 16), ("bf16", 32, 128, 32), ("f32", 2, 64, 16),
                                          ("f16", 8, 128, 8), ("bf16", 4, 64, 64)])
def test_copy_blocks_bit_exact(dtype, H, D, bs):
    """Copy-on-write block copies equal the oracle's bit for bit; blocks that
    are not destinations keep their bits; a pair naming a block outside the
    pool is skipped by the kernel's own bounds check."""
    rng = np.random.default_rng(21)
    nb = 64
    from workloads import normal
    kc = normal(rng, (nb, H, bs, D), dtype)
    vc = normal(rng, (nb, H, bs, D), dtype)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:20], perm[20:40]], 1).astype(np.int32)
    kref, vref = oracle.copy_blocks(kc, vc, pairs, dtype)
    dk, dv = dev(kc, dtype), dev(vc, dtype)
    pa.copy_blocks(dk, dv, dev(pairs))
    assert np.array_equal(bits(host(dk)), bits(kref)) and np.array_equal(bits(host(dv)), bits(vref))
    outside = np.array([[perm[40], nb], [nb + 5, perm[41]]], dtype=np.int32)
    pa.copy_blocks(dk, dv, dev(outside))
    assert np.array_equal(bits(host(dk)), bits(kref)) and np.array_equal(bits(host(dv)), bits(vref))
    pa.copy_blocks(dk, dv, dev(np.zeros((0, 2), dtype=np.int32)))
    torch.cuda.synchronize()


def test_copy_on_write_with_the_native_allocator_then_decode():
    """Parallel sampling end to end: the library's allocator forks a 37-token
    prompt into 4 samples; each sample's next tokens trigger a copy of the
    shared partly filled block; the copies run on the GPU, the new tokens are
    written, and decode over all samples matches the oracle fed the same
    tables, copies and writes."""
    H, D, bs, dtype, nb = 8, 128, 16, "f16", 48
    rng = np.random.default_rng(22)
    from workloads import normal
    alloc = pa.BlockAllocator(nb, bs)
    prompt = alloc.new_sequence()
    prompt_slots = alloc.append(prompt, 37)
    assert alloc.take_copies().shape[0] == 0  # close the batch: the prompt's writes go first
    samples = [prompt] + [alloc.fork(prompt) for _ in range(3)]
    kc = normal(rng, (nb, H, bs, D), dtype)
    vc = normal(rng, (nb, H, bs, D), dtype)
    pk, pv = normal(rng, (37, H, D), dtype), normal(rng, (37, H, D), dtype)
    kc, vc = oracle.reshape_and_cache(pk, pv, kc, vc, prompt_slots, bs, dtype)
    new_slots, copies = [], []
    for i, sq in enumerate(samples[::-1]):           # the prompt itself writes last, in place
        new_slots.append(alloc.append(sq, 2 + 7 * i))
        copies.append(alloc.take_copies())
    copies = np.concatenate(copies)
    assert copies.shape[0] == 3 and len(set(copies[:, 1])) == 3
    slots = np.concatenate(new_slots)
    nk, nv = normal(rng, (slots.size, H, D), dtype), normal(rng, (slots.size, H, D), dtype)
    tables = [alloc.block_table(sq) for sq in samples]
    maxb = max(t.size for t in tables)
    bt = np.full((4, maxb), -1, dtype=np.int32)
    for i, t in enumerate(tables):
        bt[i, :t.size] = t
    ctx = np.array([alloc.length(sq) for sq in samples], dtype=np.int32)
    q = normal(rng, (4, H, D), dtype)
    scale = 1 / math.sqrt(D)
    rk, rv = oracle.copy_blocks(kc, vc, copies, dtype)
    rk, rv = oracle.reshape_and_cache(nk, nv, rk, rv, slots, bs, dtype)
    ref = oracle.decode(q, rk, rv, bt, ctx, scale, dtype)
    dk, dv = dev(kc, dtype), dev(vc, dtype)
    pa.copy_blocks(dk, dv, dev(copies))
    pa.reshape_and_cache(dev(nk, dtype), dev(nv, dtype), dk, dv, dev(slots))
    assert np.array_equal(bits(host(dk)), bits(rk)) and np.array_equal(bits(host(dv)), bits(rv))
    out = torch.empty((4, H, D), dtype=torch.float32, device="cuda")
    ws = pa.make_decode_workspace(4, H, D, int(ctx.max()))
    pa.paged_attention_decode(out, dev(q, dtype), dk, dv, dev(bt), dev(ctx), scale, int(ctx.max()), ws)
    _check_attention(out, ref, dtype)


@pytest.mark.parametrize("cid", [1, 3, 4])
def test_gather_kv_bit_exact(cid):
    wl, kc_ref, vc_ref = _config(cid)
    od = _on_device_written(wl)
    d = wl.decode
    cu = np.concatenate([[0], np.cumsum(d.context_lens)]).astype(np.int32)
    total = int(cu[-1])
    k_out = torch.empty((total, wl.num_heads, wl.head_dim), dtype=TORCH_DT[wl.dtype], device="cuda")
    v_out = torch.empty_like(k_out)
    pa.gather_kv(k_out, v_out, od.k_cache, od.v_cache, od.block_tables, od.context_lens, dev(cu),
                 d.max_context_len)
    k_ref, v_ref = oracle.gather_kv(kc_ref, vc_ref, d.block_tables, d.context_lens, wl.dtype)
    assert np.array_equal(bits(host(k_out)), bits(k_ref))
    assert np.array_equal(bits(host(v_out)), bits(v_ref))


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_decode_parity_full_config(cid):
    wl, _, _ = _config(cid)
    ref = _oracle_decode(cid)
    od = _on_device_written(wl)
    out32 = od.decode(torch.float32)
    err = _check_attention(out32, ref, wl.dtype)
    print(f"config {cid} decode max abs err {err:.3e}")
    if wl.dtype != "f32":
        outn = od.decode(TORCH_DT[wl.dtype])
        assert np.array_equal(bits(host(outn)), bits(rne(host(out32), wl.dtype)))


def _ragged_cases():
    cases = []
    for dtype in ("f32", "f16", "bf16"):
        for D in (64, 128):
            for bs in (16, 32):
                cases.append((dtype, D, bs))
    cases += [("f16", 128, 8), ("bf16", 128, 64), ("f32", 64, 8), ("f16", 64, 64)]
    return cases


@pytest.mark.parametrize("dtype,D,bs", _ragged_cases())
def test_decode_ragged_lengths(dtype, D, bs):
    P = pa.decode_partition_tokens()
    ctx = [1, 2, 7, 8, 9, 15, 16, 17, 31, 33, 63, 64, 65, 100, P - 1, P, P + 1, 2 * P + 7, 3 * P]
    wl = decode_workload(f"ragged_{dtype}_{D}_{bs}", 500 + D + bs, dtype, 3, D, bs, ctx,
                         maxb=math.ceil(max(ctx) / bs) + 2, pool_factor=1.3)
    od = _on_device_written(wl)
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, bs, dtype)
    d = wl.decode
    ref = oracle.decode(d.q, kc, vc, d.block_tables, d.context_lens, wl.scale, dtype)
    _check_attention(od.decode(torch.float32, split=True), ref, dtype)
    _check_attention(od.decode(torch.float32, split=False), ref, dtype)


def test_decode_rows_of_many_partitions():
    """The reduction reads the first 8 partitions' accumulators at once and
    holds one partition's (m, l) per lane: rows of 8 and 9 partitions (the
    first boundary) and of 64, 65 and 66 (past one value per lane)."""
    P = pa.decode_partition_tokens()
    ctx = [8 * P, 8 * P + 1, 9 * P, 64 * P, 64 * P + 100, 65 * P + 7]
    wl = decode_workload("many_parts", 611, "f16", 2, 128, 16, ctx, maxb=math.ceil(max(ctx) / 16), pool_factor=1.05)
    od = _on_device_written(wl)
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, 16, "f16")
    d = wl.decode
    ref = oracle.decode(d.q, kc, vc, d.block_tables, d.context_lens, wl.scale, "f16")
    _check_attention(od.decode(torch.float32, split=True), ref, "f16")
    _check_attention(od.decode(torch.float32, split=False), ref, "f16")


def _fused_rows(wl, pad_rows=(), past_pool_rows=()):
    """Per-row new tokens (fresh values) and slots for the fused decode: a
    row with a context gets its last position's slot, a row in pad_rows and
    an empty row get slot -1, a row in past_pool_rows a slot just past the
    pool (both skipped: nothing written, the row reads the cache as it
    is)."""
    from workloads import normal
    d = wl.decode
    S, H, D = d.q.shape
    rng = np.random.default_rng(5)
    nk = normal(rng, (S, H, D), wl.dtype)
    nv = normal(rng, (S, H, D), wl.dtype)
    slots = np.full(S, -1, dtype=np.int32)
    t = 0
    for r in range(S):
        if d.context_lens[r] > 0:
            if r not in pad_rows:
                slots[r] = wl.new.slot_mapping[t]
            t += 1
        if r in past_pool_rows:
            slots[r] = wl.num_blocks * wl.block_size + r
    return nk, nv, slots


def _check_fused(wl, split, pad_rows=(), past_pool_rows=()):
    """pa_paged_attention_decode_with_cache_write against reshape_and_cache
    followed by paged_attention_decode (outputs and caches bit for bit) and
    against the oracle. Both caches first hold the workload's own new tokens
    (so padding rows read finite values); the fresh tokens then replace them."""
    d = wl.decode
    nk, nv, slots = _fused_rows(wl, pad_rows, past_pool_rows)
    dt = wl.dtype
    ref = _on_device_written(wl)
    nk_d, nv_d, sl_d = dev(nk, dt), dev(nv, dt), dev(slots)
    pa.reshape_and_cache(nk_d, nv_d, ref.k_cache, ref.v_cache, sl_d)
    out_ref = ref.decode(torch.float32, split=split)
    od = _on_device_written(wl)
    out = torch.empty_like(out_ref)
    ws = pa.make_decode_workspace(d.num_seqs, wl.num_heads, wl.head_dim, d.max_context_len) if split else None
    pa.paged_attention_decode_with_cache_write(out, od.q, od.k_cache, od.v_cache, nk_d, nv_d, sl_d, od.block_tables,
                                               od.context_lens, wl.scale, d.max_context_len, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    assert np.array_equal(bits(host(od.k_cache)), bits(host(ref.k_cache)))
    assert np.array_equal(bits(host(od.v_cache)), bits(host(ref.v_cache)))
    if ws is not None:  # the two stages, as a caller that times them runs them
        st = _on_device_written(wl)
        out_st = torch.empty_like(out_ref)
        pa.paged_attention_decode_with_cache_write_partitions(out_st, st.q, st.k_cache, st.v_cache, nk_d, nv_d, sl_d,
                                                              st.block_tables, st.context_lens, wl.scale,
                                                              d.max_context_len, ws)
        pa.paged_attention_decode_with_cache_write_reduce(out_st, st.q, st.k_cache, st.v_cache, nk_d, nv_d, sl_d,
                                                          st.block_tables, st.context_lens, wl.scale,
                                                          d.max_context_len, ws)
        torch.cuda.synchronize()
        assert torch.equal(out_st, out)
        assert np.array_equal(bits(host(st.k_cache)), bits(host(ref.k_cache)))
        assert np.array_equal(bits(host(st.v_cache)), bits(host(ref.v_cache)))
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping,
                                      wl.block_size, dt)
    # the oracle takes in-range slots only: a slot past the pool is the same skip as -1
    kc, vc = oracle.reshape_and_cache(nk, nv, kc, vc, np.where(slots < wl.num_blocks * wl.block_size, slots, -1),
                                      wl.block_size, dt)
    _check_attention(out, oracle.decode(d.q, kc, vc, d.block_tables, d.context_lens, wl.scale, dt), dt)


@pytest.mark.parametrize("cid", [2, 3])
def test_decode_with_cache_write_full_config(cid):
    """The fused cache write on the LLaMA-7B and 256-sequence workloads (every
    row's last position is its new token)."""
    wl, _, _ = _config(cid)
    _check_fused(wl, split=True)


@pytest.mark.parametrize("dtype,D,bs,split", [("f16", 128, 16, True), ("bf16", 128, 8, True), ("f32", 128, 32, True),
                                              ("f16", 64, 64, False), ("f32", 64, 8, False), ("bf16", 64, 16, True)])
def test_decode_with_cache_write_ragged(dtype, D, bs, split):
    """Contexts around tile, block and partition edges (the new token in every
    row of its tile), empty rows and padding rows (slot -1: nothing written,
    the row reads the cache as it is)."""
    P = pa.decode_partition_tokens()
    ctx = [0, 1, 2, 15, 16, 17, 31, 33, 100, P - 1, P, P + 1, 2 * P + 9, 3 * P, 0, 47]
    wl = decode_workload(f"fused_{dtype}_{D}_{bs}", 640 + bs, dtype, 3, D, bs, ctx,
                         maxb=math.ceil(max(ctx) / bs), pool_factor=1.3)
    _check_fused(wl, split, pad_rows=(7,), past_pool_rows=(12,))


def test_decode_empty_context_gives_zeros():
    wl = decode_workload("empty", 601, "f16", 2, 128, 16, [0, 5, 0, 40], maxb=4, pool_blocks=8)
    od = _on_device_written(wl)
    out = host(od.decode(torch.float32)).astype(np.float64)
    assert np.all(out[[0, 2]] == 0.0)
    assert np.isfinite(out).all()


def test_decode_is_deterministic_and_stage_split_matches():
    wl, _, _ = _config(3)
    od = _on_device_written(wl)
    a = host(od.decode(torch.float32))
    b = host(od.decode(torch.float32))
    assert np.array_equal(bits(a), bits(b))
    d = wl.decode
    out = torch.empty_like(od.q, dtype=torch.float32)
    ws = pa.make_decode_workspace(d.num_seqs, wl.num_heads, wl.head_dim, d.max_context_len)
    pa.paged_attention_decode_partitions(out, od.q, od.k_cache, od.v_cache, od.block_tables, od.context_lens,
                                         wl.scale, d.max_context_len, ws)
    pa.paged_attention_decode_reduce(out, od.context_lens, wl.head_dim, d.max_context_len, od.q.dtype, ws)
    assert np.array_equal(bits(host(out)), bits(a))


def test_decode_single_partition_is_bit_identical_with_or_without_workspace():
    P = pa.decode_partition_tokens()
    wl = decode_workload("onepart", 602, "bf16", 4, 128, 32, [7, P // 2, P - 3, P], maxb=P // 32, pool_factor=1.2)
    od = _on_device_written(wl)
    assert np.array_equal(bits(host(od.decode(split=True))), bits(host(od.decode(split=False))))


def test_decode_bit_identical_under_block_permutation():
    wl, _, _ = _config(2)
    od = _on_device_written(wl)
    base = host(od.decode(torch.float32))
    g = torch.Generator(device="cpu").manual_seed(5)
    perm = torch.randperm(wl.num_blocks, generator=g).to("cuda")  # block b moves to perm[b]
    kc = torch.empty_like(od.k_cache)
    vc = torch.empty_like(od.v_cache)
    kc[perm] = od.k_cache
    vc[perm] = od.v_cache
    bt = od.block_tables.clone()
    valid = bt >= 0
    bt[valid] = perm[bt[valid].long()].int()
    out = host(od.decode(torch.float32, block_tables=bt, k_cache=kc, v_cache=vc))
    assert np.array_equal(bits(out), bits(base))


def test_decode_bit_identical_with_aliased_or_private_prefix_blocks():
    wl = config4(prompts=4, samples=8, prompt_len=256, max_tail=64, cow=True)
    od = _on_device_written(wl)
    base = host(od.decode(torch.float32))
    bt = wl.decode.block_tables.copy()
    refs = wl.notes["refcount"]
    extra_src = []
    nb = wl.num_blocks
    for s in range(bt.shape[0]):
        for i in range(bt.shape[1]):
            if bt[s, i] >= 0 and refs[bt[s, i]] > 1:
                extra_src.append(int(bt[s, i]))
                bt[s, i] = nb
                nb += 1
    src = torch.tensor(extra_src, device="cuda", dtype=torch.long)
    kc = torch.cat([od.k_cache, od.k_cache[src]])
    vc = torch.cat([od.v_cache, od.v_cache[src]])
    out = host(od.decode(torch.float32, block_tables=dev(bt), k_cache=kc, v_cache=vc))
    assert np.array_equal(bits(out), bits(base))
    # and against the oracle on the aliased layout
    kc_ref, vc_ref = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, 16,
                                              "f16")
    d = wl.decode
    ref = oracle.decode(d.q, kc_ref, vc_ref, d.block_tables, d.context_lens, wl.scale, "f16")
    assert np.abs(base.astype(np.float64) - ref).max() <= ATOL["f16"]


def _to_big_pool(kc, vc, nb_big):
    """Copy a compact pool's blocks into a pool of nb_big blocks: even block
    ids stay, odd ones move to the top of the pool (byte offsets past
    2^32). Returns the big caches and the old id -> new id map."""
    nb = kc.shape[0]
    ids = torch.arange(nb, device="cuda")
    new_id = torch.where(ids % 2 == 0, ids, nb_big - 1 - ids)
    kb = torch.empty((nb_big,) + tuple(kc.shape[1:]), dtype=kc.dtype, device="cuda")
    vb = torch.empty_like(kb)
    kb[new_id] = kc
    vb[new_id] = vc
    return kb, vb, new_id


def _same_bits(a, b):
    """Bitwise equality (the pools hold NaN poison in never-written slots)."""
    iv = {2: torch.int16, 4: torch.int32}[a.element_size()]
    return a.shape == b.shape and torch.equal(a.contiguous().view(iv), b.contiguous().view(iv))


def _remap_tables(bt, new_id):
    out = bt.clone()
    valid = bt >= 0
    out[valid] = new_id[bt[valid].long()].int()
    return out


def test_pool_beyond_4gib_is_bit_identical():
    """Caches of more than 4 GiB each, with half of the workload's blocks at
    ids whose byte offsets pass 2^32: the cache write, block copies, the
    gather, the decode, the shared-prefix decode and the prefill give bit for
    bit what they give on the compact pool (every offset is 64-bit)."""
    wl = config4(prompts=4, samples=4, prompt_len=256, max_tail=64, cow=True)
    H, D, bs = wl.num_heads, wl.head_dim, wl.block_size
    block_bytes = H * bs * D * 2
    nb_big = (9 << 29) // block_bytes + 2 * wl.num_blocks  # > 4.5 GiB per cache
    assert (nb_big - 2 * wl.num_blocks) * block_bytes > (1 << 32)
    od = OnDevice(wl)
    kb, vb, new_id = _to_big_pool(od.k_cache, od.v_cache, nb_big)
    # cache write through remapped slots
    slots = od.slot_mapping.long()
    big_slots = torch.where(slots >= 0, new_id[(slots // bs).clamp(min=0)] * bs + slots % bs, slots).int()
    od.write_new_tokens()
    pa.reshape_and_cache(od.new_k, od.new_v, kb, vb, big_slots)
    assert _same_bits(kb[new_id], od.k_cache) and _same_bits(vb[new_id], od.v_cache)
    d = wl.decode
    bt_big = _remap_tables(od.block_tables, new_id)
    # decode, plain and shared-prefix
    base = od.decode(torch.float32)
    got = od.decode(torch.float32, block_tables=bt_big, k_cache=kb, v_cache=vb)
    assert _same_bits(base, got)
    gs, pl, samples = _groups_for_prefix_workload(wl)
    ws = pa.make_decode_shared_workspace(d.num_seqs, H, D, d.max_context_len)
    sh = [torch.empty(od.q.shape, dtype=torch.float32, device="cuda") for _ in range(2)]
    for o, (bt, k, v) in zip(sh, [(od.block_tables, od.k_cache, od.v_cache), (bt_big, kb, vb)]):
        pa.paged_attention_decode_shared_prefix(o, od.q, k, v, bt, od.context_lens, dev(gs), dev(pl), wl.scale,
                                                d.max_context_len, samples, int(pl.max()), ws)
    assert _same_bits(sh[0], sh[1])
    # gather
    cu = dev(np.concatenate([[0], np.cumsum(d.context_lens)]).astype(np.int32))
    total = int(d.context_lens.sum())
    outs = []
    for bt, k, v in [(od.block_tables, od.k_cache, od.v_cache), (bt_big, kb, vb)]:
        ko = torch.empty((total, H, D), dtype=k.dtype, device="cuda")
        vo = torch.empty_like(ko)
        pa.gather_kv(ko, vo, k, v, bt, od.context_lens, cu, d.max_context_len)
        outs.append((ko, vo))
    assert _same_bits(outs[0][0], outs[1][0]) and _same_bits(outs[0][1], outs[1][1])
    # block copies between the two halves of the id range
    pairs = np.array([[1, 2], [4, 3], [5, 7]], dtype=np.int32)
    pa.copy_blocks(od.k_cache, od.v_cache, dev(pairs))
    pa.copy_blocks(kb, vb, new_id[torch.from_numpy(pairs).long().cuda()].int().contiguous())
    assert _same_bits(kb[new_id], od.k_cache) and _same_bits(vb[new_id], od.v_cache)
    del kb, vb
    # prefill of a chunk workload with the same cache shape, in a big pool
    pw = prefill_workload("pf_big", 790, "f16", H, D, bs, [0, 200, 37], [100, 64, 130], maxb=20, pool_factor=1.2)
    op = _on_device_written(pw)
    kp, vp, pid = _to_big_pool(op.k_cache, op.v_cache, nb_big)
    p = pw.prefill
    res = []
    for bt, k, v in [(op.pf_block_tables, op.k_cache, op.v_cache), (_remap_tables(op.pf_block_tables, pid), kp, vp)]:
        o = torch.empty(op.pf_q.shape, dtype=torch.float32, device="cuda")
        pa.paged_attention_prefill(o, op.pf_q, k, v, bt, op.pf_context_lens, op.pf_qsl, pw.scale,
                                   max_q_len=p.max_q_len, max_context_len=p.max_context_len)
        res.append(o)
    assert _same_bits(res[0], res[1])
    del kp, vp
    torch.cuda.empty_cache()


# ------------------------------------------------- shared-prefix decode

def _groups_for_prefix_workload(wl):
    """Group metadata of the prefix-sharing workload: consecutive rows of one
    prompt, sharing the prompt's whole blocks."""
    notes = wl.notes
    samples = len(notes["tails"][0])
    plens = notes["prompt_lens"]
    gs = np.arange(0, samples * len(plens) + 1, samples, dtype=np.int32)
    pl = np.array([(p // wl.block_size) * wl.block_size for p in plens], dtype=np.int32)
    return gs, pl, samples


def _shared_decode(od, wl, gs, pl, max_group, out_dtype=torch.float32):
    d = wl.decode
    out = torch.empty(od.q.shape, dtype=out_dtype, device="cuda")
    ws = pa.make_decode_shared_workspace(d.num_seqs, wl.num_heads, wl.head_dim, d.max_context_len)
    pa.paged_attention_decode_shared_prefix(out, od.q, od.k_cache, od.v_cache, od.block_tables, od.context_lens,
                                            dev(gs), dev(pl), wl.scale, d.max_context_len, max_group,
                                            int(pl.max()), ws, validate=True)
    return out


@pytest.mark.parametrize("cow", [False, True])
def test_shared_prefix_decode_prefix_workload(cow):
    wl = config4(cow=True) if cow else _config(4)[0]
    if cow:
        kc_ref, vc_ref = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping,
                                                  wl.block_size, wl.dtype)
    else:
        _, kc_ref, vc_ref = _config(4)
    od = _on_device_written(wl)
    gs, pl, samples = _groups_for_prefix_workload(wl)
    d = wl.decode
    ref = oracle.decode(d.q, kc_ref, vc_ref, d.block_tables, d.context_lens, wl.scale, wl.dtype)
    out = _shared_decode(od, wl, gs, pl, samples)
    err = _check_attention(out, ref, wl.dtype)
    plain = host(od.decode(torch.float32)).astype(np.float64)
    assert np.abs(host(out).astype(np.float64) - plain).max() <= ATOL[wl.dtype]
    outn = _shared_decode(od, wl, gs, pl, samples, TORCH_DT[wl.dtype])
    assert np.array_equal(bits(host(outn)), bits(rne(host(out), wl.dtype)))
    print(f"shared-prefix decode ({'cow' if cow else 'aligned'}) max abs err {err:.2e}")


def _grouped_batch(dtype, bs, groups, seed):
    """groups: list of (members, prefix_tokens, [tail tokens per member]).
    Blocks come from the library's allocator (fork shares the prefix)."""
    from workloads import normal
    rng = np.random.default_rng(seed)
    H, D = 4, 128
    need = sum(-(-p // bs) + sum(-(-t // bs) + 1 for t in tails) for _, p, tails in groups) + 8
    alloc = pa.BlockAllocator(need, bs)
    rows, gs, pl = [], [0], []
    for members, prefix, tails in groups:
        assert members == len(tails) and prefix % bs == 0
        first = alloc.new_sequence()
        alloc.append(first, prefix)
        seqs = [first] + [alloc.fork(first) for _ in range(members - 1)]
        for sq, t in zip(seqs, tails):
            alloc.append(sq, t)
        rows += seqs
        gs.append(gs[-1] + members)
        pl.append(prefix)
    assert alloc.take_copies().shape[0] == 0  # whole-block prefixes: nothing copied
    tables = [alloc.block_table(r) for r in rows]
    ctx = np.array([alloc.length(r) for r in rows], dtype=np.int32)
    maxb = max(1, max(t.size for t in tables))
    bt = np.full((len(rows), maxb), -1, dtype=np.int32)
    for i, t in enumerate(tables):
        bt[i, :t.size] = t
    kc = normal(rng, (need, H, bs, D), dtype)
    vc = normal(rng, (need, H, bs, D), dtype)
    q = normal(rng, (len(rows), H, D), dtype)
    return kc, vc, q, bt, ctx, np.array(gs, dtype=np.int32), np.array(pl, dtype=np.int32)


@pytest.mark.parametrize("dtype,bs", [("f16", 16), ("bf16", 32), ("f16", 32), ("f32", 16), ("f16", 8),
                                      ("bf16", 64)])
def test_shared_prefix_decode_ragged_groups(dtype, bs):
    groups = [(1, 0, [37]), (3, bs, [0, 5, 700]), (8, 512, [0] * 4 + [1, 16, 300, 513]),
              (11, 1056 if bs in (8, 16) else 1024, [int(x) for x in np.arange(11) * 37]), (2, 512, [0, 0]),
              (5, 0, [1, 2, 3, 600, 1200]), (4, 520 if bs == 8 else 512, [9, 0, 33, 64]),
              (3, 2112 if bs >= 32 else 1040, [0, 7, 530])]  # several shared partitions at every block size
    kc, vc, q, bt, ctx, gs, pl = _grouped_batch(dtype, bs, groups, 31 + bs)
    H, D = q.shape[1], q.shape[2]
    scale = 1 / math.sqrt(D)
    ref = oracle.decode(q, kc, vc, bt, ctx, scale, dtype)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    maxctx = int(ctx.max())
    ws = pa.make_decode_shared_workspace(len(ctx), H, D, maxctx)
    dq, dk, dv = dev(q, dtype), dev(kc, dtype), dev(vc, dtype)
    pa.paged_attention_decode_shared_prefix(out, dq, dk, dv, dev(bt), dev(ctx), dev(gs), dev(pl), scale, maxctx,
                                            int(np.diff(gs).max()), int(pl.max()), ws, validate=True)
    _check_attention(out, ref, dtype)
    again = torch.empty_like(out)
    pa.paged_attention_decode_shared_prefix(again, dq, dk, dv, dev(bt), dev(ctx), dev(gs), dev(pl), scale, maxctx,
                                            int(np.diff(gs).max()), int(pl.max()), ws)
    assert torch.equal(out, again)


@pytest.mark.parametrize("n_groups", [63, 70])
def test_shared_prefix_decode_more_groups_than_a_wave_has_lanes(n_groups):
    """63 prefix-sharing groups (the most whose starts and prefixes one wave
    reads in a single load per lane) and 70: a row then finds its group by
    counting the group starts at or before it, 64 starts per ballot, so
    this takes two."""
    rng = np.random.default_rng(n_groups)
    groups = []
    for i in range(n_groups):
        n = 1 + i % 3
        groups.append((n, 16 * (i % 5), [int(t) for t in rng.integers(0, 40, n)]))
    kc, vc, q, bt, ctx, gs, pl = _grouped_batch("f16", 16, groups, 77)
    H, D = q.shape[1], q.shape[2]
    scale = 1 / math.sqrt(D)
    ref = oracle.decode(q, kc, vc, bt, ctx, scale, "f16")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    maxctx = int(ctx.max())
    ws = pa.make_decode_shared_workspace(len(ctx), H, D, maxctx)
    pa.paged_attention_decode_shared_prefix(out, dev(q, "f16"), dev(kc, "f16"), dev(vc, "f16"), dev(bt), dev(ctx),
                                            dev(gs), dev(pl), scale, maxctx, int(np.diff(gs).max()), int(pl.max()), ws,
                                            validate=True)
    _check_attention(out, ref, "f16")


# ----------------------------------------------------------------- prefill

@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("bs", [8, 16, 32, 64])
def test_prefill_parity_small_chunks(dtype, bs):
    prior = [0, 5, 33, 100, 0, 300]
    chunk = [1, 17, 64, 130, 200, 77]
    maxb = math.ceil(max(p + c for p, c in zip(prior, chunk)) / bs)
    wl = prefill_workload(f"pf_{dtype}_{bs}", 700 + bs, dtype, 4, 128, bs, prior, chunk, maxb=maxb, pool_factor=1.2)
    od = _on_device_written(wl)
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, bs, dtype)
    p = wl.prefill
    ref = oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, dtype)
    out32 = od.prefill(torch.float32)
    tol = ATOL[dtype]
    got = host(out32).astype(np.float64)
    err = np.abs(got - ref).max()
    assert err <= tol, f"prefill max abs err {err:.3e}"
    if dtype != "f32":
        outn = od.prefill(TORCH_DT[dtype])
        assert np.array_equal(bits(host(outn)), bits(rne(host(out32), dtype)))


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_prefill_empty_chunks_between_others(dtype):
    """Chunks of no queries (equal neighbours in query_start_loc) in the
    middle and at the end of the batch: their workgroups do nothing and the
    other chunks' rows are unaffected."""
    wl = prefill_workload(f"pf_empty_{dtype}", 712, dtype, 3, 128, 16, [40, 300, 0, 77, 5, 9],
                          [33, 0, 20, 0, 140, 0], maxb=24, pool_factor=1.2)
    od = _on_device_written(wl)
    p = wl.prefill
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, 16, dtype)
    ref = oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, dtype)
    got = host(od.prefill(torch.float32)).astype(np.float64)
    assert got.shape == ref.shape
    assert np.abs(got - ref).max() <= ATOL[dtype]


@pytest.mark.parametrize("dtype,bs", [("f16", 8), ("bf16", 16), ("f16", 64), ("f32", 8), ("f32", 64)])
def test_prefill_head_dim_64(dtype, bs):
    """head_dim 64: a wave's V rows of one load span two 8-token blocks at
    block size 8 (the kernel's per-lane block choice)."""
    prior = [0, 9, 40, 250]
    chunk = [3, 70, 129, 33]
    maxb = math.ceil(max(p + c for p, c in zip(prior, chunk)) / bs)
    wl = prefill_workload(f"pf64_{dtype}_{bs}", 760 + bs, dtype, 3, 64, bs, prior, chunk, maxb=maxb, pool_factor=1.3)
    od = _on_device_written(wl)
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, bs, dtype)
    p = wl.prefill
    ref = oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, dtype)
    got = host(od.prefill(torch.float32)).astype(np.float64)
    err = np.abs(got - ref).max()
    assert err <= ATOL[dtype], f"prefill max abs err {err:.3e}"


@pytest.mark.parametrize("dtype,bs", [("f16", 8), ("bf16", 16), ("f16", 32), ("bf16", 64), ("f32", 8), ("f32", 16)])
def test_prefill_tile_aligned_contexts(dtype, bs):
    """Contexts and chunk starts on multiples of the 32-key tile: the last key
    tile is full (no rows past the context to clear), and query tiles start
    exactly on key-tile edges. The pool's unused slots hold NaN poison, so a
    read past a context shows up as a non-finite output."""
    prior = [0, 32, 64, 96, 224]
    chunk = [32, 32, 64, 160, 64]
    maxb = math.ceil(max(p + c for p, c in zip(prior, chunk)) / bs)
    wl = prefill_workload(f"pf_aligned_{dtype}_{bs}", 780 + bs, dtype, 3, 128, bs, prior, chunk, maxb=maxb,
                          pool_factor=1.2)
    od = _on_device_written(wl)
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, bs, dtype)
    p = wl.prefill
    ref = oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, dtype)
    got = host(od.prefill(torch.float32)).astype(np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    assert err <= ATOL[dtype], f"prefill max abs err {err:.3e}"


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_prefill_negative_and_zero_scale(dtype, scale):
    """A negative scale (run as |scale| on sign-flipped queries) and a zero
    scale (every allowed key weighs the same; the causal mask still holds)."""
    prior, chunk = [0, 60, 200], [40, 100, 17]
    maxb = math.ceil(max(p + c for p, c in zip(prior, chunk)) / 16)
    wl = prefill_workload(f"pf_scale_{dtype}_{scale}", 770, dtype, 2, 128, 16, prior, chunk, maxb=maxb,
                          pool_factor=1.2, scale=scale)
    od = _on_device_written(wl)
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, 16, dtype)
    p = wl.prefill
    ref = oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, dtype)
    got = host(od.prefill(torch.float32)).astype(np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    assert err <= ATOL[dtype], f"prefill max abs err {err:.3e}"


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("scale", [None, 1.0])
def test_prefill_long_context_and_wide_scores(dtype, scale):
    """Contexts of hundreds of blocks (block ids read far into the table row)
    and, with scale 1, scores spread over hundreds of log2 units (the running
    max is raised and the accumulators rescaled many times)."""
    prior, chunk = [4500, 8200, 0], [70, 150, 90]
    maxb = math.ceil(max(p + c for p, c in zip(prior, chunk)) / 16)
    wl = prefill_workload(f"pf_long_{dtype}", 705, dtype, 2, 128, 16, prior, chunk, maxb=maxb, pool_factor=1.1,
                          scale=scale)
    od = _on_device_written(wl)
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, 16, dtype)
    p = wl.prefill
    ref = oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, dtype)
    got = host(od.prefill(torch.float32)).astype(np.float64)
    err = np.abs(got - ref).max()
    assert np.isfinite(got).all()
    assert err <= ATOL[dtype], f"prefill max abs err {err:.3e}"


@pytest.mark.parametrize("dtype,D,bs", [("f16", 128, 16), ("bf16", 128, 16), ("f16", 64, 32), ("bf16", 128, 64),
                                        ("f16", 128, 8), ("f32", 128, 16), ("f32", 64, 8)])
def test_prefill_many_workgroups_grouped_order(dtype, D, bs):
    """More query tiles than the chip holds at once (15 chunks x 13 heads x 4
    tiles of 128 queries = 780 workgroups, more than 3 per compute unit): the
    kernel then dispatches the query tiles of each (sequence, head) pair
    together, in groups of 8 pairs, as far as the chip holds them at once,
    and the pairs after those (a partial group here) by query tile, heaviest
    first. Every
    output element against the oracle, and the first two chunks bit-identical to a call
    that holds only them (104 workgroups, every one resident at once: the
    plain order, run by the kernel's wide shape of 8 waves x 16 queries
    where head dim is 128)."""
    rng = np.random.default_rng(11)
    prior = [int(x) for x in rng.integers(0, 600, 15)]
    chunk = [int(x) for x in rng.integers(385, 513, 15)]
    chunk[0] = 512
    maxb = math.ceil(max(a + b for a, b in zip(prior, chunk)) / bs)
    wl = prefill_workload(f"pf_grouped_{dtype}_{D}_{bs}", 706 + bs, dtype, 13, D, bs, prior, chunk, maxb=maxb,
                          pool_factor=1.1)
    od = _on_device_written(wl)
    p = wl.prefill
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, bs, dtype)
    out32 = host(od.prefill(torch.float32))
    got = out32.astype(np.float64)
    assert np.isfinite(got).all()
    ref = oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, dtype)
    err = np.abs(got - ref).max()
    assert err <= ATOL[dtype], f"prefill max abs err {err:.3e}"
    n2 = int(p.query_start_loc[2])
    sub = torch.empty((n2, wl.num_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    pa.paged_attention_prefill(sub, od.pf_q[:n2], od.k_cache, od.v_cache, od.pf_block_tables[:2],
                               od.pf_context_lens[:2], od.pf_qsl[:3], wl.scale, max_q_len=p.max_q_len,
                               max_context_len=p.max_context_len)
    assert np.array_equal(bits(host(sub)), bits(out32[:n2]))
    outn = od.prefill(TORCH_DT[dtype])
    assert np.array_equal(bits(host(outn)), bits(rne(out32, dtype)))


def test_prefill_bench_workload_full_output():
    """bench.py's compute-bound prefill (8 chunks of 512 queries after 1536
    cached tokens, 40 heads: 1280 workgroups, the grouped order) in the
    launch configuration it times: every output element against the oracle
    (150 GFLOP of fp64 work), and the output in the input type equal to the
    rounded f32 output."""
    import bench
    wl = bench.prefill_config()
    od = _on_device_written(wl)
    p = wl.prefill
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping,
                                      wl.block_size, wl.dtype)
    out32 = host(od.prefill(torch.float32))
    assert np.isfinite(out32).all()
    ref = oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, wl.dtype)
    err = np.abs(out32.astype(np.float64) - ref).max()
    print(f"prefill_long max abs err {err:.3e}")
    assert err <= ATOL[wl.dtype]
    outn = od.prefill(TORCH_DT[wl.dtype])
    assert np.array_equal(bits(host(outn)), bits(rne(out32, wl.dtype)))


def test_prefill_f32_bench_workload_full_output():
    """bench.py's f32 prefill (the mixed step's 4 chunks with f32 caches,
    40 heads x 128, 640 workgroups) in the launch configuration it times:
    every output element against the oracle."""
    import bench
    wl = bench.prefill_config("prefill_f32")
    od = _on_device_written(wl)
    p = wl.prefill
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping,
                                      wl.block_size, wl.dtype)
    out32 = host(od.prefill(torch.float32))
    assert np.isfinite(out32).all()
    ref = oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, wl.dtype)
    err = np.abs(out32.astype(np.float64) - ref).max()
    print(f"prefill_f32 max abs err {err:.3e}")
    assert err <= ATOL[wl.dtype]


def test_prefill_config5_full_output():
    """The mixed step's 4 causal chunks (40 heads x 128, f16, bs 16): every
    output element against the oracle, and the output in the input type
    equal to the rounded f32 output."""
    wl, _, _ = _config(5)
    od = _on_device_written(wl)
    out32 = host(od.prefill(torch.float32))
    assert np.isfinite(out32).all()
    ref = _oracle_prefill(5)
    assert out32.shape == ref.shape
    err = np.abs(out32.astype(np.float64) - ref).max()
    print(f"config 5 prefill max abs err {err:.3e}")
    assert err <= ATOL[wl.dtype]
    outn = od.prefill(TORCH_DT[wl.dtype])
    assert np.array_equal(bits(host(outn)), bits(rne(out32, wl.dtype)))


def test_prefill_single_query_chunk_matches_decode():
    ctx = [1, 40, 300, 1000]
    wl = prefill_workload("pf1", 704, "f16", 4, 128, 16, [c - 1 for c in ctx], [1] * 4, maxb=64)
    od = _on_device_written(wl)
    p = wl.prefill
    pf = host(od.prefill(torch.float32)).astype(np.float64)
    out = torch.empty((4, 4, 128), dtype=torch.float32, device="cuda")
    pa.paged_attention_decode(out, od.pf_q, od.k_cache, od.v_cache, od.pf_block_tables, od.pf_context_lens,
                              wl.scale, max_context_len=p.max_context_len)
    assert np.abs(pf - host(out).astype(np.float64)).max() <= 2 * ATOL["f16"]


# ------------------------------------------------------------- HIP graphs

def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_mixed_step_graph_replays_match_eager():
    """The whole mixed step (cache write, prefill, split-K decode) captured as
    a HIP graph: every replay, with eager work and syncs in between, equals the
    eager step bit for bit."""
    wl, _, _ = _config(5)
    od = OnDevice(wl)
    d, p = wl.decode, wl.prefill
    ws = pa.make_decode_workspace(d.num_seqs, wl.num_heads, wl.head_dim, d.max_context_len)
    dout = torch.empty_like(od.q)
    pout = torch.empty_like(od.pf_q)

    def step():
        pa.reshape_and_cache(od.new_k, od.new_v, od.k_cache, od.v_cache, od.slot_mapping)
        pa.paged_attention_prefill(pout, od.pf_q, od.k_cache, od.v_cache, od.pf_block_tables, od.pf_context_lens,
                                   od.pf_qsl, wl.scale, p.max_q_len, p.max_context_len)
        pa.paged_attention_decode(dout, od.q, od.k_cache, od.v_cache, od.block_tables, od.context_lens, wl.scale,
                                  d.max_context_len, ws)

    step()
    torch.cuda.synchronize()
    dref, pref = dout.clone(), pout.clone()
    g = _capture(step)
    for i in range(4):
        dout.zero_()
        pout.zero_()
        extra = od.decode(torch.float32)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dout, dref), f"decode differs on replay {i}"
        assert torch.equal(pout, pref), f"prefill differs on replay {i}"
        assert torch.isfinite(extra).all()


def test_decode_with_cache_write_graph_replays_match_eager():
    """The decode call with the cache write inside (LLaMA-7B workload)
    captured as a HIP graph: before every replay the new tokens' slots are
    overwritten with other values (eager launches); every replay gives the
    eager output bit for bit and puts the new tokens back into their slots."""
    wl, _, _ = _config(2)
    d = wl.decode
    od = OnDevice(wl)
    ws = pa.make_decode_workspace(d.num_seqs, wl.num_heads, wl.head_dim, d.max_context_len)
    out = torch.empty_like(od.q)
    poison_k = torch.randn_like(od.new_k.float()).to(od.new_k.dtype)
    poison_v = torch.randn_like(od.new_v.float()).to(od.new_v.dtype)

    def step():
        pa.paged_attention_decode_with_cache_write(out, od.q, od.k_cache, od.v_cache, od.new_k, od.new_v,
                                                   od.slot_mapping, od.block_tables, od.context_lens, wl.scale,
                                                   d.max_context_len, ws)

    step()
    torch.cuda.synchronize()
    ref, kref, vref = out.clone(), od.k_cache.clone(), od.v_cache.clone()
    g = _capture(step)
    def same(x, y):  # bit for bit (the caches' unused slots hold NaN poison)
        return torch.equal(x.view(torch.int16), y.view(torch.int16))

    for i in range(4):
        out.zero_()
        pa.reshape_and_cache(poison_k, poison_v, od.k_cache, od.v_cache, od.slot_mapping)
        torch.cuda.synchronize()
        assert not same(od.k_cache, kref)
        g.replay()
        torch.cuda.synchronize()
        assert same(out, ref), f"output differs on replay {i}"
        assert same(od.k_cache, kref) and same(od.v_cache, vref), f"caches differ on replay {i}"


@pytest.mark.parametrize("side,dtype", [(False, None), (True, None), (True, "f32")])
def test_attention_step_matches_the_separate_calls(side, dtype):
    """One scheduler iteration in one call (cache write, prefill, decode),
    in order on one stream or with the prefill on a side stream (and with
    f32 caches): both fp32 outputs within tolerance of the oracle on every
    element, outputs and caches equal, bit for bit, those of the three
    separate calls; captured as a graph (fork/join across the two streams),
    every replay too."""
    args = (5,) if dtype is None else (5, dtype)  # the same cache entries as the other tests
    wl, _, _ = _config(*args)
    d, p = wl.decode, wl.prefill
    ref = OnDevice(wl)
    ws = pa.make_decode_workspace(d.num_seqs, wl.num_heads, wl.head_dim, d.max_context_len)
    ref.write_new_tokens()
    pref = torch.empty_like(ref.pf_q, dtype=torch.float32)
    dref = torch.empty_like(ref.q, dtype=torch.float32)
    pa.paged_attention_prefill(pref, ref.pf_q, ref.k_cache, ref.v_cache, ref.pf_block_tables, ref.pf_context_lens,
                               ref.pf_qsl, wl.scale, p.max_q_len, p.max_context_len)
    pa.paged_attention_decode(dref, ref.q, ref.k_cache, ref.v_cache, ref.block_tables, ref.context_lens, wl.scale,
                              d.max_context_len, ws)
    torch.cuda.synchronize()

    od = OnDevice(wl)
    pout = torch.empty_like(od.pf_q, dtype=torch.float32)
    dout = torch.empty_like(od.q, dtype=torch.float32)
    ws2 = pa.make_decode_workspace(d.num_seqs, wl.num_heads, wl.head_dim, d.max_context_len)
    side_stream = torch.cuda.Stream() if side else None
    fe, je = pa.make_step_events() if side else (None, None)

    def step():
        pa.attention_step(od.k_cache, od.v_cache, wl.scale, od.new_k, od.new_v, od.slot_mapping,
                          prefill_out=pout, prefill_q=od.pf_q, prefill_block_tables=od.pf_block_tables,
                          prefill_context_lens=od.pf_context_lens, prefill_query_start_loc=od.pf_qsl,
                          prefill_max_q_len=p.max_q_len, prefill_max_context_len=p.max_context_len,
                          decode_out=dout, decode_q=od.q, decode_block_tables=od.block_tables,
                          decode_context_lens=od.context_lens, decode_max_context_len=d.max_context_len,
                          workspace=ws2, side_stream=side_stream, fork_event=fe, join_event=je)

    step()
    torch.cuda.synchronize()
    assert torch.equal(pout, pref) and torch.equal(dout, dref)
    # and the step's own outputs against the oracle, element by element
    _check_attention(pout, _oracle_prefill(*args), wl.dtype)
    _check_attention(dout, _oracle_decode(*args), wl.dtype)
    # unused slots hold NaN poison: compare the caches' bits
    assert np.array_equal(bits(host(od.k_cache)), bits(host(ref.k_cache)))
    assert np.array_equal(bits(host(od.v_cache)), bits(host(ref.v_cache)))
    g = _capture(step)
    for i in range(3):
        pout.zero_()
        dout.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(pout, pref), f"prefill differs on replay {i}"
        assert torch.equal(dout, dref), f"decode differs on replay {i}"
