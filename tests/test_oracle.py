"""Pins for the fp64 oracle: each check ties it to something other than itself
(a library routine, brute force written independently, closed forms, the
method's invariants) so that a dropped term, a wrong sign or index or a
transposed operand in the oracle fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests._dense import dense_attention, draw, page, to64
from workloads import POISON_BITS, bits, config1, config4, decode_workload, poison_array, prefill_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- widening

def test_widen_f16_every_bit_pattern_matches_numpy():
    pat = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.widen(pat.view(np.float16), "f16")
    ref = pat.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_widen_bf16_every_bit_pattern_matches_torch():
    pat = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.widen(pat, "bf16")
    ref = torch.from_numpy(pat.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_widen_f32_exact():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32) * 1e3
    assert np.array_equal(oracle.widen(x, "f32"), x.astype(np.float64))


# ------------------------------------------------------------- brute force

def _random_case(rng, dtype, ctxs, H, D, bs, extra_blocks=5):
    ks = [draw(rng, (c, H, D), dtype) for c in ctxs]
    vs = [draw(rng, (c, H, D), dtype) for c in ctxs]
    need = sum(math.ceil(c / bs) for c in ctxs)
    kc, vc, bt = page(ks, vs, bs, need + extra_blocks, rng, dtype)
    return ks, vs, kc, vc, bt


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bs", [16, 32])
def test_decode_matches_dense_brute_force(dtype, bs):
    rng = np.random.default_rng(7 + bs)
    H, D = 2, 24
    ctxs = [1, 5, bs, bs + 1, 40, 3 * bs - 1]
    ks, vs, kc, vc, bt = _random_case(rng, dtype, ctxs, H, D, bs)
    q = draw(rng, (len(ctxs), H, D), dtype)
    scale = 0.37
    got = oracle.decode(q, kc, vc, bt, np.array(ctxs), scale, dtype)
    for s, c in enumerate(ctxs):
        for h in range(H):
            ref = dense_attention(to64(q[s, h], dtype), to64(ks[s][:, h], dtype), to64(vs[s][:, h], dtype), scale)
            np.testing.assert_allclose(got[s, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_prefill_matches_dense_brute_force_with_explicit_mask(dtype):
    rng = np.random.default_rng(11)
    H, D, bs = 2, 16, 16
    prior, chunk = [0, 3, 17, 30], [5, 1, 20, 33]
    ctxs = [p + L for p, L in zip(prior, chunk)]
    ks, vs, kc, vc, bt = _random_case(rng, dtype, ctxs, H, D, bs)
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = draw(rng, (int(qsl[-1]), H, D), dtype)
    scale = 0.25
    got = oracle.prefill(q, kc, vc, bt, np.array(ctxs), qsl, scale, dtype)
    for s in range(len(ctxs)):
        c = ctxs[s]
        # mask[j, t]: query j of the chunk is at position prior+j
        mask = np.arange(c)[None, :] <= (prior[s] + np.arange(chunk[s]))[:, None]
        for j in range(chunk[s]):
            r = qsl[s] + j
            for h in range(H):
                ref = dense_attention(to64(q[r, h], dtype), to64(ks[s][:, h], dtype), to64(vs[s][:, h], dtype),
                                      scale, mask[j])
                np.testing.assert_allclose(got[r, h], ref, rtol=0, atol=1e-12)


def test_prefill_without_prior_equals_torch_causal_sdpa():
    rng = np.random.default_rng(12)
    H, D, bs, L = 3, 32, 16, 45
    ks, vs, kc, vc, bt = _random_case(rng, "f32", [L], H, D, bs)
    q = draw(rng, (L, H, D), "f32")
    got = oracle.prefill(q, kc, vc, bt, np.array([L]), np.array([0, L]), 1 / math.sqrt(D), "f32")
    tq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]
    tk = torch.from_numpy(ks[0].astype(np.float64)).permute(1, 0, 2)[None]
    tv = torch.from_numpy(vs[0].astype(np.float64)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_prefill_with_prior_equals_torch_sdpa_bottom_right_mask():
    rng = np.random.default_rng(13)
    H, D, bs, c, L = 2, 32, 16, 23, 18
    ks, vs, kc, vc, bt = _random_case(rng, "f32", [c + L], H, D, bs)
    q = draw(rng, (L, H, D), "f32")
    got = oracle.prefill(q, kc, vc, bt, np.array([c + L]), np.array([0, L]), 0.2, "f32")
    mask = torch.arange(c + L)[None, :] <= (c + torch.arange(L))[:, None]
    tq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]
    tk = torch.from_numpy(ks[0].astype(np.float64)).permute(1, 0, 2)[None]
    tv = torch.from_numpy(vs[0].astype(np.float64)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.2)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------ closed forms

def test_golden_closed_form_example():
    g = json.load(open(os.path.join(GOLDEN, "closed_form_attention.json")))
    bs, D = g["block_size"], g["head_dim"]
    k = np.array(g["k_logical"], np.float32)
    v = np.array(g["v_logical"], np.float32)
    nb = g["num_blocks"]
    kc = poison_array((nb, 1, bs, D), "f32")
    vc = poison_array((nb, 1, bs, D), "f32")
    for t in range(k.shape[0]):
        b = g["block_table"][t // bs]
        kc[b, 0, t % bs] = k[t]
        vc[b, 0, t % bs] = v[t]
    q = np.array(g["q"], np.float32).reshape(1, 1, D)
    bt = np.array([g["block_table"]], np.int32)
    out = oracle.decode(q, kc, vc, bt, np.array([k.shape[0]]), g["scale"], "f32")
    np.testing.assert_allclose(out[0, 0], g["expected_out"], rtol=0, atol=g["tolerance"])


def test_single_token_returns_its_value_row_exactly():
    wl = config1()  # sequence 0 has one token, which is new this step
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping,
                                      wl.block_size, wl.dtype)
    d = wl.decode
    out = oracle.decode(d.q, kc, vc, d.block_tables, d.context_lens, wl.scale, wl.dtype)
    assert d.context_lens[0] == 1
    assert np.array_equal(out[0], wl.new.v[0].astype(np.float64))


def test_zero_query_and_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    H, D, bs, c = 2, 16, 16, 37
    ks, vs, kc, vc, bt = _random_case(rng, "f16", [c], H, D, bs)
    zero_q = np.zeros((1, H, D), np.float16)
    out = oracle.decode(zero_q, kc, vc, bt, np.array([c]), 0.5, "f16")
    mean = vs[0].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[0], mean, rtol=0, atol=1e-13)
    same_k = [np.broadcast_to(ks[0][:1], ks[0].shape).copy()]
    kc2, vc2, bt2 = page(same_k, vs, bs, 4, rng, "f16")
    q = draw(rng, (1, H, D), "f16")
    out2 = oracle.decode(q, kc2, vc2, bt2, np.array([c]), 0.5, "f16")
    np.testing.assert_allclose(out2[0], mean, rtol=0, atol=1e-13)


def test_dominant_key_selects_its_value_row():
    rng = np.random.default_rng(4)
    H, D, bs, c, j = 1, 64, 16, 50, 29
    q = draw(rng, (1, H, D), "f32")
    k = draw(rng, (c, H, D), "f32")
    qv = q[0, 0].astype(np.float64)
    k[j, 0] = (50.0 * qv / np.linalg.norm(qv) * math.sqrt(D)).astype(np.float32)
    v = draw(rng, (c, H, D), "f32")
    kc, vc, bt = page([k], [v], bs, 6, rng, "f32")
    out = oracle.decode(q, kc, vc, bt, np.array([c]), 1 / math.sqrt(D), "f32")
    np.testing.assert_allclose(out[0, 0], v[j, 0].astype(np.float64), rtol=0, atol=1e-12)


def test_affine_map_of_values_passes_through():
    """Softmax weights sum to one, so out(a*V + b) = a*out(V) + b."""
    rng = np.random.default_rng(5)
    H, D, bs, c = 2, 8, 16, 33
    ks = [draw(rng, (c, H, D), "f32")]
    vs = [draw(rng, (c, H, D), "f16").astype(np.float32)]  # 11-bit values: 2v+3 stays exact in f32
    kc, vc, bt = page(ks, vs, bs, 3, rng, "f32")
    q = draw(rng, (1, H, D), "f32")
    base = oracle.decode(q, kc, vc, bt, np.array([c]), 0.3, "f32")
    vs2 = [(vs[0] * np.float32(2.0) + np.float32(3.0)).astype(np.float32)]
    assert np.array_equal(vs2[0].astype(np.float64), 2.0 * vs[0].astype(np.float64) + 3.0)
    kc2, vc2, bt2 = page(ks, vs2, bs, 3, rng, "f32")
    out = oracle.decode(q, kc2, vc2, bt2, np.array([c]), 0.3, "f32")
    np.testing.assert_allclose(out, 2.0 * base + 3.0, rtol=0, atol=1e-12)


def test_empty_context_gives_zeros():
    rng = np.random.default_rng(6)
    ks, vs, kc, vc, bt = _random_case(rng, "f32", [5], 1, 8, 16)
    q = draw(rng, (2, 1, 8), "f32")
    bt2 = np.concatenate([bt, np.full_like(bt, -1)])
    out = oracle.decode(q, kc, vc, bt2, np.array([5, 0]), 1.0, "f32")
    assert np.array_equal(out[1], np.zeros((1, 8)))


# -------------------------------------------------------------- invariants

def _decode(wl, kc=None, vc=None, bt=None):
    d = wl.decode
    return oracle.decode(d.q, wl.k_cache if kc is None else kc, wl.v_cache if vc is None else vc,
                         d.block_tables if bt is None else bt, d.context_lens, wl.scale, wl.dtype)


def _with_new_tokens(wl):
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping,
                                      wl.block_size, wl.dtype)
    wl.k_cache, wl.v_cache = kc, vc
    return wl


def test_output_is_bit_identical_under_physical_block_permutation():
    wl = _with_new_tokens(decode_workload("perm", 21, "f16", 2, 64, 16, [3, 16, 47, 90], maxb=8, pool_blocks=20))
    base = _decode(wl)
    perm = np.random.default_rng(0).permutation(wl.num_blocks)  # block b moves to perm[b]
    kc = np.empty_like(wl.k_cache)
    vc = np.empty_like(wl.v_cache)
    kc[perm] = wl.k_cache
    vc[perm] = wl.v_cache
    bt = wl.decode.block_tables.copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    assert np.array_equal(_decode(wl, kc, vc, bt), base)


def test_output_is_bit_identical_when_shared_prefix_blocks_are_private_copies():
    wl = _with_new_tokens(config4(prompts=2, samples=3, prompt_len=64, max_tail=40, H=2, D=64))
    base = _decode(wl)
    # give every sequence private copies of its shared blocks
    bt = wl.decode.block_tables.copy()
    kc, vc = [wl.k_cache], [wl.v_cache]
    nb = wl.num_blocks
    n_shared = 0
    for s in range(bt.shape[0]):
        for i in range(bt.shape[1]):
            b = bt[s, i]
            if b >= 0 and wl.notes["refcount"][b] > 1:
                kc.append(wl.k_cache[b:b + 1])
                vc.append(wl.v_cache[b:b + 1])
                bt[s, i] = nb
                nb += 1
                n_shared += 1
    assert n_shared > 0
    out = _decode(wl, np.concatenate(kc), np.concatenate(vc), bt)
    assert np.array_equal(out, base)


def test_output_ignores_unread_slots_and_stale_table_entries():
    wl = _with_new_tokens(decode_workload("stale", 22, "bf16", 2, 64, 32, [1, 31, 33, 64, 70], maxb=4,
                                          pool_blocks=12))
    base = _decode(wl)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    poisoned = bits(kc, "bf16") == POISON_BITS["bf16"]
    assert poisoned.any()
    bits(kc, "bf16")[poisoned] = 0x7F80  # +inf instead of NaN
    bits(vc, "bf16")[bits(vc, "bf16") == POISON_BITS["bf16"]] = 0x4479  # 1000.0
    bt = wl.decode.block_tables.copy()
    bt[bt < 0] = 10 ** 6
    assert np.array_equal(_decode(wl, kc, vc, bt), base)


def test_output_is_bit_identical_under_reblocking_16_to_32():
    rng = np.random.default_rng(8)
    H, D = 2, 32
    ctxs = [9, 16, 33, 64, 77]
    ks = [draw(rng, (c, H, D), "f16") for c in ctxs]
    vs = [draw(rng, (c, H, D), "f16") for c in ctxs]
    q = draw(rng, (len(ctxs), H, D), "f16")
    outs = []
    for bs in (16, 32):
        kc, vc, bt = page(ks, vs, bs, 30, rng, "f16")
        outs.append(oracle.decode(q, kc, vc, bt, np.array(ctxs), 0.3, "f16"))
    assert np.array_equal(outs[0], outs[1])


def test_last_prefill_row_equals_decode_and_single_query_chunk_equals_decode():
    wl = _with_new_tokens(prefill_workload("pf", 23, "f16", 2, 64, 16, prior=[0, 7, 40], chunk=[9, 1, 30], maxb=8))
    p = wl.prefill
    out = oracle.prefill(p.q, wl.k_cache, wl.v_cache, p.block_tables, p.context_lens, p.query_start_loc,
                         wl.scale, wl.dtype)
    last = p.query_start_loc[1:] - 1
    dec = oracle.decode(p.q[last], wl.k_cache, wl.v_cache, p.block_tables, p.context_lens, wl.scale, wl.dtype)
    assert np.array_equal(out[last], dec)


def test_sampled_pairs_match_full_run():
    wl = _with_new_tokens(config1())
    full = _decode(wl)
    pairs = np.array([[3, 1], [0, 0], [2, 1]])
    d = wl.decode
    got = oracle.decode(d.q, wl.k_cache, wl.v_cache, d.block_tables, d.context_lens, wl.scale, wl.dtype,
                        pairs=pairs)
    assert np.array_equal(got, full[pairs[:, 0], pairs[:, 1]])


# -------------------------------------------------- cache writes and gather

def test_reshape_and_cache_round_trip_and_untouched_slots():
    wl = decode_workload("rt", 24, "f16", 3, 64, 16, [5, 16, 17, 40], maxb=4, pool_blocks=16)
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping,
                                      wl.block_size, wl.dtype)
    sm = wl.new.slot_mapping
    blk, off = sm // 16, sm % 16
    # independent readback of the written slots
    assert np.array_equal(bits(kc[blk, :, off, :], "f16"), bits(wl.new.k, "f16"))
    assert np.array_equal(bits(vc[blk, :, off, :], "f16"), bits(wl.new.v, "f16"))
    # every other slot keeps its old bits
    written = np.zeros((wl.num_blocks, 16), bool)
    written[blk, off] = True
    keep = ~written
    assert np.array_equal(bits(kc, "f16").transpose(0, 2, 1, 3)[keep], bits(wl.k_cache, "f16").transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(bits(vc, "f16").transpose(0, 2, 1, 3)[keep], bits(wl.v_cache, "f16").transpose(0, 2, 1, 3)[keep])


def test_reshape_and_cache_skips_negative_and_rejects_bad_slots():
    wl = decode_workload("neg", 25, "f32", 1, 64, 16, [4, 9], maxb=1, pool_blocks=4)
    sm = wl.new.slot_mapping.copy()
    sm[0] = -1
    kc, _ = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, sm, 16, "f32")
    b, o = divmod(int(wl.new.slot_mapping[0]), 16)
    assert np.array_equal(bits(kc[b, :, o], "f32"), bits(wl.k_cache[b, :, o], "f32"))
    for bad in ([5, 5], [0, 4 * 16]):
        with pytest.raises(oracle.OracleError):
            oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, np.array(bad), 16, "f32")


def test_gather_matches_independent_index_arithmetic():
    wl = _with_new_tokens(decode_workload("g", 26, "bf16", 2, 64, 32, [1, 32, 33, 100], maxb=4, pool_blocks=10))
    d = wl.decode
    ko, vo = oracle.gather_kv(wl.k_cache, wl.v_cache, d.block_tables, d.context_lens, "bf16")
    row = 0
    for s, c in enumerate(d.context_lens):
        t = np.arange(c)
        phys = d.block_tables[s, t // 32]
        assert np.array_equal(bits(ko[row:row + c], "bf16"), bits(wl.k_cache[phys, :, t % 32, :], "bf16"))
        assert np.array_equal(bits(vo[row:row + c], "bf16"), bits(wl.v_cache[phys, :, t % 32, :], "bf16"))
        row += c
    assert not np.any(bits(ko, "bf16") == POISON_BITS["bf16"])


def test_out_of_range_block_id_is_rejected():
    wl = decode_workload("bad", 27, "f32", 1, 64, 16, [20], maxb=2, pool_blocks=3)
    bt = wl.decode.block_tables.copy()
    bt[0, 1] = -1
    with pytest.raises(oracle.OracleError):
        oracle.decode(wl.decode.q, wl.k_cache, wl.v_cache, bt, wl.decode.context_lens, 1.0, "f32")
    bt[0, 1] = 3
    with pytest.raises(oracle.OracleError):
        oracle.decode(wl.decode.q, wl.k_cache, wl.v_cache, bt, wl.decode.context_lens, 1.0, "f32")


def test_copy_blocks_matches_numpy_block_assignment_and_rejects_ambiguous_maps():
    """Copy-on-write copies: block dst of both caches equals block src bit for
    bit, every other block is untouched (numpy fancy-index assignment is the
    independent reference); a destination named twice, a destination that is
    also a source, and ids outside the pool are rejected."""
    rng = np.random.default_rng(11)
    for dtype, shape in (("f16", (12, 3, 16, 64)), ("bf16", (9, 2, 32, 128)), ("f32", (7, 2, 16, 64))):
        n = int(np.prod(shape))
        kc = (rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16) if dtype != "f32"
              else rng.standard_normal(n).astype(np.float32)).reshape(shape)
        if dtype == "f16":
            kc = kc.view(np.float16)
        vc = kc[::-1].copy()
        perm = rng.permutation(shape[0])
        pairs = np.stack([perm[:3], perm[3:6]], 1).astype(np.int32)
        k2, v2 = oracle.copy_blocks(kc, vc, pairs, dtype)
        ek, ev = kc.copy(), vc.copy()
        ek[pairs[:, 1]] = kc[pairs[:, 0]]
        ev[pairs[:, 1]] = vc[pairs[:, 0]]
        view = {"f16": np.uint16, "bf16": np.uint16, "f32": np.uint32}[dtype]
        assert np.array_equal(k2.view(view), ek.view(view)) and np.array_equal(v2.view(view), ev.view(view))
        assert not np.array_equal(k2.view(view), kc.view(view))
        for bad in ([[0, 1], [2, 1]], [[0, 1], [1, 2]], [[0, shape[0]]], [[-1, 1]]):
            with pytest.raises(oracle.OracleError):
                oracle.copy_blocks(kc, vc, bad, dtype)
