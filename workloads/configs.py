"""Seeded synthetic inputs for paged-KV attention.

Input construction only: lengths, block tables, slot mappings, random q/K/V
and poison for never-written slots. Nothing here computes attention or moves
cached K/V for a kernel; both the fp64 oracle and the HIP library consume the
arrays built here.

Workloads (sizes follow the shapes the pages talk about: LLaMA-7B has 32
heads x 128, LLaMA-13B 40 x 128, block sizes 16/32, max_num_seqs 256,
max_model_len 4096, a per-step token budget of 2048):

1. ``tiny``      4 seqs, 2 heads, d 64, f32, bs 16, ctx {1,17,33,100},
                 13 blocks at random places in a 64-block pool.
2. ``llama7b``   64 seqs, 32 heads, d 128, f16, bs 16, ctx ~ U[128,2048],
                 pool sized to fit exactly, tables = slices of one random
                 permutation.
3. ``mixed256``  256 seqs, 32 x 128, bf16, bs 32, ctx ~ round(LogNormal(
                 ln 600 - 1/2, 1)) clipped to [1,4096]; pool 1.25x the blocks
                 needed, used blocks at random places.
4. ``prefix13b`` 32 prompts x 8 samples, 40 x 128, f16, bs 16, prompt 1024
                 tokens shared by its 8 samples (refcount 8), per-sample tail
                 ~ U[0,256] in private blocks. ``cow=True`` shortens each
                 prompt by r ~ U[1,15] tokens so that its last block is
                 partial and is copied on write by samples that extend it.
5. ``mixed_step`` 40 x 128, f16, bs 16: 2048 new-token rows (4 prefill
                 chunks with L ~ U[256,512] over prior context c ~ U[0,1024],
                 96 decode tokens with ctx ~ U[256,4096], then filler rows to
                 random unused slots), then causal prefill of the 4 chunks and
                 decode of the 96 sequences.

Conventions: a decode sequence's last token (position ctx-1) and a prefill
chunk's tokens are *new* this step: they are poison in the pool and arrive as
rows of ``new.k``/``new.v`` with their slots in ``new.slot_mapping`` (slot =
block * block_size + offset, -1 = skip). All earlier tokens are already in the
pool. Slots that no sequence references hold a quiet-NaN poison pattern, and
block-table entries past a sequence's last block are -1.

q/K/V values are N(0,1) float32 draws rounded to nearest-even in the storage
dtype. bf16 is stored as its uint16 bit pattern. Seeds are 391 + config id
with one spawned child stream per array family, so that changing one shape
does not shift the others.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .allocator import BlockAllocator, Sequence

DTYPES = ("f32", "f16", "bf16")
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
# quiet NaNs with a recognisable payload
POISON_BITS = {"f32": 0x7FC55555, "f16": 0x7E55, "bf16": 0x7FD5}
_BITS_VIEW = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}

BASE_SEED = 391
_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))

CONFIG_NAMES = {1: "tiny", 2: "llama7b", 3: "mixed256", 4: "prefix13b", 5: "mixed_step"}


def bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Raw bit view of a storage array."""
    return a.view(_BITS_VIEW[dtype])


def f32_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (nearest-even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    u = x.view(np.uint32)
    r = (u >> 16) + (((u & 0xFFFF) + ((u >> 16) & 1)) > 0x8000)
    return r.astype(np.uint16)


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of storage values to float32 (bf16 by bit shift)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def _fill_chunk(args):
    g, out, dtype = args
    out[:] = f32_to_storage(g.standard_normal(out.shape[0], dtype=np.float32), dtype)


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) draws rounded to ``dtype``. The draw is split into fixed chunks
    of 2**22 values, each from its own child of ``rng``, so the result does
    not depend on how many threads fill it."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=STORAGE[dtype])
    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks:
        gens = rng.spawn(nchunks)
        jobs = [(g, out[i * _CHUNK: min(n, (i + 1) * _CHUNK)], dtype) for i, g in enumerate(gens)]
        if nchunks == 1:
            _fill_chunk(jobs[0])
        else:
            with ThreadPoolExecutor(min(_THREADS, nchunks)) as ex:
                list(ex.map(_fill_chunk, jobs))
    return out.reshape(shape)


def poison_array(shape, dtype: str) -> np.ndarray:
    return np.full(shape, POISON_BITS[dtype], dtype=_BITS_VIEW[dtype]).view(STORAGE[dtype])


@dataclass
class DecodeBatch:
    q: np.ndarray             # [S,H,D] storage dtype
    block_tables: np.ndarray  # int32 [S,maxb]
    context_lens: np.ndarray  # int32 [S]

    @property
    def num_seqs(self):
        return int(self.context_lens.shape[0])

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if self.context_lens.size else 0


@dataclass
class PrefillBatch:
    q: np.ndarray                # [sum L, H, D]
    block_tables: np.ndarray     # int32 [S,maxb]
    context_lens: np.ndarray     # int32 [S], includes the chunk
    query_start_loc: np.ndarray  # int32 [S+1]

    @property
    def num_seqs(self):
        return int(self.context_lens.shape[0])

    @property
    def total_q(self):
        return int(self.query_start_loc[-1])

    @property
    def max_q_len(self):
        return int(np.diff(self.query_start_loc).max()) if self.num_seqs else 0

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if self.context_lens.size else 0


@dataclass
class NewTokens:
    k: np.ndarray             # [T,H,D]
    v: np.ndarray             # [T,H,D]
    slot_mapping: np.ndarray  # int32 [T]


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    k_cache: np.ndarray  # [nb,H,bs,D], state before this step's writes
    v_cache: np.ndarray
    new: NewTokens
    decode: DecodeBatch | None = None
    prefill: PrefillBatch | None = None
    notes: dict = field(default_factory=dict)

    @property
    def elt_bytes(self):
        return ELT_BYTES[self.dtype]


# ---------------------------------------------------------------------------
# builder: tables first (allocator), then a random placement in the pool, then
# contents replayed in write order


class _Builder:
    def __init__(self, block_size: int):
        # generous virtual pool, sequential ids; compacted afterwards
        self.alloc = BlockAllocator(1 << 17, block_size)
        self.bs = block_size
        self.events = []  # ("write", slots) | ("copy", src, dst)

    def append(self, seq: Sequence, n: int, record: bool = True) -> list[int]:
        c0 = len(self.alloc.copies)
        slots = self.alloc.append(seq, n)
        new_copies = self.alloc.copies[c0:]
        # the only copy-on-write an append can trigger is before its first token
        for src, dst in new_copies:
            self.events.append(("copy", src, dst))
        if record and slots:
            self.events.append(("write", slots))
        return slots

    def place(self, seqs, pool_blocks: int | None, rng: np.random.Generator, extra_blocks: int = 0):
        used = sorted({b for s in seqs for b in s.table} |
                      {b for e in self.events if e[0] == "copy" for b in e[1:]})
        n_used = len(used)
        nb = n_used + extra_blocks if pool_blocks is None else pool_blocks
        if nb < n_used:
            raise ValueError("pool too small")
        dest = rng.permutation(nb)[:n_used]
        remap = dict(zip(used, (int(x) for x in dest)))
        return nb, remap


def _tables(seqs, remap, maxb):
    bt = np.full((len(seqs), maxb), -1, dtype=np.int32)
    for i, s in enumerate(seqs):
        if len(s.table) > maxb:
            raise ValueError("sequence longer than max_blocks_per_seq")
        bt[i, : len(s.table)] = [remap[b] for b in s.table]
    return bt


def _remap_slot(slot, remap, bs):
    return remap[slot // bs] * bs + slot % bs


def _materialise(b: _Builder, remap, nb, H, D, dtype, rng_k, rng_v):
    """Replay the builder's writes and copy-on-writes on a poisoned pool. The
    values of all written tokens are drawn in one go, in write order."""
    bs = b.bs
    kc = poison_array((nb, H, bs, D), dtype)
    vc = poison_array((nb, H, bs, D), dtype)
    n_written = sum(len(ev[1]) for ev in b.events if ev[0] == "write")
    kvals = normal(rng_k, (n_written, H, D), dtype)
    vvals = normal(rng_v, (n_written, H, D), dtype)
    pos = 0
    for ev in b.events:
        if ev[0] == "copy":
            s, d = remap[ev[1]], remap[ev[2]]
            kc[d] = kc[s]
            vc[d] = vc[s]
        else:
            slots = np.array([_remap_slot(x, remap, bs) for x in ev[1]], dtype=np.int64)
            blk, off = slots // bs, slots % bs
            n = len(slots)
            kc[blk, :, off, :] = kvals[pos:pos + n]
            vc[blk, :, off, :] = vvals[pos:pos + n]
            pos += n
    return kc, vc


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    names = ("lengths", "tables", "q", "kpool", "vpool", "newk", "newv")
    return {n: np.random.default_rng(c) for n, c in zip(names, ss.spawn(len(names)))}


def decode_workload(name, seed, dtype, H, D, bs, ctx, maxb, pool_blocks=None,
                    pool_factor=None, streams=None, scale=None) -> Workload:
    """Independent sequences of the given context lengths; each one's last
    token is new this step."""
    st = streams or _streams(seed)
    ctx = [int(c) for c in ctx]
    b = _Builder(bs)
    seqs, new_slots = [], []
    for c in ctx:
        s = b.alloc.new_sequence()
        if c > 0:
            b.append(s, c - 1)
            new_slots += b.append(s, 1, record=False)
        seqs.append(s)
    n_used = len({x for s in seqs for x in s.table})
    if pool_factor is not None:
        pool_blocks = int(math.ceil(pool_factor * n_used))
    nb, remap = b.place(seqs, pool_blocks, st["tables"])
    kc, vc = _materialise(b, remap, nb, H, D, dtype, st["kpool"], st["vpool"])
    S = len(ctx)
    T = len(new_slots)
    wl = Workload(
        name=name, seed=seed, dtype=dtype, num_heads=H, head_dim=D, block_size=bs,
        num_blocks=nb, max_blocks_per_seq=maxb,
        scale=float(1.0 / math.sqrt(D)) if scale is None else float(scale),
        k_cache=kc, v_cache=vc,
        new=NewTokens(k=normal(st["newk"], (T, H, D), dtype), v=normal(st["newv"], (T, H, D), dtype),
                      slot_mapping=np.array([_remap_slot(x, remap, bs) for x in new_slots], dtype=np.int32)),
        decode=DecodeBatch(q=normal(st["q"], (S, H, D), dtype), block_tables=_tables(seqs, remap, maxb),
                           context_lens=np.array(ctx, dtype=np.int32)),
    )
    return wl


def config1(seed=None) -> Workload:
    seed = BASE_SEED + 1 if seed is None else seed
    return decode_workload("tiny", seed, "f32", 2, 64, 16, [1, 17, 33, 100], maxb=7, pool_blocks=64)


def config2(seed=None, num_seqs=64, block_size=16) -> Workload:
    """LLaMA-7B layer decode; ``block_size`` other than 16 keeps the same
    lengths and values (for the block-size trade-off)."""
    seed = BASE_SEED + 2 if seed is None else seed
    st = _streams(seed)
    ctx = st["lengths"].integers(128, 2048, size=num_seqs, endpoint=True)
    return decode_workload("llama7b", seed, "f16", 32, 128, block_size, ctx, maxb=-(-2048 // block_size),
                           streams=st)


def lognormal_lengths(rng, n, mean=600.0, sigma=1.0, lo=1, hi=4096):
    mu = math.log(mean) - 0.5 * sigma * sigma
    x = np.rint(rng.lognormal(mu, sigma, size=n))
    return np.clip(x, lo, hi).astype(np.int64)


def config3(seed=None, num_seqs=256) -> Workload:
    seed = BASE_SEED + 3 if seed is None else seed
    st = _streams(seed)
    ctx = lognormal_lengths(st["lengths"], num_seqs)
    return decode_workload("mixed256", seed, "bf16", 32, 128, 32, ctx, maxb=128, pool_factor=1.25, streams=st)


def config4(seed=None, prompts=32, samples=8, prompt_len=1024, max_tail=256, cow=False,
            H=40, D=128, bs=16, dtype="f16") -> Workload:
    """Parallel sampling: each prompt's blocks are shared by its samples."""
    seed = BASE_SEED + 4 if seed is None else seed
    st = _streams(seed)
    rl = st["lengths"]
    plens = [prompt_len - (int(rl.integers(1, 15, endpoint=True)) if cow else 0) for _ in range(prompts)]
    tails = rl.integers(0, max_tail, size=(prompts, samples), endpoint=True)
    b = _Builder(bs)
    seqs, new_slots = [], []
    for p in range(prompts):
        parent = b.alloc.new_sequence()
        b.append(parent, plens[p])
        group = [parent] + [b.alloc.fork(parent) for _ in range(samples - 1)]
        for i, s in enumerate(group):
            t = int(tails[p, i])
            if t > 0:
                b.append(s, t - 1)
                new_slots += b.append(s, 1, record=False)
            else:
                new_slots.append(-1)  # last token sits in a shared block: already cached
            seqs.append(s)
    maxb = int(math.ceil((prompt_len + max_tail) / bs))
    nb, remap = b.place(seqs, None, st["tables"])
    kc, vc = _materialise(b, remap, nb, H, D, dtype, st["kpool"], st["vpool"])
    S = len(seqs)
    T = len(new_slots)
    refs = np.zeros(nb, dtype=np.int64)
    for s in seqs:
        for x in s.table:
            refs[remap[x]] += 1
    wl = Workload(
        name="prefix13b" + ("_cow" if cow else ""), seed=seed, dtype=dtype, num_heads=H, head_dim=D,
        block_size=bs, num_blocks=nb, max_blocks_per_seq=maxb, scale=1.0 / math.sqrt(D),
        k_cache=kc, v_cache=vc,
        new=NewTokens(k=normal(st["newk"], (T, H, D), dtype), v=normal(st["newv"], (T, H, D), dtype),
                      slot_mapping=np.array([-1 if x < 0 else _remap_slot(x, remap, bs) for x in new_slots],
                                            dtype=np.int32)),
        decode=DecodeBatch(q=normal(st["q"], (S, H, D), dtype), block_tables=_tables(seqs, remap, maxb),
                           context_lens=np.array([s.length for s in seqs], dtype=np.int32)),
        notes={"prompt_lens": plens, "tails": tails.tolist(), "refcount": refs,
               "cow_copies": sum(1 for e in b.events if e[0] == "copy")},
    )
    return wl


def config5(seed=None, H=40, D=128, bs=16, dtype="f16", budget=2048, chunks=4, decodes=96,
            chunk_len=(256, 512), prior=(0, 1024), dec_ctx=(256, 4096), maxb=256) -> Workload:
    """One mixed step under a 2048-token budget: prefill chunks + decodes +
    filler rows, all written by one reshape_and_cache."""
    seed = BASE_SEED + 5 if seed is None else seed
    st = _streams(seed)
    rl = st["lengths"]
    while True:
        L = rl.integers(chunk_len[0], chunk_len[1], size=chunks, endpoint=True)
        c = rl.integers(prior[0], prior[1], size=chunks, endpoint=True)
        dctx = rl.integers(dec_ctx[0], dec_ctx[1], size=decodes, endpoint=True)
        if int(L.sum()) + decodes <= budget:
            break
    n_fill = budget - int(L.sum()) - decodes
    b = _Builder(bs)
    pf_seqs, dec_seqs, chunk_slots, dec_slots = [], [], [], []
    for i in range(chunks):
        s = b.alloc.new_sequence()
        b.append(s, int(c[i]))
        chunk_slots += b.append(s, int(L[i]), record=False)
        pf_seqs.append(s)
    for j in range(decodes):
        s = b.alloc.new_sequence()
        b.append(s, int(dctx[j]) - 1)
        dec_slots += b.append(s, 1, record=False)
        dec_seqs.append(s)
    extra = int(math.ceil(n_fill / bs))
    nb, remap = b.place(pf_seqs + dec_seqs, None, st["tables"], extra_blocks=extra)
    kc, vc = _materialise(b, remap, nb, H, D, dtype, st["kpool"], st["vpool"])
    # filler rows: distinct slots that no sequence references
    referenced = np.zeros(nb * bs, dtype=bool)
    for s in pf_seqs + dec_seqs:
        for t in range(s.length):
            referenced[remap[s.table[t // bs]] * bs + t % bs] = True
    free_slots = np.flatnonzero(~referenced)
    fill = st["tables"].choice(free_slots, size=n_fill, replace=False) if n_fill else np.zeros(0, np.int64)
    slots = [_remap_slot(x, remap, bs) for x in chunk_slots + dec_slots] + [int(x) for x in fill]
    T = len(slots)
    qsl = np.zeros(chunks + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(L)
    wl = Workload(
        name="mixed_step", seed=seed, dtype=dtype, num_heads=H, head_dim=D, block_size=bs,
        num_blocks=nb, max_blocks_per_seq=maxb, scale=1.0 / math.sqrt(D),
        k_cache=kc, v_cache=vc,
        new=NewTokens(k=normal(st["newk"], (T, H, D), dtype), v=normal(st["newv"], (T, H, D), dtype),
                      slot_mapping=np.array(slots, dtype=np.int32)),
        prefill=PrefillBatch(q=normal(st["q"], (int(L.sum()), H, D), dtype),
                             block_tables=_tables(pf_seqs, remap, maxb),
                             context_lens=np.array([s.length for s in pf_seqs], dtype=np.int32),
                             query_start_loc=qsl),
        decode=DecodeBatch(q=normal(st["q"], (decodes, H, D), dtype), block_tables=_tables(dec_seqs, remap, maxb),
                           context_lens=np.array([s.length for s in dec_seqs], dtype=np.int32)),
        notes={"chunk_L": L.tolist(), "chunk_prior": c.tolist(), "n_fill": n_fill},
    )
    return wl


def prefill_workload(name, seed, dtype, H, D, bs, prior, chunk, maxb, pool_factor=None, scale=None) -> Workload:
    """Chunks of ``chunk[i]`` new tokens after ``prior[i]`` cached ones."""
    st = _streams(seed)
    b = _Builder(bs)
    seqs, slots = [], []
    for c, L in zip(prior, chunk):
        s = b.alloc.new_sequence()
        b.append(s, int(c))
        slots += b.append(s, int(L), record=False)
        seqs.append(s)
    n_used = len({x for s in seqs for x in s.table})
    pool_blocks = None if pool_factor is None else int(math.ceil(pool_factor * n_used))
    nb, remap = b.place(seqs, pool_blocks, st["tables"])
    kc, vc = _materialise(b, remap, nb, H, D, dtype, st["kpool"], st["vpool"])
    T = len(slots)
    qsl = np.zeros(len(seqs) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(np.asarray(chunk, dtype=np.int64))
    return Workload(
        name=name, seed=seed, dtype=dtype, num_heads=H, head_dim=D, block_size=bs, num_blocks=nb,
        max_blocks_per_seq=maxb, scale=float(1.0 / math.sqrt(D)) if scale is None else float(scale),
        k_cache=kc, v_cache=vc,
        new=NewTokens(k=normal(st["newk"], (T, H, D), dtype), v=normal(st["newv"], (T, H, D), dtype),
                      slot_mapping=np.array([_remap_slot(x, remap, bs) for x in slots], dtype=np.int32)),
        prefill=PrefillBatch(q=normal(st["q"], (T, H, D), dtype), block_tables=_tables(seqs, remap, maxb),
                             context_lens=np.array([s.length for s in seqs], dtype=np.int32),
                             query_start_loc=qsl),
    )


def make_config(cid: int, **kw) -> Workload:
    return {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}[cid](**kw)


# ---------------------------------------------------------------------------
# accounting helpers (memory-utilisation arithmetic the pages print)


def contiguous_utilisation(lengths, reserve=None) -> float:
    """Fraction of reserved slots used when every sequence reserves
    ``reserve`` contiguous slots (default: the longest length)."""
    lengths = [int(x) for x in lengths]
    r = max(lengths) if reserve is None else int(reserve)
    return sum(lengths) / (r * len(lengths))


def paged_slots(lengths, block_size) -> int:
    return sum(int(math.ceil(int(x) / block_size)) * block_size for x in lengths)


def paged_utilisation(lengths, block_size) -> float:
    return sum(int(x) for x in lengths) / paged_slots(lengths, block_size)
