"""Paged-KV attention for MI355X (gfx950): Python binding of libpagedattn.

Argument marshalling only: every step runs in the HIP kernels of
``libpagedattn.so`` (built in-tree by ``build.py``). torch supplies device
memory and the current HIP stream. Nothing here falls back to the CPU; a
missing library raises.

Calls mirror the C ABI in ``include/pagedattn.h``:

* ``reshape_and_cache(k, v, k_cache, v_cache, slot_mapping)``
* ``copy_blocks(k_cache, v_cache, block_mapping)`` and ``BlockAllocator``
  (host block manager: on-demand blocks, fork with reference counts,
  copy-on-write, free)
* ``paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, ...)``
* ``paged_attention_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, ...)``
* ``gather_kv(...)``, ``decode_workspace_bytes(...)`` and the two decode stages.
* ``attention_step(...)``: one scheduler iteration (cache write, prefill,
  decode) in one call, the prefill optionally on a side stream.

Caches are ``[num_blocks, num_heads, block_size, head_dim]``; block tables
``int32 [num_seqs, max_blocks_per_seq]``; slots ``block * block_size + offset``.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = 0, -1, -2, -3, -4
PA_ERR_NO_BLOCKS, PA_ERR_NO_MEMORY, PA_ERR_PENDING_WRITES, PA_ERR_SCRATCH_LIMIT = -5, -6, -7, -8
_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_lib = None

_P, _I = ctypes.c_void_p, ctypes.c_int32


class StepArgs(ctypes.Structure):
    """Mirror of ``pa_step_args`` (C layout; checked against the header by
    the tests)."""
    _fields_ = [("k_cache", _P), ("v_cache", _P), ("num_blocks", _I), ("num_heads", _I), ("head_dim", _I),
                ("block_size", _I), ("dtype", ctypes.c_int), ("scale", ctypes.c_float), ("new_k", _P),
                ("new_v", _P), ("slot_mapping", _P), ("num_new_tokens", _I), ("prefill_out", _P),
                ("prefill_out_dtype", ctypes.c_int), ("prefill_q", _P), ("prefill_block_tables", _P),
                ("prefill_context_lens", _P), ("prefill_query_start_loc", _P), ("num_prefill_seqs", _I),
                ("prefill_total_q", _I), ("prefill_max_q_len", _I), ("prefill_max_blocks_per_seq", _I),
                ("prefill_max_context_len", _I), ("decode_out", _P), ("decode_out_dtype", ctypes.c_int),
                ("decode_q", _P), ("decode_block_tables", _P), ("decode_context_lens", _P), ("num_decode_seqs", _I),
                ("decode_max_blocks_per_seq", _I), ("decode_max_context_len", _I), ("workspace", _P),
                ("workspace_bytes", ctypes.c_size_t)]


class PagedAttnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with paged_kv_cache_391_amd.build "
                               "(or __graft_entry__.build()) before use")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        L.pa_status_string.argtypes = [ctypes.c_int]
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_reshape_and_cache.argtypes = [P, P, P, P, P, I, I, I, I, I, ctypes.c_int, P]
        L.pa_gather_kv.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, ctypes.c_int, P]
        L.pa_decode_partition_tokens.argtypes = []
        L.pa_decode_partition_tokens.restype = I
        L.pa_decode_workspace_bytes.argtypes = [I, I, I, I]
        L.pa_decode_workspace_bytes.restype = Z
        dec = [P, ctypes.c_int, P, P, P, P, P, I, I, I, I, I, I, I, I, F, ctypes.c_int, P, Z, P]
        L.pa_paged_attention_decode.argtypes = dec
        L.pa_paged_attention_decode_partitions.argtypes = dec
        L.pa_paged_attention_decode_with_cache_write.argtypes = dec[:5] + [P, P, P] + dec[5:]
        L.pa_paged_attention_decode_with_cache_write_partitions.argtypes = dec[:5] + [P, P, P] + dec[5:]
        L.pa_paged_attention_decode_with_cache_write_reduce.argtypes = dec[:5] + [P, P, P] + dec[5:]
        L.pa_paged_attention_decode_noalloc.argtypes = dec[:17] + [P]
        L.pa_paged_attention_decode_noalloc.restype = ctypes.c_int
        L.pa_decode_noalloc_scratch_bytes.argtypes = []
        L.pa_decode_noalloc_scratch_bytes.restype = Z
        L.pa_paged_attention_decode_reduce.argtypes = [P, ctypes.c_int, P, I, I, I, I, ctypes.c_int, P, Z, P]
        L.pa_paged_attention_prefill.argtypes = [P, ctypes.c_int, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, F,
                                                 ctypes.c_int, P]
        L.pa_copy_blocks.argtypes = [P, P, P, I, I, I, I, I, ctypes.c_int, P]
        L.pa_attention_step.argtypes = [ctypes.POINTER(StepArgs), P, P, P, P]
        L.pa_attention_step.restype = ctypes.c_int
        L.pa_decode_shared_workspace_bytes.argtypes = [I, I, I, I]
        L.pa_decode_shared_workspace_bytes.restype = Z
        L.pa_paged_attention_decode_shared_prefix.argtypes = [P, ctypes.c_int, P, P, P, P, P, P, P, I, I, I, I, I, I,
                                                              I, I, I, I, I, F, ctypes.c_int, P, Z, P]
        L.pa_paged_attention_decode_shared_prefix.restype = ctypes.c_int
        PI = ctypes.POINTER(ctypes.c_int32)
        L.pa_allocator_create.argtypes = [I, I, ctypes.POINTER(P)]
        L.pa_allocator_destroy.argtypes = [P]
        L.pa_allocator_destroy.restype = None
        L.pa_allocator_num_free.argtypes = [P]
        L.pa_allocator_refcount.argtypes = [P, I]
        L.pa_allocator_new_sequence.argtypes = [P, PI]
        L.pa_allocator_fork.argtypes = [P, I, PI]
        L.pa_allocator_append.argtypes = [P, I, I, P]
        L.pa_allocator_free_sequence.argtypes = [P, I]
        L.pa_allocator_sequence_length.argtypes = [P, I]
        L.pa_allocator_block_table.argtypes = [P, I, P, I, PI]
        L.pa_allocator_take_copies.argtypes = [P, P, I, PI]
        for name in ("pa_allocator_num_free", "pa_allocator_refcount", "pa_allocator_sequence_length"):
            getattr(L, name).restype = I
        for name in ("pa_copy_blocks", "pa_allocator_create", "pa_allocator_new_sequence", "pa_allocator_fork",
                     "pa_allocator_append", "pa_allocator_free_sequence", "pa_allocator_block_table",
                     "pa_allocator_take_copies"):
            getattr(L, name).restype = ctypes.c_int
        for name in ("pa_reshape_and_cache", "pa_gather_kv", "pa_paged_attention_decode",
                     "pa_paged_attention_decode_with_cache_write",
                     "pa_paged_attention_decode_with_cache_write_partitions",
                     "pa_paged_attention_decode_with_cache_write_reduce",
                     "pa_paged_attention_decode_partitions", "pa_paged_attention_decode_reduce",
                     "pa_paged_attention_prefill"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn, status):
    if status != PA_OK:
        raise PagedAttnError(fn, status, lib().pa_status_string(status).decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _i32(*ts):
    for t in ts:
        if t.dtype != torch.int32:
            raise ValueError("index tensors must be int32")


def _cache_dims(k_cache, v_cache):
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype or k_cache.dim() != 4:
        raise ValueError("k_cache and v_cache must both be [num_blocks, num_heads, block_size, head_dim]")
    return tuple(int(x) for x in k_cache.shape)


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping):
    """Write rows ``k[n], v[n]`` ([T, H, D]) into slot ``slot_mapping[n]``
    (skipped when negative)."""
    _dev(k, v, k_cache, v_cache, slot_mapping)
    _i32(slot_mapping)
    nb, H, bs, D = _cache_dims(k_cache, v_cache)
    T = int(slot_mapping.shape[0])
    if k.shape != (T, H, D) or v.shape != (T, H, D) or k.dtype != k_cache.dtype or v.dtype != k_cache.dtype:
        raise ValueError("k and v must be [num_tokens, num_heads, head_dim] in the cache dtype")
    _check("reshape_and_cache", lib().pa_reshape_and_cache(
        _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, H, D, bs, nb,
        _DT[k_cache.dtype], _stream()))


def copy_blocks(k_cache, v_cache, block_mapping):
    """Copy-on-write: block ``block_mapping[i, 1]`` of both caches becomes a
    copy of block ``block_mapping[i, 0]`` (int32 ``[pairs, 2]`` on the GPU)."""
    _dev(k_cache, v_cache, block_mapping)
    _i32(block_mapping)
    nb, H, bs, D = _cache_dims(k_cache, v_cache)
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [num_pairs, 2]")
    _check("copy_blocks", lib().pa_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_mapping), int(block_mapping.shape[0]), H, D, bs, nb,
        _DT[k_cache.dtype], _stream()))


class BlockAllocator:
    """Host block manager of the library (``pa_allocator_*``): blocks on
    demand, forks sharing blocks with reference counts, copy-on-write of a
    shared partly filled last block, release on free. Sequence ids are ints."""

    def __init__(self, num_blocks: int, block_size: int):
        h = ctypes.c_void_p()
        _check("allocator_create", lib().pa_allocator_create(int(num_blocks), int(block_size), ctypes.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if self._h:
            lib().pa_allocator_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return int(lib().pa_allocator_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(lib().pa_allocator_refcount(self._h, int(block)))

    def new_sequence(self) -> int:
        sid = ctypes.c_int32()
        _check("allocator_new_sequence", lib().pa_allocator_new_sequence(self._h, ctypes.byref(sid)))
        return sid.value

    def fork(self, parent: int) -> int:
        sid = ctypes.c_int32()
        _check("allocator_fork", lib().pa_allocator_fork(self._h, int(parent), ctypes.byref(sid)))
        return sid.value

    def append(self, seq: int, num_tokens: int):
        """Slots (``block * block_size + offset``) of ``num_tokens`` new
        tokens at the end of ``seq``, as an int32 numpy array."""
        import numpy as np
        slots = np.zeros(max(0, int(num_tokens)), dtype=np.int32)
        _check("allocator_append", lib().pa_allocator_append(self._h, int(seq), int(num_tokens),
                                                                slots.ctypes.data_as(ctypes.c_void_p)))
        return slots

    def free(self, seq: int) -> None:
        _check("allocator_free_sequence", lib().pa_allocator_free_sequence(self._h, int(seq)))

    def length(self, seq: int) -> int:
        return int(lib().pa_allocator_sequence_length(self._h, int(seq)))

    def block_table(self, seq: int):
        import numpy as np
        n = ctypes.c_int32()
        _check("allocator_block_table", lib().pa_allocator_block_table(self._h, int(seq), None, 0, ctypes.byref(n)))
        t = np.zeros(n.value, dtype=np.int32)
        if n.value:
            _check("allocator_block_table", lib().pa_allocator_block_table(
                self._h, int(seq), t.ctypes.data_as(ctypes.c_void_p), n.value, ctypes.byref(n)))
        return t

    def take_copies(self):
        """Pending copy-on-write (src, dst) block pairs, oldest first, as an
        int32 ``[n, 2]`` numpy array; the queue is emptied and the open batch
        closed (queue these copies, then the batch's cache writes)."""
        import numpy as np
        n = ctypes.c_int32()
        _check("allocator_take_copies", lib().pa_allocator_take_copies(self._h, None, 0, ctypes.byref(n)))
        buf = np.zeros((max(1, n.value), 2), dtype=np.int32)  # capacity > 0 closes the batch
        _check("allocator_take_copies", lib().pa_allocator_take_copies(
            self._h, buf.ctypes.data_as(ctypes.c_void_p), buf.shape[0], ctypes.byref(n)))
        return buf[:n.value].copy()


def gather_kv(k_out, v_out, k_cache, v_cache, block_tables, context_lens, cu_context_lens, max_context_len: int):
    """Copy each sequence's logical K/V to rows ``cu_context_lens[s] + t``."""
    _dev(k_out, v_out, k_cache, v_cache, block_tables, context_lens, cu_context_lens)
    _i32(block_tables, context_lens, cu_context_lens)
    nb, H, bs, D = _cache_dims(k_cache, v_cache)
    S = int(context_lens.shape[0])
    _check("gather_kv", lib().pa_gather_kv(
        _ptr(k_out), _ptr(v_out), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(cu_context_lens), S, int(max_context_len), H, D, bs, nb, int(block_tables.shape[1]),
        _DT[k_cache.dtype], _stream()))


def decode_partition_tokens() -> int:
    return int(lib().pa_decode_partition_tokens())


def decode_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int) -> int:
    return int(lib().pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len))


def make_decode_workspace(num_seqs, num_heads, head_dim, max_context_len, device="cuda"):
    """A split-K workspace of the size the library asks for (None if not needed)."""
    n = decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len)
    return None if n == 0 else torch.empty(n // 4, dtype=torch.float32, device=device)


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, workspace):
    _dev(out, q, k_cache, v_cache, block_tables, context_lens, workspace)
    _i32(block_tables, context_lens)
    nb, H, bs, D = _cache_dims(k_cache, v_cache)
    S = int(context_lens.shape[0])
    if q.shape != (S, H, D) or q.dtype != k_cache.dtype:
        raise ValueError("q must be [num_seqs, num_heads, head_dim] in the cache dtype")
    if out.shape != (S, H, D) or out.dtype not in (torch.float32, q.dtype):
        raise ValueError("out must be [num_seqs, num_heads, head_dim], float32 or the input dtype")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if S else 0  # synchronises
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(out), _DT[out.dtype], _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), S, H, H, D, bs, nb, int(block_tables.shape[1]), int(max_context_len),
            float(scale), _DT[q.dtype], _ptr(workspace), ws_bytes, _stream())


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                           max_context_len: int | None = None, workspace=None):
    """Decode attention of ``q[s]`` over the ``context_lens[s]`` cached tokens
    of sequence ``s``. ``workspace`` (see ``make_decode_workspace``) enables
    split-K over long contexts. Pass ``max_context_len`` to avoid a sync."""
    _check("paged_attention_decode", lib().pa_paged_attention_decode(
        *_decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, workspace)))


def paged_attention_decode_with_cache_write(out, q, k_cache, v_cache, new_k, new_v, slot_mapping, block_tables,
                                            context_lens, scale: float, max_context_len: int | None = None,
                                            workspace=None):
    """One decode step in one launch: ``reshape_and_cache(new_k, new_v,
    k_cache, v_cache, slot_mapping)`` (one new token per sequence, at
    position ``context_lens[s] - 1``) followed by ``paged_attention_decode``,
    with the same outputs and caches bit for bit."""
    args = _decode_with_cache_write_args(out, q, k_cache, v_cache, new_k, new_v, slot_mapping, block_tables,
                                         context_lens, scale, max_context_len, workspace)
    _check("paged_attention_decode_with_cache_write", lib().pa_paged_attention_decode_with_cache_write(*args))


def paged_attention_decode_with_cache_write_partitions(out, q, k_cache, v_cache, new_k, new_v, slot_mapping,
                                                       block_tables, context_lens, scale: float,
                                                       max_context_len: int, workspace=None):
    """First stage of ``paged_attention_decode_with_cache_write`` (the
    partition kernel, which uses the new tokens);
    ``paged_attention_decode_with_cache_write_reduce`` is the second."""
    args = _decode_with_cache_write_args(out, q, k_cache, v_cache, new_k, new_v, slot_mapping, block_tables,
                                         context_lens, scale, max_context_len, workspace)
    _check("paged_attention_decode_with_cache_write_partitions",
           lib().pa_paged_attention_decode_with_cache_write_partitions(*args))


def paged_attention_decode_with_cache_write_reduce(out, q, k_cache, v_cache, new_k, new_v, slot_mapping,
                                                   block_tables, context_lens, scale: float, max_context_len: int,
                                                   workspace=None):
    """Second stage of ``paged_attention_decode_with_cache_write`` (the
    reduction, which also writes the new tokens into their slots; nothing
    when the call is not split). Same arguments as the first stage."""
    args = _decode_with_cache_write_args(out, q, k_cache, v_cache, new_k, new_v, slot_mapping, block_tables,
                                         context_lens, scale, max_context_len, workspace)
    _check("paged_attention_decode_with_cache_write_reduce",
           lib().pa_paged_attention_decode_with_cache_write_reduce(*args))


def _decode_with_cache_write_args(out, q, k_cache, v_cache, new_k, new_v, slot_mapping, block_tables, context_lens,
                                  scale, max_context_len, workspace):
    _dev(new_k, new_v, slot_mapping)
    _i32(slot_mapping)
    S = int(context_lens.shape[0])
    if (new_k.shape != q.shape or new_v.shape != q.shape or new_k.dtype != k_cache.dtype
            or new_v.dtype != k_cache.dtype or tuple(slot_mapping.shape) != (S,)):
        raise ValueError("new_k and new_v must be [num_seqs, num_heads, head_dim] in the cache dtype, "
                         "slot_mapping [num_seqs]")
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, workspace)
    return (*args[:5], _ptr(new_k), _ptr(new_v), _ptr(slot_mapping), *args[5:])


def decode_noalloc_scratch_bytes() -> int:
    """Size of the split-K scratch built into the library (per device)."""
    return int(lib().pa_decode_noalloc_scratch_bytes())


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                                   max_context_len: int | None = None):
    """``paged_attention_decode`` with split-K on and its partials in the
    library's built-in scratch: the call allocates nothing. Calls that may
    overlap on one device race (they share the scratch)."""
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, None)
    _check("paged_attention_decode_noalloc", lib().pa_paged_attention_decode_noalloc(*args[:17], args[19]))


def decode_shared_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int) -> int:
    return int(lib().pa_decode_shared_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len))


def make_decode_shared_workspace(num_seqs, num_heads, head_dim, max_context_len, device="cuda"):
    n = decode_shared_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len)
    return torch.empty(max(1, n // 4), dtype=torch.float32, device=device)


def check_shared_prefix_groups(block_tables, context_lens, group_starts, prefix_lens, block_size: int):
    """The shared-prefix call's data preconditions, checked on host copies
    (this reads device memory, so it synchronises: for tests and debugging,
    not the serving path). Raises ValueError naming the first broken one."""
    gs = group_starts.cpu().numpy()
    pl = prefix_lens.cpu().numpy()
    ctx = context_lens.cpu().numpy()
    bt = block_tables.cpu().numpy()
    S = ctx.shape[0]
    if gs[0] != 0 or gs[-1] != S or (gs[1:] < gs[:-1]).any():
        raise ValueError("group_starts must rise from 0 to num_seqs")
    for g in range(pl.shape[0]):
        rows = slice(int(gs[g]), int(gs[g + 1]))
        p = int(pl[g])
        if p < 0 or p % block_size:
            raise ValueError(f"prefix_lens[{g}] = {p} is not a non-negative multiple of block_size")
        if gs[g + 1] > gs[g]:
            if p > int(ctx[rows].min()):
                raise ValueError(f"prefix_lens[{g}] = {p} exceeds a member's context length")
            nb = p // block_size
            if nb and (bt[rows, :nb] != bt[int(gs[g]), :nb]).any():
                raise ValueError(f"group {g}'s members do not share the prefix's blocks")


def paged_attention_decode_shared_prefix(out, q, k_cache, v_cache, block_tables, context_lens, group_starts,
                                         prefix_lens, scale: float, max_context_len: int, max_group_size: int,
                                         max_prefix_len: int, workspace, validate: bool = False):
    """Decode where the rows ``group_starts[g]:group_starts[g+1]`` share their
    first ``prefix_lens[g]`` tokens through aliased blocks; each shared tile is
    read once per group. Same result as ``paged_attention_decode``.
    ``validate=True`` first checks the groups' data preconditions on the host
    (``check_shared_prefix_groups``; synchronises)."""
    _dev(group_starts, prefix_lens)
    _i32(group_starts, prefix_lens)
    G = int(prefix_lens.shape[0])
    if group_starts.shape != (G + 1,):
        raise ValueError("group_starts must be [num_groups + 1]")
    if validate:
        check_shared_prefix_groups(block_tables, context_lens, group_starts, prefix_lens, int(k_cache.shape[2]))
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, workspace)
    # (out, odt, q, kc, vc, bt, ctx, S, H, KVH, D, bs, nb, maxb, maxctx, scale, dt, ws, wsb, stream)
    _check("paged_attention_decode_shared_prefix", lib().pa_paged_attention_decode_shared_prefix(
        *args[:7], _ptr(group_starts), _ptr(prefix_lens), G, int(max_group_size), int(max_prefix_len), *args[7:]))


def paged_attention_decode_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                                      max_context_len: int, workspace=None):
    """First stage of the decode call (partition kernel only)."""
    _check("paged_attention_decode_partitions", lib().pa_paged_attention_decode_partitions(
        *_decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, workspace)))


def paged_attention_decode_reduce(out, context_lens, head_dim: int, max_context_len: int, in_dtype, workspace):
    """Second stage of the decode call (merges split-K partials)."""
    _dev(out, context_lens, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("paged_attention_decode_reduce", lib().pa_paged_attention_decode_reduce(
        _ptr(out), _DT[out.dtype], _ptr(context_lens), int(context_lens.shape[0]), int(out.shape[1]),
        int(head_dim), int(max_context_len), _DT[in_dtype], _ptr(workspace), ws_bytes, _stream()))


def make_step_events(n=2):
    """Events for the fork/join of ``attention_step`` (created on the device:
    a torch event gets its handle on its first record)."""
    evs = [torch.cuda.Event() for _ in range(n)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    return evs


def attention_step(k_cache, v_cache, scale: float, new_k=None, new_v=None, slot_mapping=None, prefill_out=None,
                   prefill_q=None, prefill_block_tables=None, prefill_context_lens=None,
                   prefill_query_start_loc=None, prefill_max_q_len=None, prefill_max_context_len=None,
                   decode_out=None, decode_q=None, decode_block_tables=None, decode_context_lens=None,
                   decode_max_context_len=None, workspace=None, side_stream=None, fork_event=None,
                   join_event=None):
    """One scheduler iteration: cache write of the new tokens, causal
    prefill of the chunks and split-K decode, against the same cache. With
    ``side_stream`` (and two events from ``make_step_events``) the prefill
    runs on it concurrently with the decode on the current stream."""
    nb, H, bs, D = _cache_dims(k_cache, v_cache)
    a = StepArgs()
    a.k_cache, a.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
    a.num_blocks, a.num_heads, a.head_dim, a.block_size = nb, H, D, bs
    a.dtype, a.scale = _DT[k_cache.dtype], float(scale)
    _dev(k_cache, v_cache)
    if slot_mapping is not None:
        _dev(new_k, new_v, slot_mapping)
        _i32(slot_mapping)
        T = int(slot_mapping.shape[0])
        if new_k.shape != (T, H, D) or new_v.shape != (T, H, D) or new_k.dtype != k_cache.dtype:
            raise ValueError("new_k/new_v must be [num_tokens, num_heads, head_dim] in the cache dtype")
        a.new_k, a.new_v, a.slot_mapping, a.num_new_tokens = new_k.data_ptr(), new_v.data_ptr(), \
            slot_mapping.data_ptr(), T
    if prefill_q is not None:
        _dev(prefill_out, prefill_q, prefill_block_tables, prefill_context_lens, prefill_query_start_loc)
        _i32(prefill_block_tables, prefill_context_lens, prefill_query_start_loc)
        S = int(prefill_context_lens.shape[0])
        TQ = int(prefill_q.shape[0])
        if prefill_q.shape != (TQ, H, D) or prefill_out.shape != (TQ, H, D) or prefill_q.dtype != k_cache.dtype:
            raise ValueError("prefill q/out must be [total_q, num_heads, head_dim]")
        if prefill_query_start_loc.shape != (S + 1,):
            raise ValueError("prefill_query_start_loc must be [num_seqs + 1]")
        a.prefill_out, a.prefill_out_dtype, a.prefill_q = prefill_out.data_ptr(), _DT[prefill_out.dtype], \
            prefill_q.data_ptr()
        a.prefill_block_tables, a.prefill_context_lens = prefill_block_tables.data_ptr(), \
            prefill_context_lens.data_ptr()
        a.prefill_query_start_loc = prefill_query_start_loc.data_ptr()
        a.num_prefill_seqs, a.prefill_total_q = S, TQ
        a.prefill_max_q_len, a.prefill_max_context_len = int(prefill_max_q_len), int(prefill_max_context_len)
        a.prefill_max_blocks_per_seq = int(prefill_block_tables.shape[1])
    if decode_q is not None:
        _dev(decode_out, decode_q, decode_block_tables, decode_context_lens, workspace)
        _i32(decode_block_tables, decode_context_lens)
        S = int(decode_context_lens.shape[0])
        if decode_q.shape != (S, H, D) or decode_out.shape != (S, H, D) or decode_q.dtype != k_cache.dtype:
            raise ValueError("decode q/out must be [num_seqs, num_heads, head_dim]")
        a.decode_out, a.decode_out_dtype, a.decode_q = decode_out.data_ptr(), _DT[decode_out.dtype], \
            decode_q.data_ptr()
        a.decode_block_tables, a.decode_context_lens = decode_block_tables.data_ptr(), decode_context_lens.data_ptr()
        a.num_decode_seqs, a.decode_max_context_len = S, int(decode_max_context_len)
        a.decode_max_blocks_per_seq = int(decode_block_tables.shape[1])
        if workspace is not None:
            a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    side = ctypes.c_void_p(side_stream.cuda_stream) if side_stream is not None else ctypes.c_void_p(0)
    if side_stream is not None and (fork_event is None or join_event is None or not fork_event.cuda_event
                                    or not join_event.cuda_event):
        raise ValueError("a side stream needs two created events (see make_step_events)")
    fe = ctypes.c_void_p(fork_event.cuda_event if fork_event is not None else 0)
    je = ctypes.c_void_p(join_event.cuda_event if join_event is not None else 0)
    _check("attention_step", lib().pa_attention_step(ctypes.byref(a), _stream(), side, fe, je))


def paged_attention_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale: float,
                            max_q_len: int | None = None, max_context_len: int | None = None):
    """Causal attention of query chunks: chunk ``s`` is rows
    ``query_start_loc[s]:query_start_loc[s+1]`` and the last L_s tokens of
    its ``context_lens[s]``-token context. ``max_q_len`` and
    ``max_context_len`` left as None are read from the device tensors, which
    waits for the stream; pass them to keep the call asynchronous."""
    _dev(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc)
    _i32(block_tables, context_lens, query_start_loc)
    nb, H, bs, D = _cache_dims(k_cache, v_cache)
    S = int(context_lens.shape[0])
    TQ = int(q.shape[0])
    if q.shape != (TQ, H, D) or q.dtype != k_cache.dtype:
        raise ValueError("q must be [total_q, num_heads, head_dim] in the cache dtype")
    if out.shape != (TQ, H, D) or out.dtype not in (torch.float32, q.dtype):
        raise ValueError("out must be [total_q, num_heads, head_dim], float32 or the input dtype")
    if query_start_loc.shape != (S + 1,):
        raise ValueError("query_start_loc must be [num_seqs + 1]")
    if max_q_len is None:
        max_q_len = int((query_start_loc[1:] - query_start_loc[:-1]).max().item()) if S else 0  # synchronises
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if S else 0  # synchronises
    _check("paged_attention_prefill", lib().pa_paged_attention_prefill(
        _ptr(out), _DT[out.dtype], _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(query_start_loc), S, TQ, int(max_q_len), H, H, D, bs, nb, int(block_tables.shape[1]),
        int(max_context_len), float(scale), _DT[q.dtype], _stream()))
