"""fp64 CPU oracle for paged-KV attention -- TEST INFRASTRUCTURE ONLY.

Python face of ``pagedattn_oracle.c``. Only the tests, the smoke check and the
benchmark's CPU-baseline leg use this module; the HIP library never does.
Inputs are the numpy arrays built by ``workloads``; outputs are float64.

* ``reshape_and_cache``: bit copy of new K/V rows into their slots.
* ``copy_blocks``: bit copy of whole blocks (copy-on-write of shared blocks).
* ``gather_kv``: raw copy of each sequence's logical K/V through its table.
* ``decode``: one query per sequence over its ctx cached tokens.
* ``prefill``: causal query chunks, bottom-right aligned (the chunk is the
  last L of ctx tokens).

Every function is pinned by CPU tests against brute force, closed forms,
library routines and invariants; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_DT = {"f32": 0, "f16": 1, "bf16": 2}
_ERR = {-1: "bad argument", -2: "slot out of range", -3: "duplicate slot", -4: "block id out of range",
        -5: "bad context length", -6: "out of memory"}
_lib = None


class OracleError(RuntimeError):
    pass


def _open(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_widen.argtypes = [P, P, ctypes.c_int64, I]
    lib.oracle_reshape_and_cache.argtypes = [P, P, P, P, P, I, I, I, I, I, I]
    lib.oracle_copy_blocks.argtypes = [P, P, P, I, I, I, I, I, I]
    lib.oracle_gather_kv.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I]
    lib.oracle_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, ctypes.c_double, I, P, I, I]
    lib.oracle_prefill.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, ctypes.c_double, I, P, I, I]
    for f in (lib.oracle_widen, lib.oracle_reshape_and_cache, lib.oracle_copy_blocks, lib.oracle_gather_kv,
              lib.oracle_decode, lib.oracle_prefill):
        f.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        _lib = _open(_build.LIB)
    return _lib


def use_library(path: str | None):
    """Point this module at another build of the oracle source (the tests use
    it to run the pins against deliberately broken copies). ``None`` returns
    to the normal build."""
    global _lib
    _lib = None if path is None else _open(path)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise OracleError(_ERR.get(rc, f"error {rc}"))


def _c(a, dtype=None):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of every storage element."""
    a = _c(a)
    out = np.empty(a.shape, dtype=np.float64)
    _check(_load().oracle_widen(_p(out), _p(a), a.size, _DT[dtype]))
    return out


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, block_size: int, dtype: str):
    """Return copies of the caches with the new rows written."""
    kc, vc = k_cache.copy(), v_cache.copy()
    k, v, sm = _c(k), _c(v), _c(slot_mapping, np.int32)
    T = sm.shape[0]
    nb, H, bs, D = kc.shape
    assert bs == block_size and k.shape == (T, H, D) and v.shape == (T, H, D)
    _check(_load().oracle_reshape_and_cache(_p(k), _p(v), _p(kc), _p(vc), _p(sm), T, H, D, bs, nb, _DT[dtype]))
    return kc, vc


def copy_blocks(k_cache, v_cache, pairs, dtype: str):
    """Return copies of the caches where block ``pairs[i, 1]`` holds the bits
    of block ``pairs[i, 0]`` (both caches, every head and offset)."""
    kc, vc = k_cache.copy(), v_cache.copy()
    pr = _c(pairs, np.int32).reshape(-1, 2)
    nb, H, bs, D = kc.shape
    _check(_load().oracle_copy_blocks(_p(kc), _p(vc), _p(pr), pr.shape[0], H, D, bs, nb, _DT[dtype]))
    return kc, vc


def gather_kv(k_cache, v_cache, block_tables, context_lens, dtype: str):
    """Logical K and V of every sequence, rows ``[sum ctx, H, D]`` in sequence
    order (raw storage values)."""
    kc, vc = _c(k_cache), _c(v_cache)
    bt, ctx = _c(block_tables, np.int32), _c(context_lens, np.int32)
    nb, H, bs, D = kc.shape
    total = int(ctx.sum())
    ko = np.empty((total, H, D), dtype=kc.dtype)
    vo = np.empty((total, H, D), dtype=vc.dtype)
    _check(_load().oracle_gather_kv(_p(ko), _p(vo), _p(kc), _p(vc), _p(bt), _p(ctx), ctx.shape[0], H, D, bs, nb,
                                    bt.shape[1], _DT[dtype]))
    return ko, vo


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str, pairs=None,
           threads: int = 0) -> np.ndarray:
    """fp64 decode attention. Returns ``[S,H,D]``, or ``[len(pairs), D]`` when
    ``pairs`` lists the (seq, head) pairs to compute."""
    q, kc, vc = _c(q), _c(k_cache), _c(v_cache)
    bt, ctx = _c(block_tables, np.int32), _c(context_lens, np.int32)
    nb, H, bs, D = kc.shape
    S = ctx.shape[0]
    full = pairs is None
    if full:
        pairs = np.stack(np.meshgrid(np.arange(S), np.arange(H), indexing="ij"), -1).reshape(-1, 2)
    pr = _c(pairs, np.int32).reshape(-1, 2)
    out = np.empty((pr.shape[0], D), dtype=np.float64)
    _check(_load().oracle_decode(_p(out), _p(q), _p(kc), _p(vc), _p(bt), _p(ctx), S, H, D, bs, nb, bt.shape[1],
                                 float(scale), _DT[dtype], _p(pr), pr.shape[0], int(threads)))
    return out.reshape(S, H, D) if full else out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale: float, dtype: str,
            rows=None, threads: int = 0) -> np.ndarray:
    """fp64 causal prefill. Returns ``[total_q,H,D]``, or ``[len(rows), D]``
    when ``rows`` lists the (query row, head) pairs to compute."""
    q, kc, vc = _c(q), _c(k_cache), _c(v_cache)
    bt, ctx, qsl = _c(block_tables, np.int32), _c(context_lens, np.int32), _c(query_start_loc, np.int32)
    nb, H, bs, D = kc.shape
    S = ctx.shape[0]
    TQ = int(qsl[-1])
    full = rows is None
    if full:
        rows = np.stack(np.meshgrid(np.arange(TQ), np.arange(H), indexing="ij"), -1).reshape(-1, 2)
    rr = _c(rows, np.int32).reshape(-1, 2)
    out = np.empty((rr.shape[0], D), dtype=np.float64)
    _check(_load().oracle_prefill(_p(out), _p(q), _p(kc), _p(vc), _p(bt), _p(ctx), _p(qsl), S, H, D, bs, nb,
                                  bt.shape[1], float(scale), _DT[dtype], _p(rr), rr.shape[0], int(threads)))
    return out.reshape(TQ, H, D) if full else out
