"""The oracle: a plain CPU statement of non-uniform paged decode attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import anything here.  The product
library (``non_uniform_paged_amd``) never imports, links or calls it, and the
oracle shares no code with it: no kernels, headers, helpers or tables.  The
only module both sides use is ``workloads`` (seeded random inputs, none of
the method's arithmetic).

Contents
  attention.c / decode()      fp64 attention over the paged cache (C, OpenMP)
  pager.py                    head grouping, block pager, append, coalescer,
                              gather: the integer / data-movement parts
  worktable.py                what makes a split-K work table valid
  brute.py                    pure-Python attention for tiny inputs

Parity status of each function is stated in its own docstring; every one is
pinned by ``tests/test_oracle_*.py`` against closed forms, library special
cases, hand-worked fixtures or brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_liboracle.so")
_lib = None

STATUS = {"OK": 0, "E_ARG": 1, "E_NOPAGES": 2, "E_CAPACITY": 3, "E_STATE": 4,
          "E_HIP": 5, "E_INDEX": 6}


def build(force: bool = True) -> str:
    """Compile the C part of the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "attention.c")
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC",
                               "-std=c99", src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_decode.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P,
                                      P, I, ctypes.c_double, P, P, I]
        lib.oracle_decode.restype = I
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def decode(q, pool_k, pool_v, page_table, lengths, group_of_head, slot_of_head,
           scale, tokens=None, num_threads=None):
    """fp64 decode attention (see attention.c for the definition).

    q:            uint16 bf16 bits [B][Hq][D]
    pool_k/v:     uint16 bf16 bits [num_pages][G_h][P][D]
    page_table:   int32 [n_g][B][max_pages]
    lengths:      int32 [B][Hkv]   (0 for inactive sequences)
    group_of_head, slot_of_head: int32 [Hkv]
    tokens:       optional int32 [B][Hkv][K] logical positions
    returns (out float64 [B][Hq][D], lse float64 [B][Hq])
    """
    lib = _load()
    B, Hq, D = q.shape
    num_pages, G_h, P, D2 = pool_k.shape
    assert D2 == D and pool_v.shape == pool_k.shape
    n_g, B2, max_pages = page_table.shape
    assert B2 == B
    Hkv = lengths.shape[1]
    keep = []
    args = []
    for a, dt in ((q, np.uint16), (pool_k, np.uint16), (pool_v, np.uint16),
                  (page_table, np.int32), (lengths, np.int32),
                  (group_of_head, np.int32), (slot_of_head, np.int32)):
        arr, p = _c(a, dt)
        keep.append(arr)
        args.append(p)
    K = 0
    if tokens is not None:
        tok, tp = _c(tokens, np.int32)
        keep.append(tok)
        K = tok.shape[-1]
    else:
        tp = None
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    nt = num_threads or os.cpu_count() or 1
    rc = lib.oracle_decode(B, Hq, Hkv, D, P, G_h, max_pages, *args, tp, K,
                           float(scale), out.ctypes.data_as(ctypes.c_void_p),
                           lse.ctypes.data_as(ctypes.c_void_p), int(nt))
    if rc != 0:
        raise ValueError("token position outside the retained range")
    return out, lse
