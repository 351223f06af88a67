"""Python binding of libnupaged.so (non-uniform paged decode attention, MI355X).

Argument marshalling only: every step of the path runs in the library's
host code and HIP kernels.  The functions carry the C ABI's names and take
torch tensors (device buffers) or numpy arrays (host buffers); PyTorch is
used only to own device memory and to provide the stream.

Importing this module loads the library; if it has not been built the
import fails loudly (build with ``python -m non_uniform_paged_amd.build`` or
``__graft_entry__.build()``) -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnupaged.so")

NUP_OK, NUP_E_ARG, NUP_E_NOPAGES, NUP_E_CAPACITY, NUP_E_STATE, NUP_E_HIP, NUP_E_INDEX = range(7)
STATUS_NAMES = {0: "NUP_OK", 1: "NUP_E_ARG", 2: "NUP_E_NOPAGES", 3: "NUP_E_CAPACITY",
                4: "NUP_E_STATE", 5: "NUP_E_HIP", 6: "NUP_E_INDEX"}
PLAN_BALANCED, PLAN_UNIFORM, PLAN_SHARED = 0, 1, 2
MERGE_AUTO, MERGE_LAUNCH, MERGE_IN_SPLIT = 0, 1, 2
PAGE = 16


class NupError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class NupConfig(ctypes.Structure):
    _fields_ = [("num_kv_heads", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_groups", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_workers", ctypes.c_int32), ("plan_mode", ctypes.c_int32),
                ("uniform_splits", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("merge_mode", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("desc", ctypes.c_void_p), ("free_list_init", ctypes.c_void_p)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run non_uniform_paged_amd/build.py")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
_sigs = {
    "nup_desc_bytes": [_P, _P],
    "nup_create": [_P, _P],
    "kv_alloc_groups": [_P, _I, _P, _P, _P, _P],
    "kv_alias": [_P, _I, _P, _P, _P, _P, _P],
    "kv_free_seqs": [_P, _I, _P],
    "kv_gather_trains_dma": [_P, _P, _P, _P, _P, _P],
    "nup_commit": [_P, _P],
    "kv_append": [_P, _P, _P, _P],
    "kv_gather_compact": [_P, _I, _P, _I, _P, _P, _P, _P, _P],
    "nup_workspace_bytes": [_P, _I, _P],
    "attn_decode_nonuniform": [_P, _P, _P, _P, ctypes.c_float, _P, _S, _P],
    "attn_decode_nonuniform_append": [_P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _S, _P],
    "attn_decode_nonuniform_noalloc": [_P, _P, _P, _P, ctypes.c_float, _P],
    "attn_decode_topk": [_P, _P, _P, _P, _I, _P, _P, ctypes.c_float, _P, _S, _P],
    "attn_decode_topk_paged": [_P, _P, _P, _I, _P, _P, ctypes.c_float, _P, _S, _P],
    "kv_select_topk": [_P, _P, _I, _I, _P, _P, _S, _P],
    "nup_select_workspace_bytes": [_P, _P],
    "nup_get_page_table": [_P, _P],
    "nup_get_lengths": [_P, _P],
    "nup_get_groups": [_P, _P, _P],
    "nup_get_free_list": [_P, _P, _P],
    "nup_get_refcounts": [_P, _P],
    "kv_select_topk_centroids": [_P, _P, _P, _I, _P, _P, _I, _I, _I, _P, _P, _S, _P],
    "nup_centroid_workspace_bytes": [_P, _I, _P],
    "nup_set_layer": [_P, _I],
    "nup_note_appends": [_P, _I, _I],
    "nup_get_runs": [_P, _P, _I, _P],
    "nup_get_plan": [_P, _P, _P, _P, _P, _P],
    "nup_get_plan_head_rows": [_P, _P],
    "nup_get_plan_gangs": [_P, _P, _P, _P],
    "nup_set_timing": [_P, _I],
    "nup_kernel_time": [_P, _P, _P, _I],
    "nup_device_errors": [_P, _P, _P],
    "nup_probe_copy": [_P, _P, _S, _P],
    "nup_probe_read": [_P, _S, _P, _P],
}
for _name, _args in _sigs.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int32
_lib.nup_destroy.argtypes = [_P]
_lib.nup_destroy.restype = None
_lib.nup_last_error.argtypes = [_P]
_lib.nup_last_error.restype = ctypes.c_char_p

EXPORTED = sorted(list(_sigs) + ["nup_destroy", "nup_last_error"])


def _ptr(x) -> Optional[int]:
    """Address of a torch tensor, a numpy array, or None."""
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    if isinstance(x, int):
        return x
    raise TypeError(f"cannot pass {type(x)}")


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


class Context:
    """Owns an nup_ctx and keeps the device buffers it points to alive."""

    def __init__(self, *, num_kv_heads, num_q_heads, head_dim, num_groups, max_batch,
                 num_pages, max_pages, k_pool=None, v_pool=None, desc=None,
                 free_list_init=None, num_workers=0, plan_mode=PLAN_BALANCED,
                 uniform_splits=0, num_layers=1, merge_mode=0):
        cfg = NupConfig(num_kv_heads, num_q_heads, head_dim, PAGE, num_groups, max_batch,
                        num_pages, max_pages, num_workers, plan_mode, uniform_splits, num_layers,
                        merge_mode, _ptr(k_pool), _ptr(v_pool), _ptr(desc), None)
        self._fl = None
        if free_list_init is not None:
            self._fl = _i32(free_list_init)
            cfg.free_list_init = self._fl.ctypes.data
        self.cfg = cfg
        self._keep = (k_pool, v_pool, desc)
        h = ctypes.c_void_p()
        st = _lib.nup_create(ctypes.byref(cfg), ctypes.byref(h))
        if st != NUP_OK:
            raise NupError(st, "nup_create rejected the configuration")
        self.handle = h
        self.H, self.Hq, self.D = num_kv_heads, num_q_heads, head_dim
        self.ng, self.B, self.num_pages, self.max_pages = num_groups, max_batch, num_pages, max_pages
        self.num_layers = max(1, num_layers)
        self.V = self.num_layers * num_kv_heads      # the pager's (layer, KV head) pairs

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:        # at interpreter exit the module may be torn down first
            _lib.nup_destroy(h)
            self.handle = None

    def check(self, st: int):
        if st != NUP_OK:
            raise NupError(st, _lib.nup_last_error(self.handle).decode())
        return st


def desc_bytes(**cfg) -> int:
    c = NupConfig(cfg["num_kv_heads"], cfg["num_q_heads"], cfg["head_dim"], PAGE,
                  cfg["num_groups"], cfg["max_batch"], cfg["num_pages"], cfg["max_pages"],
                  cfg.get("num_workers", 0), cfg.get("plan_mode", 0),
                  cfg.get("uniform_splits", 0), cfg.get("num_layers", 1), cfg.get("merge_mode", 0),
                  None, None, None, None)
    n = ctypes.c_size_t()
    st = _lib.nup_desc_bytes(ctypes.byref(c), ctypes.byref(n))
    if st != NUP_OK:
        raise NupError(st, "nup_desc_bytes rejected the configuration")
    return n.value


# ---- the five path calls, plus commit / free ---------------------------------

def kv_alloc_groups(ctx: Context, slots, cap, len=None, raise_on_error=True):
    slots = _i32(slots)
    cap = _i32(cap).reshape(len_(slots), ctx.V)
    ln = None if len is None else _i32(len).reshape(len_(slots), ctx.V)
    goh = np.zeros(ctx.V, np.int32)
    st = _lib.kv_alloc_groups(ctx.handle, len_(slots), slots.ctypes.data, cap.ctypes.data,
                              None if ln is None else ln.ctypes.data, goh.ctypes.data)
    if raise_on_error:
        ctx.check(st)
        return goh
    return st


def len_(a) -> int:
    return int(np.asarray(a).shape[0])


def kv_alias(ctx: Context, slots, src_slots, share_pages, cap, len, raise_on_error=True):
    slots = _i32(slots)
    n = len_(slots)
    src = _i32(src_slots).reshape(n)
    share = _i32(share_pages).reshape(n, ctx.ng)
    cap = _i32(cap).reshape(n, ctx.V)
    ln = _i32(len).reshape(n, ctx.V)
    st = _lib.kv_alias(ctx.handle, n, slots.ctypes.data, src.ctypes.data, share.ctypes.data,
                       cap.ctypes.data, ln.ctypes.data)
    return ctx.check(st) if raise_on_error else st


def kv_free_seqs(ctx: Context, slots, raise_on_error=True):
    slots = _i32(slots)
    st = _lib.kv_free_seqs(ctx.handle, len_(slots), slots.ctypes.data if len_(slots) else None)
    return ctx.check(st) if raise_on_error else st


def nup_commit(ctx: Context, stream=None, raise_on_error=True):
    st = _lib.nup_commit(ctx.handle, _stream(stream))
    return ctx.check(st) if raise_on_error else st


def kv_append(ctx: Context, k_new, v_new, stream=None, raise_on_error=True):
    st = _lib.kv_append(ctx.handle, _ptr(k_new), _ptr(v_new), _stream(stream))
    return ctx.check(st) if raise_on_error else st


def kv_gather_compact(ctx: Context, mode: int, k_out, v_out, idx=None, K: int = 0,
                      row_off=None, phys_out=None, stream=None, raise_on_error=True):
    st = _lib.kv_gather_compact(ctx.handle, mode, _ptr(idx), K, _ptr(k_out), _ptr(v_out),
                                _ptr(row_off), _ptr(phys_out), _stream(stream))
    return ctx.check(st) if raise_on_error else st


def kv_gather_trains_dma(ctx: Context, k_out, v_out, row_off, stream=None, raise_on_error=True):
    """row_off: host int64 array [B_max*H_kv].  Returns the number of copies
    enqueued (or the status when raise_on_error is False)."""
    ro = np.ascontiguousarray(np.asarray(row_off, dtype=np.int64).reshape(-1))
    if ro.size != ctx.B * ctx.H:
        raise ValueError("row_off must hold B_max*H_kv offsets")
    n = ctypes.c_int32()
    st = _lib.kv_gather_trains_dma(ctx.handle, _ptr(k_out), _ptr(v_out), ro.ctypes.data,
                                   ctypes.byref(n), _stream(stream))
    if raise_on_error:
        ctx.check(st)
        return n.value
    return st


def workspace_bytes(ctx: Context, K: int = 0) -> int:
    n = ctypes.c_size_t()
    ctx.check(_lib.nup_workspace_bytes(ctx.handle, K, ctypes.byref(n)))
    return n.value


def attn_decode_nonuniform(ctx: Context, q, out, lse, scale: float, workspace, stream=None,
                           raise_on_error=True):
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.attn_decode_nonuniform(ctx.handle, _ptr(q), _ptr(out), _ptr(lse), float(scale),
                                     _ptr(workspace), nbytes, _stream(stream))
    return ctx.check(st) if raise_on_error else st


NOALLOC_SCRATCH_BYTES = 32 << 20   # NUP_NOALLOC_SCRATCH_BYTES in nupaged.h


def attn_decode_nonuniform_noalloc(ctx: Context, q, out, lse, scale: float, stream=None,
                                   raise_on_error=True):
    st = _lib.attn_decode_nonuniform_noalloc(ctx.handle, _ptr(q), _ptr(out), _ptr(lse), float(scale),
                                             _stream(stream))
    return ctx.check(st) if raise_on_error else st


def attn_decode_nonuniform_append(ctx: Context, k_new, v_new, q, out, lse, scale: float, workspace,
                                  stream=None, raise_on_error=True):
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.attn_decode_nonuniform_append(ctx.handle, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                            _ptr(lse), float(scale), _ptr(workspace), nbytes, _stream(stream))
    return ctx.check(st) if raise_on_error else st


def attn_decode_topk(ctx: Context, q, k_stage, v_stage, K: int, out, lse, scale: float,
                     workspace, stream=None, raise_on_error=True):
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.attn_decode_topk(ctx.handle, _ptr(q), _ptr(k_stage), _ptr(v_stage), K, _ptr(out),
                               _ptr(lse), float(scale), _ptr(workspace), nbytes, _stream(stream))
    return ctx.check(st) if raise_on_error else st


def attn_decode_topk_paged(ctx: Context, q, idx, K: int, out, lse, scale: float, workspace,
                           stream=None, raise_on_error=True):
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.attn_decode_topk_paged(ctx.handle, _ptr(q), _ptr(idx), K, _ptr(out), _ptr(lse),
                                     float(scale), _ptr(workspace), nbytes, _stream(stream))
    return ctx.check(st) if raise_on_error else st


def kv_select_topk(ctx: Context, q, K: int, window: int, idx_out, workspace, stream=None,
                   raise_on_error=True):
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.kv_select_topk(ctx.handle, _ptr(q), K, window, _ptr(idx_out), _ptr(workspace), nbytes,
                             _stream(stream))
    return ctx.check(st) if raise_on_error else st


def kv_select_topk_centroids(ctx: Context, q, centroids, C: int, cl_start, cl_pos, P: int, K: int,
                             window: int, idx_out, workspace, stream=None, raise_on_error=True):
    st = _lib.kv_select_topk_centroids(ctx.handle, _ptr(q), _ptr(centroids), C, _ptr(cl_start),
                                       _ptr(cl_pos), P, K, window, _ptr(idx_out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream))
    return ctx.check(st) if raise_on_error else st


def centroid_workspace_bytes(ctx: Context, C: int) -> int:
    n = ctypes.c_size_t()
    ctx.check(_lib.nup_centroid_workspace_bytes(ctx.handle, C, ctypes.byref(n)))
    return n.value


def select_workspace_bytes(ctx: Context) -> int:
    n = ctypes.c_size_t()
    ctx.check(_lib.nup_select_workspace_bytes(ctx.handle, ctypes.byref(n)))
    return n.value


# ---- host-side queries ------------------------------------------------------

def get_page_table(ctx: Context) -> np.ndarray:
    out = np.zeros((ctx.ng, ctx.B, ctx.max_pages), np.int32)
    ctx.check(_lib.nup_get_page_table(ctx.handle, out.ctypes.data))
    return out


def get_lengths(ctx: Context) -> np.ndarray:
    out = np.zeros((ctx.B, ctx.V), np.int32)
    ctx.check(_lib.nup_get_lengths(ctx.handle, out.ctypes.data))
    return out


def get_groups(ctx: Context):
    g = np.zeros(ctx.V, np.int32)
    s = np.zeros(ctx.V, np.int32)
    ctx.check(_lib.nup_get_groups(ctx.handle, g.ctypes.data, s.ctypes.data))
    return g, s


def get_free_list(ctx: Context) -> np.ndarray:
    out = np.zeros(ctx.num_pages, np.int32)
    n = ctypes.c_int32()
    ctx.check(_lib.nup_get_free_list(ctx.handle, out.ctypes.data, ctypes.byref(n)))
    return out[: n.value]


def set_layer(ctx: Context, layer: int):
    """Choose the layer the per-layer calls act on."""
    ctx.check(_lib.nup_set_layer(ctx.handle, int(layer)))


def note_appends(ctx: Context, steps: int, layer: int = -1):
    """Advance the host's lengths by `steps` replayed appends of `layer`
    (-1: all layers); raises NupError(NUP_E_CAPACITY) if a head hit its
    budget, after updating the lengths as the device did."""
    ctx.check(_lib.nup_note_appends(ctx.handle, int(layer), int(steps)))


def get_refcounts(ctx: Context) -> np.ndarray:
    out = np.zeros(ctx.num_pages, np.int32)
    ctx.check(_lib.nup_get_refcounts(ctx.handle, out.ctypes.data))
    return out


def get_runs(ctx: Context) -> np.ndarray:
    n = ctypes.c_int32()
    ctx.check(_lib.nup_get_runs(ctx.handle, None, 0, ctypes.byref(n)))
    out = np.zeros((max(n.value, 1), 5), np.int32)
    ctx.check(_lib.nup_get_runs(ctx.handle, out.ctypes.data, n.value, ctypes.byref(n)))
    return out[: n.value]


def get_plan(ctx: Context):
    nr, nw = ctypes.c_int32(), ctypes.c_int32()
    ctx.check(_lib.nup_get_plan(ctx.handle, ctypes.byref(nr), ctypes.byref(nw), None, None, None))
    rows = np.zeros((max(nr.value, 1), 4), np.int32)
    ws = np.zeros(nw.value + 1, np.int32)
    hrs = np.zeros(ctx.B * ctx.H + 1, np.int32)
    ctx.check(_lib.nup_get_plan(ctx.handle, None, None, rows.ctypes.data, ws.ctypes.data,
                                hrs.ctypes.data))
    return rows[: nr.value], ws, hrs


def get_plan_head_rows(ctx: Context) -> np.ndarray:
    nr = ctypes.c_int32()
    ctx.check(_lib.nup_get_plan(ctx.handle, ctypes.byref(nr), None, None, None, None))
    out = np.zeros(max(nr.value, 1), np.int32)
    ctx.check(_lib.nup_get_plan_head_rows(ctx.handle, out.ctypes.data))
    return out[: nr.value]


def get_plan_gangs(ctx: Context):
    """(gang_rows [n_blocks][4], worker_skip [n_workers]) of the current layer's plan."""
    nb = ctypes.c_int32()
    ctx.check(_lib.nup_get_plan_gangs(ctx.handle, ctypes.byref(nb), None, None))
    nw = ctypes.c_int32()
    ctx.check(_lib.nup_get_plan(ctx.handle, None, ctypes.byref(nw), None, None, None))
    gr = np.zeros((max(nb.value, 1), 4), np.int32)
    sk = np.zeros(max(nw.value, 1), np.int32)
    ctx.check(_lib.nup_get_plan_gangs(ctx.handle, None, gr.ctypes.data, sk.ctypes.data))
    return gr[: nb.value], sk[: nw.value]


def set_timing(ctx: Context, enable: bool = True):
    ctx.check(_lib.nup_set_timing(ctx.handle, int(enable)))


def kernel_time(ctx: Context, reset: bool = True):
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    ctx.check(_lib.nup_kernel_time(ctx.handle, ctypes.byref(ms), ctypes.byref(n), int(reset)))
    return ms.value, n.value


def device_errors(ctx: Context, stream=None) -> int:
    code = ctypes.c_int32()
    ctx.check(_lib.nup_device_errors(ctx.handle, _stream(stream), ctypes.byref(code)))
    return code.value


def probe_read(src, nbytes: int, sink, stream=None):
    st = _lib.nup_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(stream))
    if st != NUP_OK:
        raise NupError(st, "nup_probe_read failed")


def probe_copy(src, dst, nbytes: int, stream=None):
    st = _lib.nup_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream))
    if st != NUP_OK:
        raise NupError(st, "nup_probe_copy failed")
