"""Seeded synthetic inputs for non-uniform paged decode attention.

This module only draws random inputs (budgets, lengths, top-K index lists,
end-of-sequence events, K/V/q contents and pool permutations).  It contains
none of the method's arithmetic: no grouping, paging, planning, gathering or
attention.  Both the oracle (``oracle/``) and the HIP path consume what it
draws, so the two sides always see the same bits.

Workload shapes follow the pages:
  * Tangram (Head Group Page, Fig 8; throughput breakdown at G = 4, Fig 10;
    KV growth of Qwen2.5-32B multi-turn sessions, Fig 1a; per-head retention
    profiles of Qwen3-4B, Fig 2 / Fig 6).
  * KVDrive (batch 8 at 122k context, Fig 5; 1.56% sparsity, Fig 16;
    sparse attention over critical entries, Fig 1).
  * KV-RM (controlled mixed-length serving, Fig 4c,d; EOS absorbed by the
    block pager, abstract).
None of the pages' datasets (SCBench, LongBench, RULER, the Azure trace) is
available; the distributions below are synthetic stand-ins.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

MASTER_SEED = 20261202
PAGE = 16  # tokens per page; every configuration uses 16-token pages

# Child streams of one SeedSequence, one per kind of random input.
_STREAMS = ("q", "k", "v", "budgets", "perm", "lengths", "indices", "eos")


def rng(kind: str, salt: int = 0) -> np.random.Generator:
    """Independent numpy generator for one kind of input (and an optional salt)."""
    idx = _STREAMS.index(kind)
    child = np.random.SeedSequence(MASTER_SEED).spawn(len(_STREAMS))[idx]
    if salt:
        child = np.random.SeedSequence([MASTER_SEED, idx, salt])
    return np.random.default_rng(child)


def torch_seed(kind: str, salt: int = 0) -> int:
    """Integer seed for torch generators (large pools are drawn with torch)."""
    return int(rng(kind, salt).integers(0, 2**62))


# --------------------------------------------------------------------------
# bf16 contents
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits.

    Inputs are finite normal draws, so NaN handling is not needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def normal_bf16(kind: str, shape: Sequence[int], salt: int = 0) -> np.ndarray:
    """N(0,1) draws rounded to bf16, as uint16 bits (numpy; small tensors)."""
    x = rng(kind, salt).standard_normal(size=tuple(shape), dtype=np.float32)
    return f32_to_bf16_bits(x)


def fill_normal_bf16_torch(t, kind: str, salt: int = 0, chunk: int = 1 << 26):
    """Fill a torch bfloat16 tensor (any device) with N(0,1) draws.

    Large pools are drawn on the tensor's own device in chunks so that no
    full-size float32 temporary is needed.  The values are reproducible for
    a given device type and seed."""
    import torch

    flat = t.view(-1)
    gen = torch.Generator(device=t.device)
    gen.manual_seed(torch_seed(kind, salt))
    n = flat.numel()
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        flat[lo:hi].copy_(torch.randn(hi - lo, generator=gen, device=t.device,
                                      dtype=torch.float32))
    return t


# --------------------------------------------------------------------------
# budgets and lengths
# --------------------------------------------------------------------------
def round_to_page(x: np.ndarray, ctx) -> np.ndarray:
    """Retained length from a fractional budget: nearest multiple of the page
    (halves round up), at least one page, at most the context."""
    x = np.asarray(x, dtype=np.float64)
    r = PAGE * np.floor(x / PAGE + 0.5)
    r = np.maximum(r, PAGE)
    return np.minimum(r, np.asarray(ctx)).astype(np.int64)


@dataclasses.dataclass
class Workload:
    """One synthetic decode batch.

    lengths[s][h]: retained tokens of (sequence slot s, KV head h)
    caps[s][h]:    reserved capacity (lengths + decode headroom)
    """
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_groups: int
    lengths: np.ndarray
    caps: np.ndarray
    num_pages: int
    free_list_init: Optional[np.ndarray] = None
    topk: int = 0
    extra: dict = dataclasses.field(default_factory=dict)

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def heads_per_group(self) -> int:
        return self.num_kv_heads // self.num_groups


def _group_footprint_pages(caps: np.ndarray, num_groups: int) -> int:
    """Upper bound of pages a head-group pager reserves for ``caps``: every
    group is charged the largest capacity in the batch.  Used only to size
    pools generously; the exact count is the pager's business."""
    per_seq = num_groups * math.ceil(int(caps.max()) / PAGE)
    return per_seq * caps.shape[0]


def tiny() -> Workload:
    """Tiny: batch 2, 4 KV heads = 4 query heads, head_dim 64, budgets
    {32, 64, 128, 256}, 2 head groups, pages permuted in a 64-page pool."""
    budgets = np.array([32, 64, 128, 256], dtype=np.int64)
    lengths = np.tile(budgets, (2, 1))
    perm = rng("perm").permutation(64).astype(np.int32)
    return Workload("tiny", 2, 4, 4, 64, 2, lengths, lengths.copy(), 64, perm)


def qwen3_4b(headroom: int = PAGE) -> Workload:
    """Qwen3-4B-shaped layer: batch 16, 32 q / 8 KV heads, d128, context 16384.

    Per-KV-head budgets are log-uniform in [256, 16384]; the pages ask for a
    50% mean, which that distribution does not have (its mean is about 24%).
    Reading: the eight draws are scaled by a common factor and clipped at the
    context so that their mean is exactly half the context, then rounded to
    the page.  Budgets are a static profile shared by all sequences."""
    ctx = 16384
    g = rng("budgets", 2)
    raw = np.exp(g.uniform(math.log(256), math.log(ctx), size=8))
    lo, hi = 1.0, 64.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(raw * mid, ctx).mean() < ctx / 2:
            lo = mid
        else:
            hi = mid
    budgets = round_to_page(np.minimum(raw * hi, ctx), ctx)
    lengths = np.tile(budgets, (16, 1))
    caps = lengths + headroom
    pool = int(math.ceil(1.25 * _group_footprint_pages(caps, 4)))
    return Workload("qwen3_4b", 16, 32, 8, 128, 4, lengths, caps, pool,
                    extra={"scale_factor": hi, "context": ctx})


def qwen3_4b_layers(num_layers: int = 36, headroom: int = PAGE, batch: int = 16,
                    context: int = 16384) -> Workload:
    """The Qwen3-4B shape over all its layers: 36 layers x 8 KV heads, one
    budget per (layer, KV head), log-uniform in [256, context] and scaled so
    the mean over all 288 heads is half the context (the same reading as the
    one-layer shape), rounded to the page.  num_kv_heads is per layer;
    lengths and caps are [batch][num_layers * 8], head index layer * 8 + h.
    A shorter context gives the same shape with short sessions."""
    ctx = context
    g = rng("budgets", 21)
    n = num_layers * 8
    raw = np.exp(g.uniform(math.log(256), math.log(ctx), size=n))
    lo, hi = 1.0, 64.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(raw * mid, ctx).mean() < ctx / 2:
            lo = mid
        else:
            hi = mid
    budgets = round_to_page(np.minimum(raw * hi, ctx), ctx)
    lengths = np.tile(budgets, (batch, 1))
    caps = lengths + headroom
    pool = int(math.ceil(1.25 * _group_footprint_pages(caps, 1) * 8))
    return Workload("qwen3_4b_layers", batch, 32, 8, 128, num_layers, lengths, caps, pool,
                    extra={"num_layers": num_layers, "context": ctx})


def qwen25_32b(headroom: int = PAGE, control: Optional[str] = None,
               batch: int = 64) -> Workload:
    """Qwen2.5-32B-shaped multi-turn layer: 64 sessions, 40 q / 8 KV heads,
    d128, per-session context uniform in [8192, 65536], per-KV-head keep
    ratio ~ Beta(0.5, 2) (a static profile of 8 draws), 4 head groups.

    control='uniform50' keeps 50% of every head (the uniform-budget control
    on the same contexts); control='uniform_mean' keeps the sample mean of
    the eight ratios (the same expected bytes as the non-uniform case)."""
    g = rng("lengths", 3)
    ctx = g.integers(8192, 65536, size=batch, endpoint=True)
    ratios = rng("budgets", 3).beta(0.5, 2.0, size=8)
    if control == "uniform50":
        ratios = np.full(8, 0.5)
    elif control == "uniform_mean":
        ratios = np.full(8, ratios.mean())
    elif control is not None:
        raise ValueError(control)
    lengths = round_to_page(ratios[None, :] * ctx[:, None], ctx[:, None])
    caps = lengths + headroom
    pool = int(math.ceil(1.25 * _group_footprint_pages(caps, 4)))
    name = "qwen25_32b" + ("" if control is None else "_" + control)
    return Workload(name, batch, 40, 8, 128, 4, lengths, caps, pool,
                    extra={"contexts": ctx, "ratios": ratios})


def qwen25_32b_prefix(prefix_ctx: int = 8192, n_sources: int = 4, batch: int = 64) -> Workload:
    """The Qwen2.5-32B-shaped batch, with forked sessions: sessions
    s >= n_sources continue source s % n_sources and share the first
    prefix_ctx tokens of its context (a common system prompt).  Head h keeps
    round_to_page(r_h * prefix_ctx) of them (its keep ratio r_h), limited by
    both sessions' retained lengths.

    extra["alias_src"][s]: the source session, -1 for the sources;
    extra["prefix_tokens"][s][h]: the retained tokens s shares with it."""
    w = qwen25_32b(batch=batch)
    ratios = w.extra["ratios"]
    keep = round_to_page(ratios * prefix_ctx, prefix_ctx)
    s_idx = np.arange(batch)
    src = np.where(s_idx < n_sources, -1, s_idx % n_sources)
    prefix = np.zeros_like(w.lengths)
    for s in range(n_sources, batch):
        prefix[s] = np.minimum(keep, np.minimum(w.lengths[s], w.lengths[src[s]]))
    w.name = "qwen25_32b_prefix"
    w.extra.update(alias_src=src, prefix_tokens=prefix, prefix_ctx=prefix_ctx)
    return w


def llama3_8b_topk(batch: int = 8, ctx: int = 122880, k: int = 2048) -> Workload:
    """Llama-3-8B-shaped sparse decode: batch 8, 32 q / 8 KV heads, d128,
    context 122880 held in full, one head group (8 heads per page), pages
    permuted in the pool, K = 2048 critical entries per (sequence, KV head)."""
    lengths = np.full((batch, 8), ctx, dtype=np.int64)
    pages = batch * (ctx // PAGE)
    perm = rng("perm", 4).permutation(pages).astype(np.int32)
    return Workload("llama3_8b_topk", batch, 32, 8, 128, 1, lengths,
                    lengths.copy(), pages, perm, topk=k)


def topk_indices(lengths: np.ndarray, k: int, salt: int = 4) -> np.ndarray:
    """Per (s, h): the k/2 most recent positions plus k/2 distinct positions
    drawn uniformly from the older history, sorted ascending (int32)."""
    g = rng("indices", salt)
    b, h = lengths.shape
    out = np.empty((b, h, k), dtype=np.int32)
    half = k // 2
    for s in range(b):
        for j in range(h):
            L = int(lengths[s, j])
            recent = np.arange(L - (k - half), L)
            old = g.choice(L - (k - half), size=half, replace=False)
            out[s, j] = np.sort(np.concatenate([old, recent]))
    return out


def cluster_lists(lengths: np.ndarray, C: int, salt: int = 5):
    """Member lists for C clusters per (s, h): every position 0..L-1 is
    assigned to a cluster uniformly at random and each list is ascending.
    Returns cl_start int32 [B][H][C+1] and cl_pos int32 [B][H][P] with
    P = max L (unused tail entries are -1)."""
    g = rng("indices", salt)
    b, h = lengths.shape
    P = int(lengths.max())
    start = np.zeros((b, h, C + 1), np.int32)
    pos = np.full((b, h, P), -1, np.int32)
    for s in range(b):
        for j in range(h):
            L = int(lengths[s, j])
            assign = g.integers(0, C, size=L)
            order = np.argsort(assign, kind="stable")          # ascending positions within a cluster
            pos[s, j, :L] = order
            start[s, j, 1:] = np.cumsum(np.bincount(assign, minlength=C))
    return start, pos


def nested_cluster_lists(lengths: np.ndarray, T: int, C: int, salt: int = 6):
    """Clustered positions for the centroid sweep.  Every position 0..L-1 of
    (s, h) draws one of T true clusters uniformly at random (the same draws
    whatever C is); the C clusters handed to the selection merge the true
    clusters whose ids are equal mod C (C divides T), so fewer centroids
    stand for coarser groups.  Returns true_of_pos int32 [B][H][P] (-1 past
    L), cl_start int32 [B][H][C+1] and cl_pos int32 [B][H][P] (each list
    ascending), P = max L."""
    assert T % C == 0
    g = rng("indices", salt)
    b, h = lengths.shape
    P = int(lengths.max())
    true_of_pos = np.full((b, h, P), -1, np.int32)
    start = np.zeros((b, h, C + 1), np.int32)
    pos = np.full((b, h, P), -1, np.int32)
    for s in range(b):
        for j in range(h):
            L = int(lengths[s, j])
            t = g.integers(0, T, size=L)
            true_of_pos[s, j, :L] = t
            assign = t % C
            pos[s, j, :L] = np.argsort(assign, kind="stable")
            start[s, j, 1:] = np.cumsum(np.bincount(assign, minlength=C))
    return true_of_pos, start, pos


def lognormal_lengths(n: int, g: np.random.Generator, median: float = 2048.0,
                      sigma: float = 1.0, lo: int = 16, hi: int = 131072) -> np.ndarray:
    """Mixed request lengths: lognormal with the given median, clipped."""
    x = g.lognormal(mean=math.log(median), sigma=sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def mixed_churn(batch: int = 256, sigma: float = 1.0, headroom: int = PAGE) -> Workload:
    """Mixed-length fixed-shape step: 256 slots, lengths lognormal (median
    2048, clipped to [16, 131072]; the spread is not stated, sigma = 1 is the
    reading), 32 q / 8 KV heads, d128, one head group.  The pool holds 1.5x
    the expected pages in use."""
    g = rng("lengths", 5)
    L = lognormal_lengths(batch, g, sigma=sigma)
    lengths = np.repeat(L[:, None], 8, axis=1)
    caps = lengths + headroom
    mean_len = 2048.0 * math.exp(sigma * sigma / 2)
    pool = int(math.ceil(1.5 * batch * (mean_len + headroom + PAGE) / PAGE))
    pool = max(pool, int(np.ceil(caps[:, 0] / PAGE).sum()) * 2)
    return Workload("mixed_churn", batch, 32, 8, 128, 1, lengths, caps, pool,
                    extra={"sigma": sigma})


class ChurnDriver:
    """Per-step EOS draws for the mixed-length workload: round(10% of the
    active slots) end each step; the freed slots come back at the next step
    with fresh lognormal lengths."""

    def __init__(self, batch: int, sigma: float = 1.0, headroom: int = PAGE,
                 frac: float = 0.1):
        self.g_eos = rng("eos", 5)
        self.g_len = rng("lengths", 55)
        self.batch, self.sigma, self.headroom, self.frac = batch, sigma, headroom, frac

    def eos(self, active_slots: np.ndarray) -> np.ndarray:
        n = int(round(self.frac * len(active_slots)))
        if n == 0:
            return np.zeros(0, dtype=np.int32)
        return np.sort(self.g_eos.choice(active_slots, size=n, replace=False)).astype(np.int32)

    def refill_lengths(self, n: int) -> np.ndarray:
        return lognormal_lengths(n, self.g_len, sigma=self.sigma)


CONFIGS = {
    "tiny": tiny,
    "qwen3_4b": qwen3_4b,
    "qwen25_32b": qwen25_32b,
    "qwen25_32b_prefix": qwen25_32b_prefix,
    "qwen3_4b_layers": qwen3_4b_layers,
    "llama3_8b_topk": llama3_8b_topk,
    "mixed_churn": mixed_churn,
}
