#!/usr/bin/env python3
"""Benchmark: non-uniform paged decode attention on one MI355X.

One step is one decode step of the Qwen2.5-32B-shaped multi-turn layer
(64 sessions, 40 query / 8 KV heads, head_dim 128, contexts uniform in
[8192, 65536], per-KV-head keep ratios ~ Beta(0.5, 2), 4 head groups, 16-token
pages): kv_append of one token per (session, KV head), the frame commit, and
attn_decode_nonuniform (split-K partial attention + log-sum-exp merge).
Inputs are synthetic (seeded) and resident in HBM before timing starts.

Prints one JSON line.  `value` is the step's algorithmic bytes per second
(GB/s); `roofline` is the split-K partial-attention kernel (the dominant
kernel) timed with HIP events on its own stream; `cpu_baseline` is the fp64
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0


def kv_bytes(lengths, D=128):
    return int(np.asarray(lengths, dtype=np.int64).sum()) * 2 * D * 2


def algorithmic_bytes(lengths, caps, B, Hq, Hkv, ng, D=128, page=16, gqa_rows=True):
    """Bytes the decode attention must move: retained K+V, q, out, the page
    table entries it walks and the lengths."""
    L = np.asarray(lengths, dtype=np.int64)
    kv = int(L.sum()) * 2 * D * 2
    q = B * Hq * D * 2
    out = B * Hq * D * 4
    gh = Hkv // ng
    pages = 0
    for g in range(ng):
        pages += int(np.ceil(np.asarray(caps)[:, g * gh:(g + 1) * gh].max(axis=1) / page).sum())
    return kv + q + out + pages * 4 + B * Hkv * 4


# where split heads are merged (nupaged.h NUP_MERGE_*): set by --merge
MERGE_MODE = 0


class Setup:
    """Pools, context and step buffers for one workload on the GPU."""

    def __init__(self, w, headroom_steps, num_workers=0, plan_mode=0, uniform_splits=0,
                 max_pages=None):
        import torch
        import non_uniform_paged_amd as nup
        import workloads as W

        self.w = w
        # decode headroom: room for the appends of the run (none when nothing is appended)
        pad = 16 * int(math.ceil((headroom_steps + 1) / 16)) if headroom_steps > 0 else 0
        self.caps = (w.lengths + pad).astype(np.int32)
        self.lengths0 = w.lengths.astype(np.int32)
        B, H, Hq, D, ng = w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, w.num_groups
        gh = H // ng
        max_pages = max_pages or int(math.ceil(self.caps.max() / 16))
        self.pad = pad
        self.max_pages = max_pages
        need = 0
        for g in range(ng):
            need += int(np.ceil(self.caps[:, g * gh:(g + 1) * gh].max(axis=1) / 16).sum())
        num_pages = max(w.num_pages, need)
        free_list = w.free_list_init
        if free_list is not None and num_pages > len(free_list):
            free_list = np.concatenate([free_list, np.arange(len(free_list), num_pages)]).astype(np.int32)
        self.kpool = torch.empty((num_pages, gh, 16, D), dtype=torch.bfloat16, device="cuda")
        self.vpool = torch.empty_like(self.kpool)
        W.fill_normal_bf16_torch(self.kpool, "k")
        W.fill_normal_bf16_torch(self.vpool, "v")
        cfg = dict(num_kv_heads=H, num_q_heads=Hq, head_dim=D, num_groups=ng, max_batch=B,
                   num_pages=num_pages, max_pages=max_pages, num_workers=num_workers,
                   plan_mode=plan_mode, uniform_splits=uniform_splits, merge_mode=MERGE_MODE)
        self.desc = torch.empty(nup.desc_bytes(**cfg), dtype=torch.uint8, device="cuda")
        self.ctx = nup.Context(**cfg, k_pool=self.kpool, v_pool=self.vpool, desc=self.desc,
                               free_list_init=free_list)
        self.free_list = free_list
        src = w.extra.get("alias_src")
        if src is None:
            nup.kv_alloc_groups(self.ctx, np.arange(B), self.caps, self.lengths0)
        else:
            # forked sessions: Reserve the sources, then Alias the forks onto
            # the whole pages of their shared prefix
            roots = np.nonzero(src < 0)[0]
            forks = np.nonzero(src >= 0)[0]
            goh = nup.kv_alloc_groups(self.ctx, roots, self.caps[roots], self.lengths0[roots])
            pre = w.extra["prefix_tokens"]
            self.share = np.zeros((len(forks), ng), np.int32)
            for g in range(ng):
                self.share[:, g] = pre[forks][:, goh == g].min(axis=1) // 16
            nup.kv_alias(self.ctx, forks, src[forks], self.share, self.caps[forks], self.lengths0[forks])
            self.goh = goh
        nup.nup_commit(self.ctx)
        self.q = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
        W.fill_normal_bf16_torch(self.q, "q")
        self.k_new = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
        self.v_new = torch.empty_like(self.k_new)
        W.fill_normal_bf16_torch(self.k_new, "k", 77)
        W.fill_normal_bf16_torch(self.v_new, "v", 77)
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        self.ws = torch.empty(nup.workspace_bytes(self.ctx), dtype=torch.uint8, device="cuda")
        self.scale = 1.0 / math.sqrt(D)
        self.num_pages = num_pages
        self.steps_done = 0

    def step(self, append=True, fused=True):
        """One decode step: frame commit, the new token's K/V append and the
        attention -- fused (two launches) or as separate calls (three)."""
        import non_uniform_paged_amd as nup
        nup.nup_commit(self.ctx)
        if append and fused:
            nup.attn_decode_nonuniform_append(self.ctx, self.k_new, self.v_new, self.q, self.out, self.lse,
                                              self.scale, self.ws)
        else:
            if append:
                nup.kv_append(self.ctx, self.k_new, self.v_new)
            nup.attn_decode_nonuniform(self.ctx, self.q, self.out, self.lse, self.scale, self.ws)
        if append:
            self.steps_done += 1

    def free(self):
        import torch
        del self.ctx
        del self.kpool, self.vpool, self.desc, self.ws
        torch.cuda.empty_cache()


class _Event:
    """A timing event on torch's current stream, created without the
    system-scope fence (hipEventDisableSystemFence): a fenced event adds a
    writeback of the caches to the interval it closes.  The HIP runtime is
    the one torch has loaded (same soname)."""
    _hip = None

    def __init__(self):
        import ctypes
        if _Event._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            _Event._hip = hip
        self._ev = ctypes.c_void_p()
        rc = _Event._hip.hipEventCreateWithFlags(ctypes.byref(self._ev), 0x20000000)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: error {rc}")

    def record(self):
        import torch
        rc = _Event._hip.hipEventRecord(self._ev, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord: error {rc}")

    def elapsed_time(self, other):
        import ctypes
        ms = ctypes.c_float()
        rc = _Event._hip.hipEventElapsedTime(ctypes.byref(ms), self._ev, other._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime: error {rc}")
        return ms.value

    def __del__(self):
        if _Event._hip is not None and self._ev:
            _Event._hip.hipEventDestroy(self._ev)


def time_steps(setup, steps, warmup, append=True, fused=True, per_step=None, kernel=True):
    """Returns (ms per step, mean lengths of those steps, split-K kernel ms per
    launch, mean lengths of the kernel pass).  The step time comes from a pass
    without the library's kernel events, since every timing event adds a few
    microseconds of GPU time between the launches it brackets; the kernel
    time (when `kernel`) from a second pass of as many steps with them.
    per_step: a list that receives each timed step's milliseconds (an event
    between consecutive steps on the launch stream)."""
    import torch
    import non_uniform_paged_amd as nup

    def one_pass(per):
        L_before = setup.lengths0 + setup.steps_done
        torch.cuda.synchronize()
        # per-step events only when asked: each one is a barrier between steps
        n_ev = steps + 1 if per is not None else 2
        ev = [_Event() for _ in range(n_ev)]
        ev[0].record()
        for i in range(steps):
            setup.step(append, fused)
            if per is not None:
                ev[i + 1].record()
        if per is None:
            ev[1].record()
        torch.cuda.synchronize()
        if per is not None:
            per.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        L_after = setup.lengths0 + setup.steps_done
        # lengths seen by the attention of each timed step: L_before+1 .. L_after
        mean_L = (L_before + L_after + 1) / 2.0 if append else L_before
        return ev[0].elapsed_time(ev[-1]) / steps, mean_L

    for _ in range(warmup):
        setup.step(append, fused)
    ms, mean_L = one_pass(per_step)
    if not kernel:
        return ms, mean_L, None, None
    nup.kernel_time(setup.ctx, reset=True)
    nup.set_timing(setup.ctx, True)
    _, kmean_L = one_pass(None)
    nup.set_timing(setup.ctx, False)
    kms, n = nup.kernel_time(setup.ctx, reset=True)
    return ms, mean_L, kms / max(n, 1), kmean_L


def plan_straggler(ctx, lengths):
    """Largest over mean per-worker pages of the committed plan, counting
    each row's pages up to the head's current length: the straggler
    measure of the split (1.0 = every worker has the same work)."""
    import non_uniform_paged_amd as nup
    rows, ws, _ = nup.get_plan(ctx)
    L = np.asarray(lengths, np.int64).reshape(-1)
    t1 = np.minimum(rows[:, 2].astype(np.int64), L[rows[:, 0]])
    t0 = rows[:, 1].astype(np.int64)
    pages = np.where(t1 > t0, (t1 + 15) // 16 - t0 // 16, 0)
    cs = np.concatenate([[0], np.cumsum(pages)])
    per = cs[ws[1:]] - cs[ws[:-1]]
    return float(per.max() / max(per.mean(), 1e-9)), int(len(ws) - 1)


def traffic_from_profiles(kernel_src_sha):
    p = os.path.join(ROOT, "profiles", "traffic_partial_attn_qwen25_32b.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except Exception:
        return None
    if t.get("kernels_hip_sha256") != kernel_src_sha:
        return None
    return t.get("hbm_bytes_per_launch")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


def oracle_spec(setup):
    """The oracle's own pager state for a Setup's first Reserve (the same
    capacities, lengths and free list as the library's)."""
    from oracle import pager as pg
    w = setup.w
    spec = pg.PagerSpec(w.num_kv_heads, w.num_groups, w.batch, setup.num_pages,
                        setup.max_pages, 16, setup.free_list)
    assert spec.alloc(np.arange(w.batch), setup.caps, setup.lengths0) == pg.OK
    return spec


def oracle_timing(setup, spec, tokens=None, budget_all_s=1.5, budget_one_s=1.0, runs_all=5, runs_one=3):
    """The fp64 oracle (test infrastructure, timed here as the CPU baseline)
    on this host's cores and on one thread: the median of `runs` calls over
    the first n sessions of the same inputs, n sized so that one call takes
    about budget seconds.  Rates are the calls' algorithmic bytes per second
    (K/V of every retained token or listed entry, q, out, page-table
    entries, lengths)."""
    import torch
    import oracle
    w = setup.w
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))

    def sample(seqs):
        sub = spec.page_table[:, seqs, :]
        used = np.unique(sub[sub >= 0])
        remap = np.full(spec.num_pages, -1, np.int64)
        remap[used] = np.arange(len(used))
        pt = np.where(sub >= 0, remap[np.maximum(sub, 0)], -1).astype(np.int32)
        idx = torch.from_numpy(used.astype(np.int64)).cuda()
        pk = setup.kpool.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
        pv = setup.vpool.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
        q = setup.q.view(torch.int16).cpu().numpy().view(np.uint16)[seqs]
        L = spec.lengths[seqs]
        tok = None if tokens is None else np.ascontiguousarray(tokens[seqs])
        if tokens is None:
            nb = algorithmic_bytes(L, setup.caps[seqs], len(seqs), w.num_q_heads, w.num_kv_heads,
                                   w.num_groups)
        else:
            n_ent = len(seqs) * w.num_kv_heads * tokens.shape[-1]
            nb = n_ent * (2 * w.head_dim * 2 + 4) + len(seqs) * w.num_q_heads * w.head_dim * (2 + 4)
        return (q, pk, pv, pt, L, tok), nb

    def call(smp, nt):
        q, pk, pv, pt, L, tok = smp
        t0 = time.perf_counter()
        oracle.decode(q, pk, pv, pt, L, spec.group_of_head, spec.slot_of_head, setup.scale,
                      tokens=tok, num_threads=nt)
        return time.perf_counter() - t0

    def size(budget, nt):
        smp, nb = sample([0])
        dt = call(smp, nt)
        n = int(max(1, min(w.batch, math.floor(budget / max(dt, 1e-4)))))
        if n > 1:
            smp, nb = sample(list(range(n)))
        return (smp, nb), n

    (smp, nb), n = size(budget_all_s, threads)
    t_all = float(np.median([call(smp, threads) for _ in range(runs_all)]))
    del smp
    (smp1, nb1), n1 = size(budget_one_s, 1)
    t_one = float(np.median([call(smp1, 1) for _ in range(runs_one)]))
    del smp1
    what = "listed entries" if tokens is not None else "retained tokens"
    return {"value": round(nb / t_all / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {w.batch} sessions (all KV heads, their {what}), one decode step of "
                      f"attention; median of {runs_all} calls of {t_all:.2f} s; fp64 C oracle with OpenMP",
            "one_thread_value": round(nb1 / t_one / 1e9, 4),
            "one_thread_sample": f"first {n1} sessions, median of {runs_one} calls of {t_one:.2f} s",
            "cpu_model": _cpu_model()}


def cpu_baseline(setup):
    """The CPU baseline of the headline line: the oracle on the same batch."""
    return oracle_timing(setup, oracle_spec(setup), budget_all_s=2.5, budget_one_s=1.5)


def _timed_stats(fn, iters, flush=None):
    """(mean, median, p90) ms of fn() over iters calls, each preceded
    (outside the timed window) by flush() when given; events on the current
    stream."""
    import torch
    times = []
    for _ in range(iters):
        if flush is not None:
            flush()
        e0, e1 = _Event(), _Event()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.mean(times)), float(np.median(times)), float(np.percentile(times, 90))


def _timed(fn, iters, flush=None):
    """Average ms of fn() over iters calls (see _timed_stats)."""
    return _timed_stats(fn, iters, flush)[0]


def _med_p90(stats, key):
    """{key_median, key_p90} from a _timed_stats triple, rounded."""
    return {key + "_median": round(stats[1], 4), key + "_p90": round(stats[2], 4)}


def _timed_call_and_kernel(ctx, fn, iters, flush=None):
    """(ms per call, ms per split-K launch, the call's _timed_stats).  The
    call time comes from a pass without the library's own kernel events,
    since every timing event adds a few microseconds of GPU time between the
    launches it brackets; the kernel time from a second pass with them."""
    import non_uniform_paged_amd as nup
    stats = _timed_stats(fn, iters, flush)
    nup.kernel_time(ctx, reset=True)
    nup.set_timing(ctx, True)
    _timed(fn, iters, flush)
    nup.set_timing(ctx, False)
    kms, n = nup.kernel_time(ctx, reset=True)
    return stats[0], kms / max(n, 1), stats


def _dma_trains(st, ks, vs, row_off, flush):
    """kv_gather_trains_dma on the current state: cold time, copies, the
    host's enqueue time, and bit equality with the gather kernel's rows."""
    import torch
    import non_uniform_paged_amd as nup
    ref_k, ref_v = ks.clone(), vs.clone()
    ks.zero_()
    vs.zero_()
    n = nup.kv_gather_trains_dma(st.ctx, ks, vs, row_off)
    torch.cuda.synchronize()
    same = bool(torch.equal(ks, ref_k) and torch.equal(vs, ref_v))
    del ref_k, ref_v
    enq = []

    def run():
        t0 = time.perf_counter()
        nup.kv_gather_trains_dma(st.ctx, ks, vs, row_off)
        enq.append(time.perf_counter() - t0)
    ms = _timed(run, 3, flush)
    nbytes = 2 * ks.shape[0] * ks.shape[1] * 2
    return {"copies": n, "ms": round(ms, 4), "GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "host_enqueue_ms": round(1e3 * float(np.mean(enq)), 3), "rows_equal_kernel": same}


def _centroid_sweep(flush, T=8192):
    """Centroid selection against the exact one on the Llama-3-8B shape, for
    2048, 4096 and 8192 centroids per KV head.  The keys have a structure of
    their own: every position belongs to one of T = 8192 true clusters and
    its key is that cluster's centre plus noise (bf16).  The clustering
    handed to the selection merges true clusters (ids equal mod C), and each
    centroid is the mean of its members' keys, so fewer centroids describe
    the keys more coarsely (KVDrive, Fig 18 / Fig 19: the number of
    centroids trades selection time against accuracy).  Reports the
    selection's time and the share of the exact selection's older entries
    it finds (the recent window, kept by both, is left out)."""
    import torch
    import non_uniform_paged_amd as nup
    import workloads as W
    w = W.llama3_8b_topk()
    st = Setup(w, 0)
    B, H, D, K = w.batch, w.num_kv_heads, w.head_dim, w.topk
    window = K // 2
    L = int(w.lengths[0, 0])
    gh = H // w.num_groups
    pt = nup.get_page_table(st.ctx)
    goh, soh = nup.get_groups(st.ctx)
    t = np.arange(L)
    exact = torch.empty((B, H, K), dtype=torch.int32, device="cuda")
    approx = torch.empty_like(exact)
    ws_sel = torch.empty(nup.select_workspace_bytes(st.ctx), dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(W.torch_seed("k", T))
    centre = torch.randn((B, H, T, D), generator=g, device="cuda")
    # keys: the true centre of each position plus noise, written through the page table
    true_of_pos, _, _ = W.nested_cluster_lists(w.lengths, T, T, salt=T)
    kflat = st.kpool.view(-1, D)
    keys_f = torch.empty((B, H, L, D), dtype=torch.float32, device="cuda")
    for s in range(B):
        for h in range(H):
            rows = (pt[goh[h], s, t // 16].astype(np.int64) * gh + soh[h]) * 16 + t % 16
            k = centre[s, h][torch.from_numpy(true_of_pos[s, h, :L].astype(np.int64)).cuda()]
            k += 0.5 * torch.randn(k.shape, generator=g, device="cuda")
            kb = k.to(torch.bfloat16)
            kflat[torch.from_numpy(rows).cuda()] = kb
            keys_f[s, h] = kb.float()
    torch.cuda.synchronize()
    nup.kv_select_topk(st.ctx, st.q, K, window, exact, ws_sel)
    e = exact.cpu().numpy()[..., :K - window]
    out = []
    for C in (2048, 4096, 8192):
        _, start, pos = W.nested_cluster_lists(w.lengths, T, C, salt=T)
        # each centroid: the mean of its members' keys (bf16)
        assign = torch.from_numpy((true_of_pos[..., :L] % C).astype(np.int64)).cuda()   # [B][H][L]
        sums = torch.zeros((B, H, C, D), dtype=torch.float32, device="cuda")
        sums.scatter_add_(2, assign[..., None].expand(B, H, L, D), keys_f)
        cnt = torch.bincount((assign + C * torch.arange(B * H, device="cuda").view(B, H, 1)).view(-1),
                             minlength=B * H * C).view(B, H, C, 1).clamp_(min=1)
        cent = (sums / cnt).to(torch.bfloat16)
        del sums, cnt, assign
        ws_c = torch.empty(nup.centroid_workspace_bytes(st.ctx, C), dtype=torch.uint8, device="cuda")
        cs, ps = torch.from_numpy(start).cuda(), torch.from_numpy(pos).cuda()
        sel = lambda: nup.kv_select_topk_centroids(st.ctx, st.q, cent, C, cs, ps, pos.shape[2], K, window,
                                                   approx, ws_c)
        sel()
        torch.cuda.synchronize()
        ms = _timed(sel, 10, flush)
        a = approx.cpu().numpy()[..., :K - window]
        recall = np.mean([len(np.intersect1d(e[s, h], a[s, h])) / (K - window)
                          for s in range(B) for h in range(H)])
        assert nup.device_errors(st.ctx) == nup.NUP_OK
        out.append({"centroids": C, "true_clusters": T, "select_ms": round(ms, 4),
                    "recall_of_exact_topk": round(float(recall), 4)})
        del cent, ws_c, cs, ps
    del keys_f, centre
    st.free()
    return out


def _layer_group_sweep(flush):
    """Reserved memory, page-table entries, host Reserve+commit time and the
    36-layer decode time for each head-group size on the 36-layer batch."""
    import torch
    import non_uniform_paged_amd as nup
    import workloads as W
    w = W.qwen3_4b_layers()
    NL, H, D, B = w.extra["num_layers"], w.num_kv_heads, w.head_dim, w.batch
    V = NL * H
    caps, lens = w.caps.astype(np.int32), w.lengths.astype(np.int32)
    max_pages = int(math.ceil(caps.max() / 16))
    used = int(lens.sum()) * 2 * D * 2
    out = []
    q = torch.empty((B, w.num_q_heads, D), dtype=torch.bfloat16, device="cuda")
    W.fill_normal_bf16_torch(q, "q")
    o = torch.empty((B, w.num_q_heads, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, w.num_q_heads), dtype=torch.float32, device="cuda")
    for G in (1, 2, 4, 8, 16, 32):
        ng = V // G
        cfg = dict(num_kv_heads=H, num_q_heads=w.num_q_heads, head_dim=D, num_groups=ng, max_batch=B,
                   max_pages=max_pages, num_layers=NL, merge_mode=MERGE_MODE)
        # exact page need from a host-only pager, then pools of that size
        probe = nup.Context(**cfg, num_pages=B * ng * max_pages)
        nup.kv_alloc_groups(probe, np.arange(B), caps, lens)
        pages = B * ng * max_pages - len(nup.get_free_list(probe))
        del probe
        kpool = torch.empty((pages, G, 16, D), dtype=torch.bfloat16, device="cuda")
        vpool = torch.empty_like(kpool)
        W.fill_normal_bf16_torch(kpool, "k")
        W.fill_normal_bf16_torch(vpool, "v")
        desc = torch.empty(nup.desc_bytes(**cfg, num_pages=pages), dtype=torch.uint8, device="cuda")
        ctx = nup.Context(**cfg, num_pages=pages, k_pool=kpool, v_pool=vpool, desc=desc)
        t0 = time.perf_counter()
        nup.kv_alloc_groups(ctx, np.arange(B), caps, lens)
        nup.nup_commit(ctx)
        host_us = (time.perf_counter() - t0) * 1e6
        ws = torch.empty(nup.workspace_bytes(ctx), dtype=torch.uint8, device="cuda")

        def step():
            for layer in range(NL):
                nup.set_layer(ctx, layer)
                nup.attn_decode_nonuniform(ctx, q, o, lse, 1.0 / math.sqrt(D), ws)
        step()
        torch.cuda.synchronize()
        ms = _timed(step, 5, flush)
        reserved = pages * G * 16 * 2 * D * 2
        out.append({"heads_per_group": G, "groups": ng, "groups_spanning_layers": G > H,
                    "reserved_GB": round(reserved / 1e9, 3),
                    "internal_fragmentation": round(1 - used / reserved, 4),
                    "page_table_entries": pages,
                    "host_reserve_commit_us": round(host_us, 1),
                    "decode_36_layers_ms": round(ms, 4),
                    "decode_GBs": round(used / (ms * 1e-3) / 1e9, 1)})
        del ctx, kpool, vpool, desc, ws
        torch.cuda.empty_cache()
    return out


def _graph_decode(flush, context, steps=10, warmup=2):
    """The 36-layer decode step (fused append + attention in every layer, 72
    launches; the three-launch form for comparison) issued call by call and
    replayed from a HIP graph captured once, each with and without a Trim +
    Reserve + commit of one session before every step.  Heads per group 8; the context sets the session
    lengths (16384: the Qwen3-4B batch; 1024: short sessions)."""
    import torch
    import non_uniform_paged_amd as nup
    import workloads as W
    w = W.qwen3_4b_layers(headroom=128, context=context)
    NL, H, Hq, D, B = w.extra["num_layers"], w.num_kv_heads, w.num_q_heads, w.head_dim, w.batch
    V, G = NL * H, 8
    ng = V // G
    caps, lens = w.caps.astype(np.int32), w.lengths.astype(np.int32)
    max_pages = int(math.ceil(caps.max() / 16))
    cfg = dict(num_kv_heads=H, num_q_heads=Hq, head_dim=D, num_groups=ng, max_batch=B,
               max_pages=max_pages, num_layers=NL, merge_mode=MERGE_MODE)
    probe = nup.Context(**cfg, num_pages=B * ng * max_pages)
    nup.kv_alloc_groups(probe, np.arange(B), caps, lens)
    pages = B * ng * max_pages - len(nup.get_free_list(probe))
    del probe
    kpool = torch.empty((pages, G, 16, D), dtype=torch.bfloat16, device="cuda")
    vpool = torch.empty_like(kpool)
    W.fill_normal_bf16_torch(kpool, "k")
    W.fill_normal_bf16_torch(vpool, "v")
    desc = torch.empty(nup.desc_bytes(**cfg, num_pages=pages), dtype=torch.uint8, device="cuda")
    ctx = nup.Context(**cfg, num_pages=pages, k_pool=kpool, v_pool=vpool, desc=desc)
    nup.kv_alloc_groups(ctx, np.arange(B), caps, lens)
    nup.nup_commit(ctx)
    ws = torch.empty(nup.workspace_bytes(ctx), dtype=torch.uint8, device="cuda")
    q = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    kn = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(kn)
    W.fill_normal_bf16_torch(q, "q")
    W.fill_normal_bf16_torch(kn, "k", 77)
    W.fill_normal_bf16_torch(vn, "v", 77)
    o = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    turn = [0]

    def churn():
        s = turn[0] % B
        turn[0] += 1
        nup.kv_free_seqs(ctx, [s])
        nup.kv_alloc_groups(ctx, [s], caps[s:s + 1], lens[s:s + 1])
        nup.nup_commit(ctx)

    def eager():
        for layer in range(NL):
            nup.set_layer(ctx, layer)
            nup.attn_decode_nonuniform_append(ctx, kn, vn, q, o, lse, scale, ws)

    def eager3():   # the same step as three launches per layer
        for layer in range(NL):
            nup.set_layer(ctx, layer)
            nup.kv_append(ctx, kn, vn)
            nup.attn_decode_nonuniform(ctx, q, o, lse, scale, ws)

    g = torch.cuda.CUDAGraph()

    def replay():
        g.replay()
        nup.note_appends(ctx, 1)

    def run(fn, with_churn):
        for _ in range(warmup):
            if with_churn:
                churn()
            fn()
        torch.cuda.synchronize()
        flush()
        e0 = _Event()
        e1 = _Event()
        host = 0.0
        e0.record()
        for _ in range(steps):
            t0 = time.perf_counter()
            if with_churn:
                churn()
            fn()
            host += time.perf_counter() - t0
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, host / steps * 1e6

    res = {"context": context, "batch": B, "heads_per_group": G, "launches_per_step": 2 * NL,
           "kv_GB_per_step": round(float(lens.astype(np.int64).sum()) * 2 * D * 2 / 1e9, 3)}
    res["eager_3_launches_ms"], res["eager_3_launches_host_us"] = run(eager3, False)
    res["eager_ms"], res["eager_host_us"] = run(eager, False)
    res["eager_churn_ms"], res["eager_churn_host_us"] = run(eager, True)
    with torch.cuda.graph(g):
        eager()
    res["graph_ms"], res["graph_host_us"] = run(replay, False)
    res["graph_churn_ms"], res["graph_churn_host_us"] = run(replay, True)
    for k in list(res):
        if isinstance(res[k], float):
            res[k] = round(res[k], 4 if k.endswith("_ms") else 1)
    del g, ctx, kpool, vpool, desc, ws
    torch.cuda.empty_cache()
    return res


EXTRA_SECTIONS = ("qwen3_4b", "llama3_8b_topk", "llama3_8b_centroids", "mixed_churn", "qwen25_32b_trains", "qwen25_32b_prefix",
                  "qwen3_4b_36_layers", "qwen3_4b_36_layers_graph", "qwen25_32b_heads_per_group")


def measure_extras(args, only=None):
    """The other configurations: attention on the Qwen3-4B shape, gather,
    selection and top-K attention on the Llama-3-8B shape, the mixed-length
    churn step (Trim / Reserve / commit on the host, trains, append,
    attention), trains by copy engines, forked sessions (Alias), head groups
    across 36 layers, and heads per group.  only: one name of
    EXTRA_SECTIONS, or None for all."""
    import torch
    import non_uniform_paged_amd as nup
    import workloads as W

    res = {}
    flush_w = torch.empty(1 << 28, dtype=torch.int32, device="cuda")
    # float32, so that the sum is one reduction over the buffer itself (an
    # int32 sum would first copy it out as int64)
    flush_r = torch.ones(1 << 28, dtype=torch.float32, device="cuda")

    def flush():
        # a cached 1 GiB write, then a cached 1 GiB read of other memory
        # (each four times the 256 MB MALL, and far beyond the L2s): what a
        # timed call reads next comes from HBM, and the write's dirty lines
        # have been written back during the read, before the timed call
        flush_w.fill_(1)
        flush_r.sum()

    def want(name):
        return only is None or only == name

    # -- Qwen3-4B-shaped layer: attention only, cold (caches flushed before each call) and warm
    if want("qwen3_4b"):
        w = W.qwen3_4b()
        st = Setup(w, 8)
        for _ in range(3):
            st.step(append=False)
        torch.cuda.synchronize()
        # cold calls (100 by default) timed after the warm-up above
        ms, kms, cst = _timed_call_and_kernel(st.ctx, lambda: st.step(append=False), args.cold_calls, flush)
        kb = algorithmic_bytes(st.lengths0, st.caps, w.batch, w.num_q_heads, w.num_kv_heads,
                               w.num_groups) - w.batch * w.num_q_heads * w.head_dim * 4
        # warm: 20 calls back to back per timed window, so that the GPU never
        # waits for the host between them; part of the 512 MiB stays in the
        # 256 MB MALL from call to call
        def batch20():
            for _ in range(20):
                st.step(append=False)
        reps = max(1, args.cold_calls // 20)
        wms = _timed(batch20, reps) / 20
        nup.kernel_time(st.ctx, reset=True)
        nup.set_timing(st.ctx, True)
        _timed(batch20, reps)
        nup.set_timing(st.ctx, False)
        wk_total, wn = nup.kernel_time(st.ctx, reset=True)
        wkms = wk_total / max(wn, 1)
        res["qwen3_4b"] = {"kv_bytes": kv_bytes(st.lengths0), "attn_call_ms": round(ms, 4),
                           **_med_p90(cst, "attn_call_ms"),
                           "tokens_per_s_per_step": round(w.batch / (cst[1] * 1e-3), 1),   # median call
                           "partial_kernel_ms": round(kms, 4),
                           "partial_kernel_GBs": round(kb / (kms * 1e-3) / 1e9, 1),
                           "frac": round(kb / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                           "warm_attn_call_ms": round(wms, 4), "warm_partial_kernel_ms": round(wkms, 4),
                           "warm_partial_kernel_GBs": round(kb / (wkms * 1e-3) / 1e9, 1),
                           "note": "cold: 1 GiB written, then 1 GiB read, through the caches before each "
                                   "call; warm: 20 calls back to back per timed window"}
        if not args.no_cpu_baseline:
            res["qwen3_4b"]["cpu_baseline"] = oracle_timing(st, oracle_spec(st))
            res["qwen3_4b"]["cpu_baseline"]["gpu_over_cpu"] = round(
                res["qwen3_4b"]["partial_kernel_GBs"] / res["qwen3_4b"]["cpu_baseline"]["value"], 1)
        st.free()
        del st

    # -- Llama-3-8B top-K: index gather into staging, then attention over it
    if want("llama3_8b_topk"):
        w = W.llama3_8b_topk()
        st = Setup(w, 0)
        K = w.topk
        idx = torch.from_numpy(W.topk_indices(w.lengths, K)).cuda()
        ks = torch.empty((w.batch, 8, K, 128), dtype=torch.bfloat16, device="cuda")
        vs = torch.empty_like(ks)
        ws = torch.empty(nup.workspace_bytes(st.ctx, K), dtype=torch.uint8, device="cuda")
        gather = lambda: nup.kv_gather_compact(st.ctx, 1, ks, vs, idx=idx, K=K)
        topk = lambda: nup.attn_decode_topk(st.ctx, st.q, ks, vs, K, st.out, st.lse, st.scale, ws)
        fused = lambda: nup.attn_decode_topk_paged(st.ctx, st.q, idx, K, st.out, st.lse, st.scale, ws)
        for _ in range(3):
            gather()
            topk()
            fused()
        rows = w.batch * 8 * K
        # cold calls (100 by default) of each
        gst = _timed_stats(gather, args.cold_calls, flush)
        tst = _timed_stats(topk, args.cold_calls, flush)
        g_ms, t_ms = gst[0], tst[0]
        f_ms, fk_ms, fst = _timed_call_and_kernel(st.ctx, fused, args.cold_calls, flush)
        both32 = _timed(lambda: [f() for _ in range(32) for f in (gather, topk)], 3) / 32
        fused32 = _timed(lambda: [fused() for _ in range(32)], 3) / 32
        # the same 32-layer stack captured in one HIP graph (launch cost amortised)
        gstream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gstream):
            fused()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=gstream):
            for _ in range(32):
                nup.attn_decode_topk_paged(st.ctx, st.q, idx, K, st.out, st.lse, st.scale, ws,
                                           stream=torch.cuda.current_stream())
        graph.replay()
        torch.cuda.synchronize()
        graph32 = _timed(graph.replay, 5) / 32
        # selection of the 2048 entries (1024 recent) from all 122880 positions
        sel_idx = torch.empty((w.batch, 8, K), dtype=torch.int32, device="cuda")
        ws_sel = torch.empty(nup.select_workspace_bytes(st.ctx), dtype=torch.uint8, device="cuda")
        select = lambda: nup.kv_select_topk(st.ctx, st.q, K, K // 2, sel_idx, ws_sel)
        select()
        s_ms = _timed(select, 5, flush)
        k_bytes = int(w.lengths.sum()) * 256
        gb = rows * 512 * 2 + rows * 4
        tb = rows * 512 + w.batch * 32 * 128 * (2 + 4)
        fb = rows * (512 + 4) + w.batch * 32 * 128 * 6
        res["llama3_8b_topk"] = {
            "gather_ms": round(g_ms, 4), **_med_p90(gst, "gather_ms"),
            "gather_GBs": round(gb / (g_ms * 1e-3) / 1e9, 1),
            "topk_attn_ms": round(t_ms, 4), **_med_p90(tst, "topk_attn_ms"),
            "topk_attn_GBs": round(tb / (t_ms * 1e-3) / 1e9, 1),
            "gather_plus_attn_ms_32_back_to_back": round(both32, 4),
            "topk_in_place_ms": round(f_ms, 4), **_med_p90(fst, "topk_in_place_ms"),
            "topk_in_place_GBs": round(fb / (f_ms * 1e-3) / 1e9, 1),
            "tokens_per_s_per_step": round(w.batch / (fst[1] * 1e-3), 1),   # over the median call
            "topk_in_place_partial_kernel_ms": round(fk_ms, 4),
            "frac": round(fb / (fk_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "topk_in_place_ms_32_back_to_back": round(fused32, 4),
            "topk_in_place_ms_32_layer_graph": round(graph32, 4),
            "select_ms": round(s_ms, 4),
            "select_score_GBs": round(k_bytes / (s_ms * 1e-3) / 1e9, 1),
            "note": "per call cold (1 GiB written, then 1 GiB read, through the caches before each); 32 "
                    "back-to-back pairs for a 32-layer stack; frac: the in-place call's split-K kernel"}
        if not args.no_cpu_baseline:
            cb = oracle_timing(st, oracle_spec(st), tokens=idx.cpu().numpy())
            cb["gpu_over_cpu"] = round(fb / (fk_ms * 1e-3) / 1e9 / cb["value"], 1)
            res["llama3_8b_topk"]["cpu_baseline"] = cb
        assert nup.device_errors(st.ctx) == nup.NUP_OK
        del graph
        st.free()
        del st, ks, vs, ws, sel_idx, ws_sel

    # -- centroid selection (KVDrive, Fig 18 / Fig 19): time and recall of the
    #    exact top-K with 2048, 4096 or 8192 centroids over keys drawn around
    #    8192 true cluster centres
    if want("llama3_8b_centroids"):
        res["llama3_8b_centroids"] = _centroid_sweep(flush)

    # -- mixed-length churn: 10% EOS per step, freed slots refilled next step
    if want("mixed_churn"):
        w = W.mixed_churn()
        # 20 warm-up steps, 20 with the library's kernel events (kernel time
        # and each step's bytes), then 20 without them (the step's GPU time:
        # every timing event adds GPU time between the launches it brackets)
        steps_warm, steps = 20, 20
        pad_steps = steps_warm + 2 * steps + 4
        st = Setup(w, pad_steps, max_pages=int(math.ceil((131072 + 16 * math.ceil((pad_steps + 1) / 16)) / 16)))
        # the oracle on the batch as first reserved (before any churn step)
        cpu = None if args.no_cpu_baseline else oracle_timing(st, oracle_spec(st))
        drv = W.ChurnDriver(w.batch)
        active = np.ones(w.batch, bool)
        freed = np.zeros(0, np.int32)
        host_us, trains, gpu_ms, step_kb, n_active = [], [], [], [], []
        all_kb = []   # every launch's K/V bytes, warm-up included (what a profiler averages over)
        timed_kb = []  # the step-timed steps' K/V bytes
        nup.kernel_time(st.ctx, reset=True)
        for it in range(steps_warm + 2 * steps):
            lib = 0.0   # host time inside the library: Reserve, Trim, frame commit
            if len(freed):
                L = drv.refill_lengths(len(freed))
                Ls = np.repeat(L[:, None], 8, axis=1).astype(np.int32)
                t0 = time.perf_counter()
                nup.kv_alloc_groups(st.ctx, freed, Ls + st.pad, Ls)
                lib += time.perf_counter() - t0
                active[freed] = True
            eos = drv.eos(np.nonzero(active)[0])
            t0 = time.perf_counter()
            nup.kv_free_seqs(st.ctx, eos)
            nup.nup_commit(st.ctx)
            lib += time.perf_counter() - t0
            active[eos] = False
            freed = eos
            kern = steps_warm <= it < steps_warm + steps       # kernel-timed steps
            timed = it >= steps_warm + steps                    # step-timed steps
            if kern or timed:
                host_us.append(lib * 1e6)
                trains.append(len(nup.get_runs(st.ctx)))
            if kern:
                nup.set_timing(st.ctx, True)
            if timed:
                n_active.append(int(active.sum()))
                e0 = _Event()
                e1 = _Event()
                e0.record()
            nup.attn_decode_nonuniform_append(st.ctx, st.k_new, st.v_new, st.q, st.out, st.lse, st.scale, st.ws)
            # the call advanced the shadow lengths by the appended token,
            # which the step also reads: these are the step's K/V bytes
            all_kb.append(kv_bytes(nup.get_lengths(st.ctx)))
            if kern:
                nup.set_timing(st.ctx, False)
                step_kb.append(all_kb[-1])
            if timed:
                e1.record()
                timed_kb.append(all_kb[-1])
            torch.cuda.synchronize()
            if timed:
                gpu_ms.append(e0.elapsed_time(e1))
        kms_total, n = nup.kernel_time(st.ctx, reset=True)
        assert n == len(step_kb), (n, len(step_kb))
        kms = kms_total / max(n, 1)
        L_now = nup.get_lengths(st.ctx)
        # train-mode gather of the final state
        lens = L_now.astype(np.int64).reshape(-1)
        row_off = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)[:-1]])).cuda()
        total = int(lens.sum())
        ksg = torch.empty((total, 128), dtype=torch.bfloat16, device="cuda")
        vsg = torch.empty_like(ksg)
        gt = lambda: nup.kv_gather_compact(st.ctx, 0, ksg, vsg, row_off=row_off)
        gt()
        g_ms = _timed(gt, 5, flush)
        dma = None if args.no_copy_engine else _dma_trains(st, ksg, vsg, row_off.cpu().numpy(), flush)
        res["mixed_churn"] = {
            "active_slots": int(active.sum()),
            "kv_bytes_per_step_mean": int(np.mean(step_kb)),
            "kv_bytes_per_step_range": [int(min(step_kb)), int(max(step_kb))],
            "kv_bytes_all_launches_mean": int(np.mean(all_kb)),
            "host_trim_reserve_commit_us_mean": round(float(np.mean(host_us)), 1),
            "gpu_append_attn_ms_mean": round(float(np.mean(gpu_ms)), 4),
            "step_kv_bytes_mean": int(np.mean(timed_kb)),
            "step_GBs": round(float(np.mean(timed_kb)) / (float(np.mean(gpu_ms)) * 1e-3) / 1e9, 1),
            "submit_share": round(float(np.mean(host_us)) / (float(np.mean(host_us)) + 1e3 * float(np.mean(gpu_ms))), 4),
            "trains_per_step_mean": round(float(np.mean(trains)), 1),
            "pages_in_use": int(st.num_pages - len(nup.get_free_list(st.ctx))),
            "tokens_per_s_per_step": round(float(np.mean(n_active)) / (float(np.mean(gpu_ms)) * 1e-3), 1),
            "partial_kernel_ms": round(kms, 4),
            "partial_kernel_GBs": round(sum(step_kb) / (kms_total * 1e-3) / 1e9, 1),
            "frac": round(sum(step_kb) / (kms_total * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "cpu_baseline": None if cpu is None else dict(
                cpu, gpu_over_cpu=round(sum(step_kb) / (kms_total * 1e-3) / 1e9 / cpu["value"], 1)),
            "gather_trains_ms": round(g_ms, 4),
            "gather_trains_GBs": round(2 * total * 512 / (g_ms * 1e-3) / 1e9, 1),
            "gather_trains_copy_engine": dma}
        st.free()
        del st, ksg, vsg
        torch.cuda.empty_cache()

    # -- the Qwen2.5-32B batch (long trains): gather kernel vs copy engines,
    #    with one head per group (linear copies) and with the 4-group layout
    if want("qwen25_32b_trains"):
        res["qwen25_32b_trains"] = []
        for ng in (8, 4):
            w = W.qwen25_32b()
            w.num_groups = ng
            st = Setup(w, 0)
            lens = st.lengths0.astype(np.int64).reshape(-1)
            ro = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
            total = int(lens.sum())
            ksg = torch.empty((total, 128), dtype=torch.bfloat16, device="cuda")
            vsg = torch.empty_like(ksg)
            ro_dev = torch.from_numpy(ro).cuda()
            gt = lambda: nup.kv_gather_compact(st.ctx, 0, ksg, vsg, row_off=ro_dev)
            gt()
            g_ms = _timed(gt, 5, flush)
            res["qwen25_32b_trains"].append({
                "heads_per_group": 8 // ng, "trains": int(len(nup.get_runs(st.ctx))), "bytes": 2 * total * 256,
                "gather_kernel_ms": round(g_ms, 4),
                "gather_kernel_GBs": round(2 * total * 512 / (g_ms * 1e-3) / 1e9, 1),
                "copy_engine": None if args.no_copy_engine else _dma_trains(st, ksg, vsg, ro, flush)})
            st.free()
            del st, ksg, vsg, ro_dev
            torch.cuda.empty_cache()

    # -- forked sessions sharing a prompt prefix (KV-RM Alias): same lengths as
    #    the Qwen2.5-32B batch, 60 of 64 sessions fork from 4 sources; the
    #    unshared batch is timed the same way for comparison
    if want("qwen25_32b_prefix"):
        res["qwen25_32b_prefix"] = {}
        for tag, w, mode in (("unshared", W.qwen25_32b(), nup.PLAN_BALANCED),
                             ("forked", W.qwen25_32b_prefix(), nup.PLAN_BALANCED),
                             ("forked_shared_plan", W.qwen25_32b_prefix(), nup.PLAN_SHARED)):
            st = Setup(w, 0, plan_mode=mode)
            for _ in range(2):
                st.step(append=False)
            torch.cuda.synchronize()
            call_ms, kms, _ = _timed_call_and_kernel(st.ctx, lambda: st.step(append=False), 10, flush)
            in_use = int(st.num_pages - len(nup.get_free_list(st.ctx)))
            entries = int(np.count_nonzero(nup.get_page_table(st.ctx) >= 0))
            kb = kv_bytes(st.lengths0)
            share = getattr(st, "share", None)
            shared_b = 0 if share is None else int(sum(int(share[i, st.goh[h]]) * 16 * 512
                                                       for i in range(len(share)) for h in range(w.num_kv_heads)))
            res["qwen25_32b_prefix"][tag] = {
                "pages_in_use": in_use, "page_table_entries": entries,
                "reserved_saving": round(1 - in_use / entries, 4),
                "kv_bytes_logical": kb, "kv_bytes_unique": kb - shared_b,
                "attn_call_ms": round(call_ms, 4),
                "partial_kernel_ms": round(kms, 4),
                "partial_kernel_logical_GBs": round(kb / (kms * 1e-3) / 1e9, 1)}
            st.free()
            del st
            torch.cuda.empty_cache()
        res["qwen25_32b_prefix"]["note"] = ("prefix 8192 tokens, 4 sources; cold (1 GiB written, then 1 GiB "
                                            "read, before each step); logical bytes count every session's reads")

    # -- head groups across layers (Tangram, Fig 11): the 36-layer Qwen3-4B
    #    shape in one pager, heads per group 1 .. 32 (groups beyond 8 span layers)
    if want("qwen3_4b_36_layers"):
        res["qwen3_4b_36_layers"] = _layer_group_sweep(flush)

    # -- the same 36-layer step replayed from a HIP graph captured once, with
    #    Trim / Reserve / commit between replays (KV-RM: a static-graph
    #    decoder over one committed descriptor per step)
    if want("qwen3_4b_36_layers_graph"):
        res["qwen3_4b_36_layers_graph"] = [_graph_decode(flush, 16384), _graph_decode(flush, 1024)]

    # -- heads per page (Tangram, Fig 8c): the Qwen2.5-32B batch with 1, 2, 4, 8 groups
    if want("qwen25_32b_heads_per_group"):
        sweep = []
        for ng in (8, 4, 2, 1):
            w = W.qwen25_32b()
            w.num_groups = ng
            gh = 8 // ng
            st = Setup(w, 8)
            reserved_slots = (st.num_pages - len(nup.get_free_list(st.ctx))) * 16 * gh
            used = int(st.lengths0.sum())
            for _ in range(2):
                st.step(append=False)
            torch.cuda.synchronize()
            nup.kernel_time(st.ctx, reset=True)
            nup.set_timing(st.ctx, True)
            _timed(lambda: st.step(append=False), 10)
            nup.set_timing(st.ctx, False)
            kms, n = nup.kernel_time(st.ctx, reset=True)
            kms /= max(n, 1)
            sweep.append({"heads_per_group": gh, "groups": ng,
                          "reserved_GB": round(reserved_slots * 512 / 1e9, 3),
                          "internal_fragmentation": round(1 - used / reserved_slots, 4),
                          "page_table_entries": int(st.num_pages - len(nup.get_free_list(st.ctx))),
                          "partial_kernel_ms": round(kms, 4),
                          "partial_kernel_GBs": round(kv_bytes(st.lengths0) / (kms * 1e-3) / 1e9, 1)})
            st.free()
            del st
            torch.cuda.empty_cache()
        res["qwen25_32b_heads_per_group"] = sweep
    del flush_w, flush_r
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-calls", type=int, default=100,
                    help="timed calls per figure of the Qwen3-4B and Llama top-K configurations")
    ap.add_argument("--no-controls", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other configurations (Qwen3-4B, Llama top-K, mixed churn)")
    ap.add_argument("--workers", type=int, default=0)
    ap.add_argument("--unfused", action="store_true",
                    help="time the step as kv_append + attn_decode_nonuniform (three launches)")
    ap.add_argument("--no-copy-engine", action="store_true",
                    help="skip the copy-engine train measurements (thousands of copies)")
    ap.add_argument("--only-extra", choices=EXTRA_SECTIONS, default=None,
                    help="run just this one of the other configurations and print its JSON")
    ap.add_argument("--probe-copy", type=int, default=0, metavar="BYTES",
                    help="only run the plain streaming copy kernel over BYTES (counter "
                         "calibration and achievable-bandwidth ceiling), then exit")
    ap.add_argument("--merge", choices=["auto", "launch", "split"], default="auto",
                    help="where split heads' partials are merged: the library's choice, a merge "
                         "launch, or inside the split-K launch")
    args = ap.parse_args()
    global MERGE_MODE
    MERGE_MODE = {"auto": 0, "launch": 1, "split": 2}[args.merge]
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the path would shard by sequence or head group "
                                   "with no exchange between GPUs, but no multi-GPU run is provided",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import non_uniform_paged_amd as nup  # noqa: F401  (fails loudly when not built)
    import workloads as W

    if args.probe_copy:
        n = args.probe_copy // 16 * 16
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(2):
            nup.probe_copy(a, b, n)
        torch.cuda.synchronize()
        e0 = _Event()
        e1 = _Event()
        reps = 5
        e0.record()
        for _ in range(reps):
            nup.probe_copy(a, b, n)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        print(json.dumps({"probe_copy_bytes": n, "ms": round(ms, 4),
                          "read_plus_write_GBs": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return

    if args.only_extra:
        print(json.dumps({"extra": args.only_extra,
                          "result": measure_extras(args, only=args.only_extra)[args.only_extra]}), flush=True)
        return

    src = open(os.path.join(ROOT, "non_uniform_paged_amd", "csrc", "kernels.hip"), "rb").read()
    sha = hashlib.sha256(src).hexdigest()

    w = W.qwen25_32b()
    headroom = 2 * args.warmup + 4 * args.steps + 8
    st = Setup(w, headroom, num_workers=args.workers)
    ms, mean_L, kms, kmean_L = time_steps(st, args.steps, args.warmup, fused=not args.unfused)
    B, Hq, H, D, ng = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_groups
    step_bytes = algorithmic_bytes(mean_L, st.caps, B, Hq, H, ng) + B * H * D * 2 * 2 * 2
    kern_bytes = algorithmic_bytes(kmean_L, st.caps, B, Hq, H, ng) - B * Hq * D * 4
    value = step_bytes / (ms * 1e-3) / 1e9
    achieved = kern_bytes / (kms * 1e-3) / 1e9
    extra = {"kv_bytes_per_step": kv_bytes(mean_L), "partial_kernel_ms": round(kms, 4),
             "pct_of_peak_step": round(100 * value / PEAK_HBM_GBS, 2)}

    extra["step_launches"] = 3 if args.unfused else 2
    ratio, nw = plan_straggler(st.ctx, nup.get_lengths(st.ctx))
    extra["straggler_balanced"] = {"max_over_mean_pages": round(ratio, 3), "workers": nw}
    if not args.no_controls:
        # the distribution of single steps, in a pass of its own (an event
        # between steps keeps them from overlapping, so these run slower)
        step_ms = []
        time_steps(st, args.steps, 0, fused=not args.unfused, per_step=step_ms, kernel=False)
        extra["single_step_ms_median"] = round(float(np.median(step_ms)), 4)
        extra["single_step_ms_p90"] = round(float(np.percentile(step_ms, 90)), 4)
        # the other form of the same step on the same batch (a few tokens longer)
        oms, oL, _, _ = time_steps(st, args.steps, args.warmup, fused=args.unfused, kernel=False)
        ob = algorithmic_bytes(oL, st.caps, B, Hq, H, ng) + B * H * D * 2 * 2 * 2
        tag = "fused" if args.unfused else "unfused_3_launches"
        extra[f"{tag}_ms_per_step"] = round(oms, 4)
        extra[f"{tag}_step_GBs"] = round(ob / (oms * 1e-3) / 1e9, 1)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(st)
    st.free()
    del st

    if not args.no_controls:
        # Uniform-budget control on the same contexts (keep 50% of every head):
        # the gate compares the non-uniform kernel's bytes/s with this one's.
        for tag, ctl in (("uniform50", "uniform50"), ("uniform_mean", "uniform_mean")):
            wc = W.qwen25_32b(control=ctl)
            sc = Setup(wc, headroom, num_workers=args.workers)
            _, _, ckms, cL = time_steps(sc, max(10, args.steps // 2), args.warmup)
            cb = algorithmic_bytes(cL, sc.caps, B, Hq, H, ng) - B * Hq * D * 4
            extra[f"control_{tag}_kernel_GBs"] = round(cb / (ckms * 1e-3) / 1e9, 1)
            extra[f"control_{tag}_kernel_ms"] = round(ckms, 4)
            sc.free()
            del sc
        extra["nonuniform_over_uniform50"] = round(achieved / extra["control_uniform50_kernel_GBs"], 4)
        # the uniform split Tangram measures against (every head cut into 8
        # chunks, one per worker) on the same non-uniform batch
        su = Setup(w, headroom, plan_mode=nup.PLAN_UNIFORM, uniform_splits=8)
        _, _, ukms, uL = time_steps(su, max(10, args.steps // 2), args.warmup)
        ub = algorithmic_bytes(uL, su.caps, B, Hq, H, ng) - B * Hq * D * 4
        extra["control_uniform_split_kernel_ms"] = round(ukms, 4)
        extra["control_uniform_split_kernel_GBs"] = round(ub / (ukms * 1e-3) / 1e9, 1)
        ratio, nw = plan_straggler(su.ctx, nup.get_lengths(su.ctx))
        extra["straggler_uniform_split"] = {"max_over_mean_pages": round(ratio, 3), "workers": nw}
        su.free()
        del su

    # achievable streaming-read ceiling on this device (4 GiB, beyond the caches)
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    nup.probe_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    e0 = _Event()
    e1 = _Event()
    e0.record()
    for _ in range(5):
        nup.probe_read(buf, nbytes, sink)
    e1.record()
    torch.cuda.synchronize()
    extra["read_ceiling_GBs"] = round(5 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    extra["partial_over_read_ceiling"] = round(achieved / extra["read_ceiling_GBs"], 4)
    del buf

    if not args.no_extras:
        extra["configs"] = measure_extras(args)

    # the pages' own figures, with the hardware they state: context only,
    # none measures this path
    extra["pages_context"] = [
        {"system": "Tangram", "figure": "up to 2.6x end-to-end serving throughput over existing baselines",
         "hardware": "not stated on the page"},
        {"system": "KVDrive", "figure": "up to 1.74x generation throughput over offloading systems",
         "hardware": "an A100 instance (roofline figure) and an L20 server (throughput figure)"},
        {"system": "KV-RM", "figure": "higher mixed-length throughput, lower tail latency, less reserved KV "
                                      "memory (no numbers on the page)",
         "hardware": "a node with 2 NVIDIA A100-40GB PCIe"}]
    if cpu is not None:
        cpu["gpu_over_cpu"] = round(achieved / cpu["value"], 1)
    traffic = traffic_from_profiles(sha)
    line = {
        "metric": "decode-attn achieved HBM GB/s (% of peak) + tokens/s/step, 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "tokens_per_s_per_step": round(B / (ms * 1e-3), 1),
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Qwen2.5-32B-shaped multi-turn decode layer: 64 sessions, 40 q / 8 KV "
                               "heads, head_dim 128, contexts U[8192,65536], keep ratio Beta(0.5,2) "
                               "per KV head, 4 head groups, 16-token pages",
                   "kv_dtype": "bf16", "batch": B, "kv_bytes": kv_bytes(mean_L),
                   "step": ("kv_append + nup_commit + attn_decode_nonuniform (append, partial, merge)"
                            if args.unfused else
                            "nup_commit + attn_decode_nonuniform_append (partial with the append, merge)")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": "partial_attn_kernel<128,5,0,false>"},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
