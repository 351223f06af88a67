"""Top-K selection through key clusters (KVDrive, Fig 18 / Fig 19):
kv_select_topk_centroids against the oracle's centroid selection."""
import math

import numpy as np
import pytest
import torch

import non_uniform_paged_amd as nup
import oracle
import workloads as W
from oracle import pager as pg
from oracle import select as osel
from tests.gpu_common import DEV, Case, assert_attention_close, u16
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _run(c, q, cent_bits, start, pos, K, window):
    C, P = cent_bits.shape[2], pos.shape[2]
    out = torch.full((c.B, c.H, K), -5, dtype=torch.int32, device=DEV)
    ws = torch.empty(nup.centroid_workspace_bytes(c.ctx, C), dtype=torch.uint8, device=DEV)
    cent = _dev(cent_bits.view(np.int16)).view(torch.bfloat16)
    nup.kv_select_topk_centroids(c.ctx, q, cent, C, _dev(start), _dev(pos), P, K, window, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _want(c, q, cent_bits, start, pos, K, window, s, h):
    gqa = c.Hq // c.H
    cs = osel.centroid_scores(u16(q), cent_bits, s, h, gqa)
    st = start[s, h]
    return osel.select_clusters(cs, st, pos[s, h], int(c.spec.lengths[s, h]), K, window), cs


def test_centroid_select_exact_inputs():
    """Integer centroid entries and q picking one dimension: every cluster
    score is exact in fp32, ties included; the selection equals the
    oracle's bit for bit."""
    B, H, gqa, D = 3, 4, 2, 128
    L = np.array([[300, 257, 64, 129], [512, 96, 400, 33], [0, 0, 0, 0]], np.int32)
    max_pages = 33
    c = Case(H=H, Hq=H * gqa, D=D, ng=2, B=B, num_pages=B * 2 * max_pages, max_pages=max_pages, salt=70)
    c.alloc([0, 1], L[:2], L[:2])                      # slot 2 inactive
    c.commit()
    rs = np.random.default_rng(70)
    qf = np.zeros((B, H * gqa, D), np.float32)
    qf[:, 0::2, 3], qf[:, 0::2, 5] = 1.0, 0.5
    qf[:, 1::2, 3], qf[:, 1::2, 5] = -0.25, 2.0
    c.q.copy_(_dev(f32_to_bf16_bits(qf).view(np.int16)).view(torch.bfloat16))
    for C in (1, 7, 64, 5000, 8192):      # up to the largest C: most lists empty
        cf = np.zeros((B, H, C, D), np.float32)
        cf[..., 3] = rs.integers(-4, 5, size=(B, H, C))
        cf[..., 5] = rs.integers(-4, 5, size=(B, H, C))
        cb = f32_to_bf16_bits(cf)
        start, pos = W.cluster_lists(np.maximum(L, 1), C, salt=70 + C)
        for K, window in ((32, 8), (33, 0), (20, 20), (1, 0)):
            got = _run(c, c.q, cb, start, pos, K, window)
            assert (got[2] == -5).all()
            for s in (0, 1):
                for h in range(H):
                    want, _ = _want(c, c.q, cb, start, pos, K, window, s, h)
                    assert got[s, h].tolist() == want.tolist(), (C, K, window, s, h)
    assert nup.device_errors(c.ctx) == nup.NUP_OK


def test_centroid_select_random_and_malformed():
    B, H, gqa, D, C = 2, 8, 4, 64, 200
    L = np.array([[1000, 2000, 3000, 700, 1500, 2500, 900, 1200]] * B, np.int32)
    max_pages = int(math.ceil(L.max() / 16))
    c = Case(H=H, Hq=H * gqa, D=D, ng=4, B=B, num_pages=B * 4 * max_pages, max_pages=max_pages, salt=71)
    c.alloc([0, 1], L, L)
    c.commit()
    cb = W.normal_bf16("k", (B, H, C, D), 71)
    start, pos = W.cluster_lists(L, C, salt=71)
    K, window = 256, 64
    got = _run(c, c.q, cb, start, pos, K, window)
    checked = 0
    for s in range(B):
        for h in range(H):
            want, cs = _want(c, c.q, cb, start, pos, K, window, s, h)
            # the fp32 and fp64 cluster orders can differ only where two scores
            # are closer than fp32 tells apart; only the cut cluster's
            # neighbours in that order decide the selection
            n = int(L[s, h]) - window
            order = np.lexsort((np.arange(C), -cs))
            st, ps = start[s, h], pos[s, h]
            below = np.array([np.sum(ps[st[k]:st[k + 1]] < n) for k in range(C)])
            cut = int(np.argmax(np.cumsum(below[order]) >= K - window))
            near = [abs(cs[order[i]] - cs[order[i + 1]]) for i in (cut - 1, cut) if 0 <= i < C - 1]
            if min(near, default=1.0) > 1e-4 * max(1.0, float(np.abs(cs).max())):
                assert got[s, h].tolist() == want.tolist(), (s, h)
                checked += 1
            g = got[s, h]
            assert (np.diff(g) > 0).all() and g[-window:].tolist() == list(range(L[s, h] - window, L[s, h]))
    assert checked >= 12
    assert nup.device_errors(c.ctx) == nup.NUP_OK
    # malformed lists for one head: offsets out of range -> error latched, -1 entries;
    # a head whose clusters cover too few positions -> the same; the others unchanged
    bad_start = start.copy()
    bad_start[0, 2, 5] = pos.shape[2] + 10
    short_start = bad_start.copy()
    short_start[1, 4, 1:] = 3                          # cluster 0 keeps 3 members, the rest are empty
    got2 = _run(c, c.q, cb, short_start, pos, K, window)
    assert nup.device_errors(c.ctx) == nup.NUP_E_INDEX
    for (s, h) in ((0, 2), (1, 4)):
        assert (got2[s, h, :K - window] == -1).all()
        assert got2[s, h, K - window:].tolist() == list(range(L[s, h] - window, L[s, h]))
    keep = [(s, h) for s in range(B) for h in range(H) if (s, h) not in ((0, 2), (1, 4))]
    for (s, h) in keep:
        assert got2[s, h].tolist() == got[s, h].tolist()


def _cut_is_clear(cs, st, ps, L, K, window, rel=1e-4):
    """Whether fp32 and fp64 must agree on a head's cluster selection: the
    clusters next to the cut cluster in score order are further apart than
    fp32 tells apart (elsewhere both selections are correct)."""
    C = len(cs)
    n = int(L) - window
    order = np.lexsort((np.arange(C), -cs))
    below = np.array([np.sum(ps[st[k]:st[k + 1]] < n) for k in range(C)])
    cut = int(np.argmax(np.cumsum(below[order]) >= K - window))
    near = [abs(cs[order[i]] - cs[order[i + 1]]) for i in (cut - 1, cut) if 0 <= i < C - 1]
    return min(near, default=1.0) > rel * max(1.0, float(np.abs(cs).max()))


def test_full_size_llama_centroid_select_then_attend():
    """Llama-3-8B shape, 2048 clusters per KV head over 122880 positions:
    select 2048 entries (1024 recent), then attend in place.  Every head's
    selection has the required structure and equals the oracle's wherever
    the cut is clear of fp32 near-ties; every head's attention is compared
    with the oracle's attention over the GPU's own (valid) index list."""
    w = W.llama3_8b_topk()
    c = Case(H=w.num_kv_heads, Hq=w.num_q_heads, D=w.head_dim, ng=w.num_groups, B=w.batch,
             num_pages=w.num_pages, max_pages=int(math.ceil(w.caps.max() / 16)),
             free_list_init=w.free_list_init, salt=72)
    c.alloc(list(range(w.batch)), w.caps, w.lengths)
    c.commit()
    C, K, window = 2048, w.topk, w.topk // 2
    cb = W.normal_bf16("k", (w.batch, 8, C, w.head_dim), 72)
    start, pos = W.cluster_lists(w.lengths, C, salt=72)
    got = _run(c, c.q, cb, start, pos, K, window)
    idx = _dev(got)
    ws = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
    nup.attn_decode_topk_paged(c.ctx, c.q, idx, K, c.out, c.lse, c.scale, ws)
    torch.cuda.synchronize()
    assert nup.device_errors(c.ctx) == nup.NUP_OK
    clear = 0
    for s in range(w.batch):
        for h in range(8):
            L = int(c.spec.lengths[s, h])
            g = got[s, h]
            assert (np.diff(g) > 0).all() and g[0] >= 0 and g[-1] < L, (s, h)
            assert g[K - window:].tolist() == list(range(L - window, L)), (s, h)
            # every older entry is a member of some cluster
            members = pos[s, h][:start[s, h][-1]]
            assert np.isin(g[:K - window], members).all(), (s, h)
            want, cs = _want(c, c.q, cb, start, pos, K, window, s, h)
            if _cut_is_clear(cs, start[s, h], pos[s, h], L, K, window):
                assert g.tolist() == want.tolist(), (s, h)
                clear += 1
    assert clear >= 56                     # a near-tie at the cut is rare
    ref, ref_lse = c.oracle(tokens=got)
    out = c.out.cpu().numpy().astype(np.float64)
    lse = c.lse.cpu().numpy().astype(np.float64)
    assert_attention_close(out, lse, ref, ref_lse, "centroid select + in-place attention, every head")
