"""GPU parity: every kernel of the path against the oracle, through the C ABI.

Attention: max-abs <= 1e-2 and rel-L2 <= 5e-3 against the fp64 oracle (and
rel-L2 <= 1e-4 as a bug detector).  Page tables, appended rows, gathered
rows and their physical row ids: bit-exact.
"""
import gc
import math

import numpy as np
import pytest
import torch

import non_uniform_paged_amd as nup
import oracle
import workloads as W
from oracle import pager as pg
from tests.gpu_common import (DEV, Case, assert_attention_close, u16)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _cleanup():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _ragged(seed, B, H, maxL, p_zero=0.1, p_one=0.1):
    rs = np.random.default_rng(seed)
    L = rs.integers(2, maxL + 1, size=(B, H))
    L[rs.random((B, H)) < p_zero] = 0
    L[rs.random((B, H)) < p_one] = 1
    caps = L + rs.integers(0, 40, size=(B, H))
    return L.astype(np.int32), caps.astype(np.int32)


def test_tiny_config():
    w = W.tiny()
    c = Case(H=4, Hq=4, D=64, ng=2, B=2, num_pages=64, max_pages=16,
             free_list_init=w.free_list_init)
    c.alloc([0, 1], w.caps, w.lengths)
    c.commit()
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert_attention_close(out, lse, ref, ref_lse, "tiny")


@pytest.mark.parametrize("D,gqa,H,ng,workers,seed", [
    (64, 1, 4, 2, 5, 1), (64, 2, 4, 1, 64, 2), (128, 4, 8, 4, 13, 3), (128, 5, 8, 4, 31, 4),
    (128, 8, 4, 2, 9, 5), (128, 5, 8, 2, 2048, 6), (128, 4, 8, 1, 1, 7), (64, 5, 8, 8, 17, 8)])
def test_ragged_shapes(D, gqa, H, ng, workers, seed):
    B = 5
    L, caps = _ragged(seed, B, H, 300)
    max_pages = int(math.ceil(caps.max() / 16)) + 1
    rs = np.random.default_rng(seed + 100)
    num_pages = B * ng * max_pages + 7
    c = Case(H=H, Hq=H * gqa, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages,
             free_list_init=rs.permutation(num_pages), num_workers=workers, salt=seed)
    c.alloc([4, 0, 2, 3], caps[:4], L[:4])      # slot 1 stays inactive
    c.commit()
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert_attention_close(out, lse, ref, ref_lse, f"D{D} gqa{gqa} ng{ng} W{workers}")


def test_long_skewed_head():
    """One head at the 131072-token clip among short ones: split over many
    workers, merged exactly."""
    H, gqa, D, B = 8, 4, 128, 2
    L = np.full((B, H), 48, np.int32)
    L[1, 3] = 131072
    L[0, 0] = 5
    caps = L.copy()
    max_pages = 131072 // 16
    num_pages = 2 * 2 * max_pages
    c = Case(H=H, Hq=H * gqa, D=D, ng=2, B=B, num_pages=num_pages, max_pages=max_pages,
             num_workers=512, salt=9)
    c.alloc([0, 1], caps, L)
    c.commit()
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert_attention_close(out, lse, ref, ref_lse, "long head")


def test_two_million_token_head():
    """One head of 2,097,152 tokens (131072 pages, page ids past 2^17, the
    head split over every worker and merged from about 2000 rows) next to
    short and empty heads, with a fused append at the end of the long head."""
    H, gqa, D, B = 4, 2, 64, 2
    L = np.array([[2 * 1024 * 1024 - 1, 40, 0, 17], [3, 1, 900, 64]], np.int32)
    caps = L + 1
    max_pages = 2 * 1024 * 1024 // 16
    num_pages = max_pages + 200
    c = Case(H=H, Hq=H * gqa, D=D, ng=H, B=B, num_pages=num_pages, max_pages=max_pages,
             num_workers=2048, salt=19)
    assert c.alloc([0, 1], caps, L) == pg.OK
    c.commit()
    kp, vp = u16(c.kpool).copy(), u16(c.vpool).copy()
    kn = W.normal_bf16("k", (B, H, D), 191)
    vn = W.normal_bf16("v", (B, H, D), 191)
    nup.attn_decode_nonuniform_append(c.ctx, torch.from_numpy(kn.view(np.int16)).to(DEV),
                                      torch.from_numpy(vn.view(np.int16)).to(DEV), c.q, c.out, c.lse,
                                      c.scale, c.ws)
    torch.cuda.synchronize()
    fk, fv = kp.reshape(-1, D), vp.reshape(-1, D)
    for s_ in range(B):
        for h in range(H):
            row = c.spec.physical_row(s_, h, int(c.spec.lengths[s_, h]))
            fk[row], fv[row] = kn[s_, h], vn[s_, h]
            c.spec.lengths[s_, h] += 1
    assert np.array_equal(nup.get_lengths(c.ctx), c.spec.lengths)
    assert np.array_equal(u16(c.kpool), kp) and np.array_equal(u16(c.vpool), vp)
    ref, ref_lse = oracle.decode(u16(c.q), kp, vp, c.spec.page_table, c.spec.lengths, c.spec.group_of_head,
                                 c.spec.slot_of_head, c.scale)
    assert_attention_close(c.out.cpu().numpy().astype(np.float64), c.lse.cpu().numpy().astype(np.float64),
                           ref, ref_lse, "2M-token head")


def test_length_one_returns_v_bit_exact():
    H, gqa, D, B = 8, 5, 128, 3
    L = np.ones((B, H), np.int32)
    c = Case(H=H, Hq=H * gqa, D=D, ng=4, B=B, num_pages=64, max_pages=2, num_workers=11, salt=10)
    c.alloc([0, 1, 2], L + 16, L)
    c.commit()
    out, _ = c.attend()
    vp = u16(c.vpool)
    for s in range(B):
        for r in range(H * gqa):
            h = r // gqa
            page = c.spec.page_table[c.spec.group_of_head[h], s, 0]
            v0 = W.bf16_bits_to_f64(vp[page, c.spec.slot_of_head[h], 0])
            assert np.array_equal(out[s, r], v0)


def test_page_permutation_bit_identical():
    H, gqa, D, B = 8, 4, 128, 4
    L, caps = _ragged(11, B, H, 500, p_zero=0, p_one=0)
    max_pages = int(math.ceil(caps.max() / 16))
    num_pages = B * 2 * max_pages + 3
    a = Case(H=H, Hq=H * gqa, D=D, ng=2, B=B, num_pages=num_pages, max_pages=max_pages,
             num_workers=37, salt=11)
    b = Case(H=H, Hq=H * gqa, D=D, ng=2, B=B, num_pages=num_pages, max_pages=max_pages,
             num_workers=37, salt=11,
             free_list_init=np.random.default_rng(5).permutation(num_pages))
    for x in (a, b):
        x.alloc(list(range(B)), caps, L)
        x.commit()
    pa = torch.from_numpy(a.spec.page_table[a.spec.page_table >= 0].astype(np.int64)).to(DEV)
    pb = torch.from_numpy(b.spec.page_table[b.spec.page_table >= 0].astype(np.int64)).to(DEV)
    b.kpool[pb] = a.kpool[pa]
    b.vpool[pb] = a.vpool[pa]
    oa, la = a.attend()
    ob, lb = b.attend()
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_split_invariance():
    H, gqa, D, B = 8, 5, 128, 3
    L, caps = _ragged(12, B, H, 900, p_zero=0)
    max_pages = int(math.ceil(caps.max() / 16))
    outs = []
    for workers in (1, 3, 64, 2048):
        c = Case(H=H, Hq=H * gqa, D=D, ng=4, B=B, num_pages=B * 4 * max_pages,
                 max_pages=max_pages, num_workers=workers, salt=12)
        c.alloc(list(range(B)), caps, L)
        c.commit()
        out, lse = c.attend()
        ref, ref_lse = c.oracle()
        assert_attention_close(out, lse, ref, ref_lse, f"W={workers}")
        outs.append(out)
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 1e-5


def test_uniform_plan_mode():
    H, gqa, D, B = 8, 4, 128, 4
    L, caps = _ragged(13, B, H, 700)
    max_pages = int(math.ceil(caps.max() / 16))
    c = Case(H=H, Hq=H * gqa, D=D, ng=4, B=B, num_pages=B * 4 * max_pages, max_pages=max_pages,
             plan_mode=nup.PLAN_UNIFORM, uniform_splits=3, salt=13)
    c.alloc(list(range(B)), caps, L)
    c.commit()
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert_attention_close(out, lse, ref, ref_lse, "uniform plan")


def test_append_then_decode():
    """Decode steps: append one token per active head, commit, attend.  The
    pool after the appends equals the oracle's placement bit-exactly."""
    H, gqa, D, B = 8, 4, 128, 3
    L, _ = _ragged(14, B, H, 60, p_zero=0.2, p_one=0.2)
    caps = L + 12
    max_pages = int(math.ceil(caps.max() / 16))
    num_pages = B * 2 * max_pages + 5
    c = Case(H=H, Hq=H * gqa, D=D, ng=2, B=B, num_pages=num_pages, max_pages=max_pages,
             free_list_init=np.random.default_rng(3).permutation(num_pages), num_workers=19,
             salt=14)
    c.alloc([0, 2], caps[[0, 2]], L[[0, 2]])   # slot 1 inactive
    c.commit()
    kp = u16(c.kpool).copy()
    vp = u16(c.vpool).copy()
    flat_k = kp.reshape(-1, D)
    flat_v = vp.reshape(-1, D)
    for step in range(10):
        kn = W.normal_bf16("k", (B, H, D), 1000 + step)
        vn = W.normal_bf16("v", (B, H, D), 1000 + step)
        nup.kv_append(c.ctx, torch.from_numpy(kn.view(np.int16)).to(DEV),
                      torch.from_numpy(vn.view(np.int16)).to(DEV))
        st, pos = c.spec.append_positions()
        assert st == pg.OK
        for s in range(B):
            if not c.spec.active[s]:
                continue
            for h in range(H):
                row = c.spec.physical_row(s, h, int(pos[s, h]))
                flat_k[row] = kn[s, h]
                flat_v[row] = vn[s, h]
        c.commit()
        assert np.array_equal(nup.get_lengths(c.ctx), c.spec.lengths)
    out, lse = c.attend()
    assert np.array_equal(u16(c.kpool), kp) and np.array_equal(u16(c.vpool), vp)
    ref, ref_lse = oracle.decode(u16(c.q), kp, vp, c.spec.page_table, c.spec.lengths,
                                 c.spec.group_of_head, c.spec.slot_of_head, c.scale)
    assert_attention_close(out, lse, ref, ref_lse, "after appends")


def test_append_errors():
    H, D, B = 4, 64, 2
    c = Case(H=H, Hq=H, D=D, ng=1, B=B, num_pages=8, max_pages=2, salt=15)
    c.alloc([0], np.array([[20, 20, 20, 20]]), np.array([[3, 20, 0, 1]]))
    kn = torch.zeros((B, H, D), dtype=torch.bfloat16, device=DEV)
    # edits pending: commit first
    assert nup.kv_append(c.ctx, kn, kn, raise_on_error=False) == nup.NUP_E_STATE
    c.commit()
    # head 1 is at its budget: nothing is written, nothing advances
    assert nup.kv_append(c.ctx, kn, kn, raise_on_error=False) == nup.NUP_E_CAPACITY
    assert nup.get_lengths(c.ctx)[0].tolist() == [3, 20, 0, 1]
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert_attention_close(out, lse, ref, ref_lse, "after refused append")


def test_all_slots_inactive():
    """Every slot ended (Reserve then Trim of all): attention writes zeros and
    -inf for every head, the gathers and the selection write nothing, an
    append is a no-op, and the next Reserve works on the returned pages."""
    H, gqa, D, B = 4, 2, 64, 3
    c = Case(H=H, Hq=H * gqa, D=D, ng=2, B=B, num_pages=40, max_pages=8, salt=19)
    caps = np.full((B, H), 100, np.int32)
    c.alloc([0, 1, 2], caps, caps - 3)
    c.commit()
    c.free([0, 1, 2])
    c.commit()
    out, lse = c.attend()
    assert (out == 0).all() and np.isneginf(lse).all()
    kn = torch.zeros((B, H, D), dtype=torch.bfloat16, device=DEV)
    before = u16(c.kpool).copy()
    nup.kv_append(c.ctx, kn, kn)
    assert np.array_equal(u16(c.kpool), before)
    ks = torch.full((64, D), -3, dtype=torch.int16, device=DEV)
    nup.kv_gather_compact(c.ctx, 0, ks, ks, row_off=torch.zeros(B * H, dtype=torch.int64, device=DEV))
    assert nup.kv_gather_trains_dma(c.ctx, ks, ks, np.zeros(B * H, np.int64)) == 0
    idx = torch.zeros((B, H, 8), dtype=torch.int32, device=DEV)
    nup.kv_gather_compact(c.ctx, 1, ks, ks, idx=idx, K=8)
    sel = torch.full((B, H, 8), -5, dtype=torch.int32, device=DEV)
    ws = torch.empty(nup.select_workspace_bytes(c.ctx), dtype=torch.uint8, device=DEV)
    nup.kv_select_topk(c.ctx, c.q, 8, 2, sel, ws)
    torch.cuda.synchronize()
    assert (ks.cpu().numpy() == -3).all() and (sel.cpu().numpy() == -5).all()
    assert nup.device_errors(c.ctx) == nup.NUP_OK
    assert len(nup.get_free_list(c.ctx)) == 40
    c.alloc([1], caps[:1], caps[:1] - 50)
    c.commit()
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert_attention_close(out, lse, ref, ref_lse, "after the pool emptied and refilled")


def test_shadow_edits_invisible_until_commit():
    H, gqa, D, B = 8, 4, 128, 4
    L, caps = _ragged(16, B, H, 200, p_zero=0)
    max_pages = int(math.ceil(caps.max() / 16))
    c = Case(H=H, Hq=H * gqa, D=D, ng=2, B=B, num_pages=B * 2 * max_pages, max_pages=max_pages,
             num_workers=23, salt=16)
    c.alloc([0, 1, 2], caps[:3], L[:3])
    c.commit()
    ref, ref_lse = c.oracle()
    # edit the shadow without committing: the kernels keep the committed frame
    c.free([1])
    c.alloc([3], caps[3:], L[3:])
    out, lse = c.attend()
    assert_attention_close(out, lse, ref, ref_lse, "pre-commit view")
    c.commit()
    out, lse = c.attend()
    ref2, ref_lse2 = c.oracle()
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert_attention_close(out, lse, ref2, ref_lse2, "post-commit view")


def _gather_case(seed, B=3, H=8, gqa=4, D=128, ng=1, maxL=700):
    rs = np.random.default_rng(seed)
    L = rs.integers(300, maxL, size=(B, H)).astype(np.int32)
    caps = L + 16
    max_pages = int(math.ceil(caps.max() / 16))
    num_pages = B * ng * max_pages + 9
    c = Case(H=H, Hq=H * gqa, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages,
             free_list_init=rs.permutation(num_pages), num_workers=29, salt=seed)
    return c, L, caps


def test_gather_index_and_topk_attention():
    c, L, caps = _gather_case(17)
    B, H, D, K = c.B, c.H, c.D, 96
    c.alloc([0, 2], caps[[0, 2]], L[[0, 2]])   # slot 1 inactive
    c.commit()
    lens = np.where(c.spec.active[:, None], c.spec.lengths, 300)
    idx = W.topk_indices(lens, K, salt=17)
    d_idx = torch.from_numpy(idx).to(DEV)
    ks = torch.full((B, H, K, D), 7, dtype=torch.int16, device=DEV)
    vs = torch.full_like(ks, 7)
    phys = torch.full((B, H, K), -7, dtype=torch.int32, device=DEV)
    nup.kv_gather_compact(c.ctx, 1, ks, vs, idx=d_idx, K=K, phys_out=phys)
    torch.cuda.synchronize()
    assert nup.device_errors(c.ctx) == nup.NUP_OK
    sk, sv, sphys = pg.gather_index(c.spec, u16(c.kpool), u16(c.vpool), idx)
    gk = ks.cpu().numpy().view(np.uint16)
    gv = vs.cpu().numpy().view(np.uint16)
    gp = phys.cpu().numpy()
    for s in (0, 2):
        assert np.array_equal(gk[s], sk[s]) and np.array_equal(gv[s], sv[s])
        assert np.array_equal(gp[s], sphys[s])
    assert (gk[1] == 7).all() and (gp[1] == -7).all()     # inactive rows untouched
    ws = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
    nup.attn_decode_topk(c.ctx, c.q, ks.view(torch.bfloat16), vs.view(torch.bfloat16), K,
                         c.out, c.lse, c.scale, ws)
    torch.cuda.synchronize()
    out = c.out.cpu().numpy().astype(np.float64)
    lse = c.lse.cpu().numpy().astype(np.float64)
    ref, ref_lse = c.oracle(tokens=idx)
    assert_attention_close(out, lse, ref, ref_lse, "top-K")


@pytest.mark.parametrize("K", [1, 16, 37])
def test_topk_ragged_k(K):
    c, L, caps = _gather_case(18 + K, B=2, gqa=5, ng=2)
    c.alloc([0, 1], caps, L)
    c.commit()
    idx = W.topk_indices(c.spec.lengths, max(K, 2), salt=18)[..., :K].copy()
    idx.sort(axis=-1)
    ks = torch.zeros((c.B, c.H, K, c.D), dtype=torch.int16, device=DEV)
    vs = torch.zeros_like(ks)
    nup.kv_gather_compact(c.ctx, 1, ks, vs, idx=torch.from_numpy(idx).to(DEV), K=K)
    ws = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
    nup.attn_decode_topk(c.ctx, c.q, ks.view(torch.bfloat16), vs.view(torch.bfloat16), K,
                         c.out, c.lse, c.scale, ws)
    torch.cuda.synchronize()
    assert nup.device_errors(c.ctx) == nup.NUP_OK
    ref, ref_lse = c.oracle(tokens=idx)
    assert_attention_close(c.out.cpu().numpy().astype(np.float64),
                           c.lse.cpu().numpy().astype(np.float64), ref, ref_lse, f"K={K}")


def test_gather_index_rejects_bad_indices():
    c, L, caps = _gather_case(19, B=2, H=4, gqa=1, D=64)
    c.alloc([0, 1], caps, L)
    c.commit()
    K = 8
    idx = np.tile(np.arange(K, dtype=np.int32) * 3, (2, 4, 1))
    idx[0, 1, 5] = idx[0, 1, 4]          # repeated
    idx[1, 2, 7] = L[1, 2]               # past the retained length
    idx[1, 3, 0] = -1                    # negative
    ks = torch.full((2, 4, K, 64), 9, dtype=torch.int16, device=DEV)
    vs = torch.full_like(ks, 9)
    nup.kv_gather_compact(c.ctx, 1, ks, vs, idx=torch.from_numpy(idx).to(DEV), K=K)
    assert nup.device_errors(c.ctx) == nup.NUP_E_INDEX
    assert nup.device_errors(c.ctx) == nup.NUP_OK        # latched word was cleared
    gk = ks.cpu().numpy().view(np.uint16)
    for (s, h, k) in ((0, 1, 5), (1, 2, 7), (1, 3, 0)):
        assert (gk[s, h, k] == 0).all()
    good = idx.copy()
    good[0, 1, 5] = good[0, 1, 4] + 1
    good[1, 2, 7] = 0
    good[1, 3, 0] = 0
    sk, _, _ = pg.gather_index(c.spec, u16(c.kpool), u16(c.vpool), np.clip(good, 0, None))
    assert np.array_equal(gk[0, 0], sk[0, 0]) and np.array_equal(gk[1, 1], sk[1, 1])


def test_gather_trains_bit_exact():
    c, L, caps = _gather_case(20, B=4, H=8, ng=2)
    c.alloc([0, 1, 3], caps[[0, 1, 3]], L[[0, 1, 3]])
    c.free([1])
    c.alloc([2], caps[[2]], L[[2]])      # reuses freed pages: trains break up
    c.commit()
    lens = c.spec.lengths.astype(np.int64)
    row_off = np.concatenate([[0], np.cumsum(lens.reshape(-1))[:-1]]).astype(np.int64)
    total = int(lens.sum())
    ks = torch.zeros((total, c.D), dtype=torch.int16, device=DEV)
    vs = torch.zeros_like(ks)
    phys = torch.full((total,), -1, dtype=torch.int32, device=DEV)
    nup.kv_gather_compact(c.ctx, 0, ks, vs, row_off=torch.from_numpy(row_off).to(DEV),
                          phys_out=phys)
    torch.cuda.synchronize()
    want = pg.gather_pages(c.spec, u16(c.kpool), u16(c.vpool), row_off)
    gk = ks.cpu().numpy().view(np.uint16)
    gv = vs.cpu().numpy().view(np.uint16)
    gp = phys.cpu().numpy()
    H = c.H
    for (s, h), (kr, vr, rows) in want.items():
        o = row_off[s * H + h]
        n = len(kr)
        assert np.array_equal(gk[o:o + n], kr) and np.array_equal(gv[o:o + n], vr)
        assert np.array_equal(gp[o:o + n], rows)
    runs = nup.get_runs(c.ctx)
    assert [tuple(r) for r in runs.tolist()] == pg.coalesce(c.spec.page_table, c.spec.n_pages,
                                                             c.spec.active)


# ---- full-size configurations, every output value checked ------------------

def _full_case(w, num_workers=0, max_pages=None):
    max_pages = max_pages or int(math.ceil(w.caps.max() / 16))
    return Case(H=w.num_kv_heads, Hq=w.num_q_heads, D=w.head_dim, ng=w.num_groups, B=w.batch,
                num_pages=w.num_pages, max_pages=max_pages, free_list_init=w.free_list_init,
                num_workers=num_workers)


def _physical_rows(spec, idx):
    """Physical row id of every entry of idx [B][H][K] (logical positions),
    from the oracle pager's page table: page * G_h * P + slot * P + t % P."""
    B, H, K = idx.shape
    g = spec.group_of_head[np.arange(H)][None, :, None]
    s = np.arange(B)[:, None, None]
    page = spec.page_table[g, s, idx // 16].astype(np.int64)
    return (page * spec.g_h + spec.slot_of_head[np.arange(H)][None, :, None]) * 16 + idx % 16


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen25_32b", "qwen25_32b_uniform50"])
def test_full_size_whole_output(name):
    """The bench's launch configuration at full size; every sequence and
    every query head is compared with the oracle."""
    if name == "qwen25_32b_uniform50":
        w = W.qwen25_32b(control="uniform50")
    else:
        w = W.CONFIGS[name]()
    c = _full_case(w)
    c.alloc(list(range(w.batch)), w.caps, w.lengths)
    c.commit()
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert_attention_close(out, lse, ref, ref_lse, name)


def test_full_size_llama_topk():
    """Llama-3-8B shape: index gather (every row and physical id) and the
    attention over the staging, every output value against the oracle."""
    w = W.llama3_8b_topk()
    c = _full_case(w)
    c.alloc(list(range(w.batch)), w.caps, w.lengths)
    c.commit()
    K = w.topk
    idx = W.topk_indices(w.lengths, K)
    ks = torch.empty((w.batch, 8, K, 128), dtype=torch.bfloat16, device=DEV)
    vs = torch.empty_like(ks)
    phys = torch.empty((w.batch, 8, K), dtype=torch.int32, device=DEV)
    nup.kv_gather_compact(c.ctx, 1, ks, vs, idx=torch.from_numpy(idx).to(DEV), K=K, phys_out=phys)
    ws = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
    nup.attn_decode_topk(c.ctx, c.q, ks, vs, K, c.out, c.lse, c.scale, ws)
    torch.cuda.synchronize()
    assert nup.device_errors(c.ctx) == nup.NUP_OK
    want = _physical_rows(c.spec, idx)
    assert np.array_equal(phys.cpu().numpy(), want)
    wt = torch.from_numpy(want.reshape(-1)).to(DEV)
    for pool, st in ((c.kpool, ks), (c.vpool, vs)):
        rows = pool.view(-1, 128).index_select(0, wt)
        assert torch.equal(rows.view(torch.int16), st.reshape(-1, 128).view(torch.int16))
    ref, ref_lse = c.oracle(tokens=idx)
    out = c.out.cpu().numpy().astype(np.float64)
    lse = c.lse.cpu().numpy().astype(np.float64)
    assert_attention_close(out, lse, ref, ref_lse, "llama top-K")


def test_full_size_mixed_churn():
    w = W.mixed_churn()
    c = _full_case(w, max_pages=int(math.ceil((131072 + 16) / 16)))
    drv = W.ChurnDriver(w.batch)
    c.alloc(list(range(w.batch)), w.caps, w.lengths)
    c.commit()
    freed = np.zeros(0, np.int32)
    for step in range(6):
        if len(freed):
            L = drv.refill_lengths(len(freed))
            Ls = np.repeat(L[:, None], 8, axis=1)
            assert c.alloc(freed, Ls + 16, Ls) == pg.OK
        active = np.nonzero(c.spec.active)[0]
        freed = drv.eos(active)
        c.free(freed)
        c.commit()
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert_attention_close(out, lse, ref, ref_lse, "mixed churn")
    for s in freed:
        assert np.all(out[s] == 0) and np.all(np.isneginf(lse[s]))


def test_repeated_launches_bit_identical():
    """No device state carries over from one launch to the next: repeated
    launches, interleaved paged and top-K calls, give identical results."""
    c, L, caps = _gather_case(21, B=3, H=8, gqa=5, ng=4)
    c.alloc([0, 1, 2], caps, L)
    c.commit()
    K = 64
    idx = W.topk_indices(c.spec.lengths, K, salt=21)
    ks = torch.zeros((c.B, c.H, K, c.D), dtype=torch.int16, device=DEV)
    vs = torch.zeros_like(ks)
    nup.kv_gather_compact(c.ctx, 1, ks, vs, idx=torch.from_numpy(idx).to(DEV), K=K)
    ws_k = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
    first = None
    for it in range(4):
        out, lse = c.attend()
        if first is None:
            first = (out, lse)
            ref, ref_lse = c.oracle()
            assert_attention_close(out, lse, ref, ref_lse, "repeat")
        else:
            assert np.array_equal(out, first[0]) and np.array_equal(lse, first[1]), f"launch {it}"
        nup.attn_decode_topk(c.ctx, c.q, ks.view(torch.bfloat16), vs.view(torch.bfloat16), K,
                             c.out, c.lse, c.scale, ws_k)
    torch.cuda.synchronize()


@pytest.mark.parametrize("K,gqa,ng,seed", [(96, 4, 1, 30), (37, 5, 2, 31), (16, 1, 4, 32), (1, 8, 2, 33)])
def test_topk_paged_matches_oracle(K, gqa, ng, seed):
    """Top-K attention read in place through indices and page tables."""
    c, L, caps = _gather_case(seed, B=3, H=8, gqa=gqa, ng=ng)
    c.alloc([0, 2], caps[[0, 2]], L[[0, 2]])      # slot 1 inactive
    c.commit()
    lens = np.where(c.spec.active[:, None], c.spec.lengths, 300)
    idx = W.topk_indices(lens, max(K, 2), salt=seed)[..., :K].copy()
    idx.sort(axis=-1)
    ws = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
    nup.attn_decode_topk_paged(c.ctx, c.q, torch.from_numpy(idx).to(DEV), K, c.out, c.lse, c.scale, ws)
    torch.cuda.synchronize()
    assert nup.device_errors(c.ctx) == nup.NUP_OK
    ref, ref_lse = c.oracle(tokens=idx)
    assert_attention_close(c.out.cpu().numpy().astype(np.float64), c.lse.cpu().numpy().astype(np.float64),
                           ref, ref_lse, f"topk paged K={K}")


def test_topk_paged_masks_bad_entries():
    """An entry outside the retained range is left out and latched; an
    out-of-order entry is read and latched."""
    c, L, caps = _gather_case(34, B=2, H=4, gqa=2, ng=2, maxL=500)
    c.alloc([0, 1], caps, L)
    c.commit()
    K = 40
    idx = W.topk_indices(c.spec.lengths, K, salt=34)
    bad = idx.copy()
    bad[1, 2, 17] = c.spec.lengths[1, 2] + 3           # past the retained length
    ws = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
    nup.attn_decode_topk_paged(c.ctx, c.q, torch.from_numpy(bad).to(DEV), K, c.out, c.lse, c.scale, ws)
    torch.cuda.synchronize()
    assert nup.device_errors(c.ctx) == nup.NUP_E_INDEX
    out = c.out.cpu().numpy().astype(np.float64)
    lse = c.lse.cpu().numpy().astype(np.float64)
    ref, ref_lse = c.oracle(tokens=idx)
    gqa = c.Hq // c.H
    keep = np.ones(out.shape[:2], bool)
    keep[1, 2 * gqa:3 * gqa] = False
    assert_attention_close(out[keep], lse[keep], ref[keep], ref_lse[keep], "unaffected heads")
    # the affected head equals attention over its other K-1 entries
    sub = np.delete(idx, 17, axis=2)                    # every head's list minus entry 17
    sub[1, 2] = np.delete(idx[1, 2], 17)
    r2, l2 = c.oracle(tokens=sub)
    assert_attention_close(out[1, 2 * gqa:3 * gqa], lse[1, 2 * gqa:3 * gqa], r2[1, 2 * gqa:3 * gqa],
                           l2[1, 2 * gqa:3 * gqa], "masked entry")
    # an out-of-order list is still read, and latched
    swapped = idx.copy()
    swapped[0, 0, [3, 4]] = swapped[0, 0, [4, 3]]
    nup.attn_decode_topk_paged(c.ctx, c.q, torch.from_numpy(swapped).to(DEV), K, c.out, c.lse, c.scale, ws)
    torch.cuda.synchronize()
    assert nup.device_errors(c.ctx) == nup.NUP_E_INDEX
    assert np.isfinite(c.out.cpu().numpy()).all()


def test_full_size_llama_topk_paged_equals_staged():
    """Llama-3-8B shape: the in-place top-K attention equals the oracle on
    every output value and the staged path (gather, then attend) bit for bit."""
    w = W.llama3_8b_topk()
    c = _full_case(w)
    c.alloc(list(range(w.batch)), w.caps, w.lengths)
    c.commit()
    K = w.topk
    idx_h = W.topk_indices(w.lengths, K)
    idx = torch.from_numpy(idx_h).to(DEV)
    ws = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
    nup.attn_decode_topk_paged(c.ctx, c.q, idx, K, c.out, c.lse, c.scale, ws)
    torch.cuda.synchronize()
    out_p = c.out.cpu().numpy().copy()
    lse_p = c.lse.cpu().numpy().copy()
    ks = torch.empty((w.batch, 8, K, 128), dtype=torch.bfloat16, device=DEV)
    vs = torch.empty_like(ks)
    nup.kv_gather_compact(c.ctx, 1, ks, vs, idx=idx, K=K)
    nup.attn_decode_topk(c.ctx, c.q, ks, vs, K, c.out, c.lse, c.scale, ws)
    torch.cuda.synchronize()
    assert nup.device_errors(c.ctx) == nup.NUP_OK
    assert np.array_equal(out_p, c.out.cpu().numpy()) and np.array_equal(lse_p, c.lse.cpu().numpy())
    ref, ref_lse = c.oracle(tokens=idx_h)
    assert_attention_close(out_p.astype(np.float64), lse_p.astype(np.float64), ref, ref_lse,
                           "llama top-K in place")


# ---- top-K selection ------------------------------------------------------

from oracle import select as osel  # noqa: E402


def _check_selection(got, spec, q, pool_k, K, window, heads, eps=1e-3):
    """got: int32 [B][H][K] from the GPU.  Structure always; membership against
    the fp64 oracle outside a margin around its threshold (fp32 scores can
    order near-ties differently)."""
    for (s, h) in heads:
        g = got[s, h]
        L = int(spec.lengths[s, h])
        assert (np.diff(g) > 0).all() and g[0] >= 0 and g[-1] < L, (s, h)
        assert g[K - window:].tolist() == list(range(L - window, L)), (s, h)
        sc = osel.scores(q, pool_k, spec, s, h)
        want = osel.select(sc, K, window)
        if K == window:
            continue
        cand = sc[: L - window]
        thr = np.sort(cand)[::-1][K - window - 1]
        sure = np.abs(cand - thr) > eps * max(1.0, abs(thr))
        gs = np.zeros(L - window, bool)
        gs[g[: K - window]] = True
        ws_ = np.zeros(L - window, bool)
        ws_[want[: K - window]] = True
        assert np.array_equal(gs[sure], ws_[sure]), (s, h)
        assert gs.sum() == ws_.sum()


@pytest.mark.parametrize("plan_mode", [nup.PLAN_BALANCED, nup.PLAN_UNIFORM])
def test_select_topk_exact_ties(plan_mode):
    """Exactly representable scores with many ties: the GPU selection equals
    the oracle's bit for bit (ties to the lower position), whichever plan the
    score kernel walks."""
    B, H, gqa, D = 2, 4, 2, 128
    L = np.array([[300, 257, 64, 129], [512, 96, 400, 33]], np.int32)
    max_pages = 33
    c = Case(H=H, Hq=H * gqa, D=D, ng=2, B=B, num_pages=B * 2 * max_pages, max_pages=max_pages,
             num_workers=13, salt=40, plan_mode=plan_mode, uniform_splits=3)
    c.alloc([0, 1], L, L)
    c.commit()
    # keys: dims 3 and 5 carry small integers (many repeats), all else zero
    rs = np.random.default_rng(40)
    kp = torch.zeros_like(c.kpool, dtype=torch.float32)
    kp[:, :, :, 3] = torch.from_numpy(rs.integers(-4, 5, size=kp.shape[:3]).astype(np.float32)).to(DEV)
    kp[:, :, :, 5] = torch.from_numpy(rs.integers(-4, 5, size=kp.shape[:3]).astype(np.float32)).to(DEV)
    c.kpool.copy_(kp.to(torch.bfloat16))
    qf = torch.zeros((B, H * gqa, D), dtype=torch.float32)
    qf[:, 0::2, 3] = 1.0
    qf[:, 0::2, 5] = 0.5
    qf[:, 1::2, 3] = -0.25
    qf[:, 1::2, 5] = 2.0
    c.q.copy_(qf.to(torch.bfloat16).to(DEV))
    for K, window in ((32, 8), (33, 0), (20, 20), (1, 0)):
        out = torch.full((B, H, K), -5, dtype=torch.int32, device=DEV)
        ws = torch.empty(nup.select_workspace_bytes(c.ctx), dtype=torch.uint8, device=DEV)
        nup.kv_select_topk(c.ctx, c.q, K, window, out, ws)
        torch.cuda.synchronize()
        want, _ = osel.select_all(u16(c.q), u16(c.kpool), c.spec, K, window)
        assert np.array_equal(out.cpu().numpy(), want), (K, window)


def test_select_topk_long_rows():
    """Few workers and long heads, so that a score-kernel row spans several
    staged segments of 512 pages (and ends in a partial one); exactly
    representable scores with ties, so the selection equals the oracle's
    bit for bit."""
    B, H, gqa, D = 1, 2, 2, 128
    L = np.array([[20000, 13001]], np.int32)
    max_pages = int(math.ceil(L.max() / 16)) + 1
    c = Case(H=H, Hq=H * gqa, D=D, ng=1, B=B, num_pages=B * max_pages + 7, max_pages=max_pages,
             num_workers=2, salt=42)
    c.alloc([0], L, L)
    c.commit()
    rs = np.random.default_rng(42)
    kp = torch.zeros_like(c.kpool, dtype=torch.float32)
    kp[:, :, :, 3] = torch.from_numpy(rs.integers(-8, 9, size=kp.shape[:3]).astype(np.float32)).to(DEV)
    kp[:, :, :, 5] = torch.from_numpy(rs.integers(-8, 9, size=kp.shape[:3]).astype(np.float32)).to(DEV)
    c.kpool.copy_(kp.to(torch.bfloat16))
    qf = torch.zeros((B, H * gqa, D), dtype=torch.float32)
    qf[:, 0::2, 3], qf[:, 0::2, 5] = 1.0, 0.5
    qf[:, 1::2, 3], qf[:, 1::2, 5] = -0.25, 2.0
    c.q.copy_(qf.to(torch.bfloat16).to(DEV))
    rows, ws_, _ = nup.get_plan(c.ctx)
    assert (rows[:, 2] - rows[:, 1]).max() > 2 * 512 * 16   # a row of three segments
    for K, window in ((64, 16), (1500, 100)):
        out = torch.full((B, H, K), -5, dtype=torch.int32, device=DEV)
        ws = torch.empty(nup.select_workspace_bytes(c.ctx), dtype=torch.uint8, device=DEV)
        nup.kv_select_topk(c.ctx, c.q, K, window, out, ws)
        torch.cuda.synchronize()
        want, _ = osel.select_all(u16(c.q), u16(c.kpool), c.spec, K, window)
        assert np.array_equal(out.cpu().numpy(), want), (K, window)


def test_select_topk_random_and_refused_cases():
    c, L, caps = _gather_case(41, B=3, H=8, gqa=5, ng=4)
    c.alloc([0, 2], caps[[0, 2]], L[[0, 2]])
    c.commit()
    K, window = 128, 32
    out = torch.full((c.B, c.H, K), -5, dtype=torch.int32, device=DEV)
    ws = torch.empty(nup.select_workspace_bytes(c.ctx), dtype=torch.uint8, device=DEV)
    nup.kv_select_topk(c.ctx, c.q, K, window, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got[1] == -5).all()                     # inactive slot untouched
    _check_selection(got, c.spec, u16(c.q), u16(c.kpool), K, window,
                     [(s, h) for s in (0, 2) for h in range(c.H)])
    # more entries than some head retains: refused on the host
    assert nup.kv_select_topk(c.ctx, c.q, int(L.max()) + 1, 0, out, ws,
                              raise_on_error=False) == nup.NUP_E_ARG
    assert nup.kv_select_topk(c.ctx, c.q, 8, 9, out, ws, raise_on_error=False) == nup.NUP_E_ARG


def test_select_topk_threshold_bin_beyond_lds():
    """More than 8192 older entries share the threshold's top key bits (all
    scores tie at 0 except a few): the select finishes with passes over the
    scores instead of in LDS, and still takes the lowest tied positions."""
    B, H, D = 1, 2, 64
    L = np.array([[12000, 20000]], np.int32)
    max_pages = 1250
    c = Case(H=H, Hq=H, D=D, ng=1, B=B, num_pages=2 * max_pages, max_pages=max_pages,
             num_workers=17, salt=42)
    c.alloc([0], L, L)
    c.commit()
    kp = torch.zeros_like(c.kpool, dtype=torch.float32)
    # a few keys with a positive score, scattered; everything else scores 0
    rs = np.random.default_rng(42)
    pt = c.spec.page_table
    for h in range(H):
        for t in rs.choice(int(L[0, h]) - 100, 40, replace=False):
            page = pt[c.spec.group_of_head[h], 0, t // 16]
            kp[page, c.spec.slot_of_head[h], t % 16, 0] = float(1 + t % 7)
    c.kpool.copy_(kp.to(torch.bfloat16))
    qf = torch.zeros((B, H, D), dtype=torch.float32)
    qf[:, :, 0] = 1.0
    c.q.copy_(qf.to(torch.bfloat16).to(DEV))
    for K, window in ((300, 50), (9000, 100)):
        out = torch.full((B, H, K), -5, dtype=torch.int32, device=DEV)
        ws = torch.empty(nup.select_workspace_bytes(c.ctx), dtype=torch.uint8, device=DEV)
        nup.kv_select_topk(c.ctx, c.q, K, window, out, ws)
        torch.cuda.synchronize()
        want, _ = osel.select_all(u16(c.q), u16(c.kpool), c.spec, K, window)
        assert np.array_equal(out.cpu().numpy(), want), (K, window)


def test_full_size_llama_select_then_attend():
    """Llama-3-8B shape: select 2048 entries (1024 recent) per KV head from
    122880, then attend in place.  Every head's selection is checked against
    the oracle's outside a margin around its threshold (fp32 and fp64 scores
    may order near-ties differently, so several selections are correct);
    every head's attention is then compared with the oracle's attention over
    the GPU's own (valid) index list."""
    w = W.llama3_8b_topk()
    c = _full_case(w)
    c.alloc(list(range(w.batch)), w.caps, w.lengths)
    c.commit()
    K, window = w.topk, w.topk // 2
    idx = torch.empty((w.batch, 8, K), dtype=torch.int32, device=DEV)
    ws_sel = torch.empty(nup.select_workspace_bytes(c.ctx), dtype=torch.uint8, device=DEV)
    nup.kv_select_topk(c.ctx, c.q, K, window, idx, ws_sel)
    ws = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
    nup.attn_decode_topk_paged(c.ctx, c.q, idx, K, c.out, c.lse, c.scale, ws)
    torch.cuda.synchronize()
    assert nup.device_errors(c.ctx) == nup.NUP_OK
    got = idx.cpu().numpy()
    out = c.out.cpu().numpy().astype(np.float64)
    lse = c.lse.cpu().numpy().astype(np.float64)
    q = u16(c.q)
    pk = u16(c.kpool)
    heads = [(s, h) for s in range(w.batch) for h in range(8)]
    _check_selection(got, c.spec, q, pk, K, window, heads)
    ref, ref_lse = c.oracle(tokens=got)
    assert_attention_close(out, lse, ref, ref_lse, "select + attend, every head")


def test_graph_replays_match_eager():
    """A 4-layer stack of in-place top-K attention calls captured in one HIP
    graph: every replay, with eager work in between, equals the eager run."""
    c, L, caps = _gather_case(50, B=2, H=8, gqa=4, ng=1)
    c.alloc([0, 1], caps, L)
    c.commit()
    K = 64
    idx = torch.from_numpy(W.topk_indices(c.spec.lengths, K, salt=50)).to(DEV)
    ws = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
    layers = 4
    outs = [torch.empty_like(c.out) for _ in range(layers)]
    lses = [torch.empty_like(c.lse) for _ in range(layers)]
    qs = [c.q.clone() for _ in range(layers)]
    for i, q in enumerate(qs):
        q.copy_((q.float() * (1.0 + 0.25 * i)).to(torch.bfloat16))
    stream = torch.cuda.Stream()

    def run():
        for i in range(layers):
            nup.attn_decode_topk_paged(c.ctx, qs[i], idx, K, outs[i], lses[i], c.scale, ws,
                                       stream=torch.cuda.current_stream())

    with torch.cuda.stream(stream):
        run()
    torch.cuda.synchronize()
    eager = [(o.clone(), l.clone()) for o, l in zip(outs, lses)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        nup.attn_decode_nonuniform(c.ctx, c.q, c.out, c.lse, c.scale,
                                   torch.empty(nup.workspace_bytes(c.ctx), dtype=torch.uint8, device=DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(layers):
            assert torch.equal(outs[i], eager[i][0]) and torch.equal(lses[i], eager[i][1]), (rep, i)
