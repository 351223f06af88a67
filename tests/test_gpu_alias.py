"""Alias (KV-RM, Fig 3): forked sequences whose leading pages are the
physical pages of a live source.  Decode over shared pages, appends after
the fork, trains gathers and Trim of the source are checked against the
oracle's own pager and fp64 attention."""
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import non_uniform_paged_amd as nup
import oracle
import workloads as W
from oracle import pager as pg
from tests.gpu_common import DEV, Case, assert_attention_close, u16

pytestmark = pytest.mark.gpu


def _group_share(goh, tokens_per_head, ng):
    """Whole pages every head of a group can share: min over its heads // 16."""
    share = np.zeros(ng, np.int64)
    for g in range(ng):
        share[g] = min(int(tokens_per_head[h]) for h in range(len(goh)) if goh[h] == g) // 16
    return share


def _append_steps(c, steps, salt):
    """Append through the library and place the same rows in a host copy of
    the pool by the oracle pager's positions."""
    kp = u16(c.kpool).copy()
    vp = u16(c.vpool).copy()
    fk, fv = kp.reshape(-1, c.D), vp.reshape(-1, c.D)
    for step in range(steps):
        kn = W.normal_bf16("k", (c.B, c.H, c.D), salt + step)
        vn = W.normal_bf16("v", (c.B, c.H, c.D), salt + step)
        nup.kv_append(c.ctx, torch.from_numpy(kn.view(np.int16)).to(DEV),
                      torch.from_numpy(vn.view(np.int16)).to(DEV))
        st, pos = c.spec.append_positions()
        assert st == pg.OK
        for s in range(c.B):
            if c.spec.active[s]:
                for h in range(c.H):
                    row = c.spec.physical_row(s, h, int(pos[s, h]))
                    fk[row], fv[row] = kn[s, h], vn[s, h]
        c.commit()
    return kp, vp


# (plan mode, workers): the share-aware plan with room for its gangs, and
# with too few workers for them (it then plans like the balanced one)
PLANS = [(nup.PLAN_BALANCED, 37), (nup.PLAN_SHARED, 64), (nup.PLAN_SHARED, 37)]


@pytest.mark.parametrize("plan_mode,workers", PLANS)
def test_alias_decode_append_gather_trim(plan_mode, workers):
    H, gqa, D, B, ng = 8, 4, 128, 6, 2
    rs = np.random.default_rng(31)
    L0 = rs.integers(200, 700, size=H)
    max_pages = 64
    num_pages = 300
    c = Case(H=H, Hq=H * gqa, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages,
             free_list_init=rs.permutation(num_pages), num_workers=workers, plan_mode=plan_mode, salt=31)
    assert c.alloc([0], (L0 + 20)[None], L0[None]) == pg.OK
    goh = c.spec.group_of_head
    forks = [1, 2, 3, 4]
    share = np.zeros((len(forks), ng), np.int64)
    lens = np.zeros((len(forks), H), np.int64)
    for i in range(len(forks)):
        most = _group_share(goh, L0, ng)
        share[i] = rs.integers(0, most + 1)
        share[i, i % ng] = most[i % ng]                   # one group shared in full
        lens[i] = share[i][goh] * 16 + rs.integers(0, 300, size=H)
    caps = lens + rs.integers(8, 40, size=lens.shape)
    assert c.alias(forks, [0] * len(forks), share, caps, lens) == pg.OK
    assert np.array_equal(nup.get_refcounts(c.ctx), c.spec.ref)
    assert c.spec.ref.max() == 1 + len(forks)
    c.commit()
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert_attention_close(out, lse, ref, ref_lse, "forks over shared pages")

    if plan_mode == nup.PLAN_SHARED and workers == 64:
        # the forks' common prefix is planned as gangs: rows in worker order
        hr = nup.get_plan_head_rows(c.ctx)
        assert not np.array_equal(hr, np.arange(len(hr)))

    # decode steps after the fork: every write lands on an unshared page
    kp, vp = _append_steps(c, 6, 3100)
    assert np.array_equal(u16(c.kpool), kp) and np.array_equal(u16(c.vpool), vp)
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert_attention_close(out, lse, ref, ref_lse, "after appends")

    # one fused step (append inside the split-K kernel, lengths advanced by
    # the merge); the oracle's pools get the rows by its own pager
    kn = W.normal_bf16("k", (c.B, c.H, c.D), 3199)
    vn = W.normal_bf16("v", (c.B, c.H, c.D), 3199)
    nup.attn_decode_nonuniform_append(c.ctx, torch.from_numpy(kn.view(np.int16)).to(DEV),
                                      torch.from_numpy(vn.view(np.int16)).to(DEV),
                                      c.q, c.out, c.lse, c.scale, c.ws)
    torch.cuda.synchronize()
    st, pos = c.spec.append_positions()
    assert st == pg.OK
    fk, fv = kp.reshape(-1, D), vp.reshape(-1, D)
    for s in range(B):
        if c.spec.active[s]:
            for h in range(H):
                row = c.spec.physical_row(s, h, int(pos[s, h]))
                fk[row], fv[row] = kn[s, h], vn[s, h]
    assert np.array_equal(u16(c.kpool), kp) and np.array_equal(u16(c.vpool), vp)
    assert np.array_equal(nup.get_lengths(c.ctx), c.spec.lengths)
    ref, ref_lse = oracle.decode(u16(c.q), kp, vp, c.spec.page_table, c.spec.lengths,
                                 c.spec.group_of_head, c.spec.slot_of_head, c.scale)
    assert_attention_close(c.out.cpu().numpy().astype(np.float64), c.lse.cpu().numpy().astype(np.float64),
                           ref, ref_lse, "fused step over shared pages")
    c.commit()

    # trains of the forked rows: bit-exact rows, shared prefix included
    lens_now = c.spec.lengths.astype(np.int64)
    row_off = np.concatenate([[0], np.cumsum(lens_now.reshape(-1))[:-1]]).astype(np.int64)
    total = int(lens_now.sum())
    ks = torch.zeros((total, D), dtype=torch.int16, device=DEV)
    vs = torch.zeros_like(ks)
    phys = torch.full((total,), -1, dtype=torch.int32, device=DEV)
    nup.kv_gather_compact(c.ctx, 0, ks, vs, row_off=torch.from_numpy(row_off).to(DEV), phys_out=phys)
    torch.cuda.synchronize()
    want = pg.gather_pages(c.spec, kp, vp, row_off)
    gk, gv, gp = ks.cpu().numpy().view(np.uint16), vs.cpu().numpy().view(np.uint16), phys.cpu().numpy()
    for (s, h), (kr, vr, rows) in want.items():
        o, n = row_off[s * H + h], len(kr)
        assert np.array_equal(gk[o:o + n], kr) and np.array_equal(gv[o:o + n], vr), (s, h)
        assert np.array_equal(gp[o:o + n], rows), (s, h)

    # Trim the source: the shared pages stay with the forks; a new sequence
    # takes only pages nobody maps
    c.free([0])
    assert np.array_equal(nup.get_free_list(c.ctx), c.spec.free_list())
    assert c.alloc([5], np.full((1, H), 200), np.full((1, H), 150)) == pg.OK
    c.commit()
    out, lse = c.attend()
    ref, ref_lse = c.oracle()
    assert_attention_close(out, lse, ref, ref_lse, "after Trim of the source")
    assert np.array_equal(nup.get_refcounts(c.ctx), c.spec.ref)


@pytest.mark.parametrize("plan_mode", [nup.PLAN_BALANCED, nup.PLAN_SHARED])
def test_alias_full_size_prefix_batch(plan_mode):
    """Qwen2.5-32B-shaped batch where 60 of 64 sessions fork from 4 sources
    (a shared 8192-token prompt); every session against the oracle, under
    the balanced plan and under the share-aware one (the bench's launch:
    2048 workers)."""
    w = W.qwen25_32b_prefix()
    src = w.extra["alias_src"]
    pre = w.extra["prefix_tokens"]
    max_pages = int(math.ceil(w.caps.max() / 16))
    c = Case(H=w.num_kv_heads, Hq=w.num_q_heads, D=w.head_dim, ng=w.num_groups, B=w.batch,
             num_pages=w.num_pages, max_pages=max_pages, plan_mode=plan_mode, salt=32)
    roots = [s for s in range(w.batch) if src[s] < 0]
    forks = [s for s in range(w.batch) if src[s] >= 0]
    assert c.alloc(roots, w.caps[roots], w.lengths[roots]) == pg.OK
    goh = c.spec.group_of_head
    share = np.stack([_group_share(goh, pre[s], w.num_groups) for s in forks])
    assert c.alias(forks, src[forks], share, w.caps[forks], w.lengths[forks]) == pg.OK
    c.commit()
    used = int((c.spec.ref > 0).sum())
    entries = int(c.spec.n_pages.sum())
    assert used == entries - int(share.sum())
    nup.attn_decode_nonuniform(c.ctx, c.q, c.out, c.lse, c.scale, c.ws)
    torch.cuda.synchronize()
    ref, ref_lse = c.oracle()
    out = c.out.cpu().numpy().astype(np.float64)
    lse = c.lse.cpu().numpy().astype(np.float64)
    assert_attention_close(out, lse, ref, ref_lse, "qwen25_32b_prefix, every session")


@settings(max_examples=int(os.environ.get("NUP_FUZZ_EXAMPLES", "30")), deadline=None, derandomize=True,
          suppress_health_check=list(HealthCheck))
@given(st.data())
def test_shared_plan_random_forks(data):
    """Random shapes, layers, groups and worker counts; sources with forks
    of random shares (and sometimes a Trim of a source), attended under the
    share-aware plan, every layer against the oracle; then one fused step."""
    D = data.draw(st.sampled_from([64, 128]))
    gqa = data.draw(st.sampled_from([1, 2, 4, 5, 8]))
    H = data.draw(st.sampled_from([1, 2, 4, 8]))
    NL = data.draw(st.sampled_from([1, 1, 2]))
    V = NL * H
    ng = data.draw(st.sampled_from([g for g in range(1, V + 1) if V % g == 0]))
    B = data.draw(st.integers(2, 8))
    workers = data.draw(st.sampled_from([5, 16, 64, 0]))
    seed = data.draw(st.integers(0, 2 ** 16))
    rs = np.random.default_rng(seed)
    maxL = 400
    max_pages = (maxL + 100) // 16 + 1     # room for a fork's share + 59 + headroom
    num_pages = B * ng * max_pages + 7
    c = Case(H=H, Hq=H * gqa, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages,
             free_list_init=rs.permutation(num_pages), num_workers=workers, plan_mode=nup.PLAN_SHARED,
             salt=seed % 83 + 1, num_layers=NL)
    n_src = int(rs.integers(1, min(3, B - 1) + 1))
    L0 = rs.integers(16, maxL + 1, size=(n_src, V)).astype(np.int32)
    assert c.alloc(list(range(n_src)), L0 + rs.integers(1, 40, size=L0.shape), L0) == pg.OK
    goh = c.spec.group_of_head
    for f in range(n_src, B):
        s0 = int(rs.integers(0, n_src))
        most = _group_share(goh, c.spec.lengths[s0], ng)
        share = rs.integers(0, most + 1)
        if rs.random() < 0.5:                  # one group shared in full
            g = int(rs.integers(0, ng))
            share[g] = most[g]
        L = (share[goh] * 16 + rs.integers(0, 60, size=V)).astype(np.int32)
        assert c.alias([f], [s0], share[None], (L + rs.integers(1, 30, size=V))[None], L[None]) == pg.OK
    if rs.random() < 0.3:
        c.free([0])
    c.commit()
    tag = f"seed {seed} D{D} gqa{gqa} H{H} NL{NL} ng{ng} B{B} W{workers}"
    for l in range(NL):
        nup.set_layer(c.ctx, l)
        out, lse = c.attend()
        sl = slice(l * H, (l + 1) * H)
        ref, ref_lse = oracle.decode(u16(c.q), u16(c.kpool), u16(c.vpool), c.spec.page_table,
                                     c.spec.lengths[:, sl], goh[sl], c.spec.slot_of_head[sl], c.scale)
        assert_attention_close(out, lse, ref, ref_lse, f"{tag} layer {l}")
    # one fused step on layer 0; the oracle's pools get the rows by its pager
    nup.set_layer(c.ctx, 0)
    kp, vp = u16(c.kpool).copy(), u16(c.vpool).copy()
    kn = W.normal_bf16("k", (B, H, D), seed + 1)
    vn = W.normal_bf16("v", (B, H, D), seed + 1)
    nup.attn_decode_nonuniform_append(c.ctx, torch.from_numpy(kn.view(np.int16)).to(DEV),
                                      torch.from_numpy(vn.view(np.int16)).to(DEV),
                                      c.q, c.out, c.lse, c.scale, c.ws)
    torch.cuda.synchronize()
    fk, fv = kp.reshape(-1, D), vp.reshape(-1, D)
    for s in range(B):
        if c.spec.active[s]:
            for h in range(H):
                row = c.spec.physical_row(s, h, int(c.spec.lengths[s, h]))
                fk[row], fv[row] = kn[s, h], vn[s, h]
                c.spec.lengths[s, h] += 1
    assert np.array_equal(u16(c.kpool), kp) and np.array_equal(u16(c.vpool), vp), tag
    assert np.array_equal(nup.get_lengths(c.ctx), c.spec.lengths), tag
    ref, ref_lse = oracle.decode(u16(c.q), kp, vp, c.spec.page_table, c.spec.lengths[:, :H],
                                 goh[:H], c.spec.slot_of_head[:H], c.scale)
    assert_attention_close(c.out.cpu().numpy().astype(np.float64), c.lse.cpu().numpy().astype(np.float64),
                           ref, ref_lse, f"{tag} fused")
    assert nup.device_errors(c.ctx) == nup.NUP_OK


def test_select_topk_under_shared_plan_equals_balanced():
    """Exact top-K selection walks every row of the plan, the gang rows of
    the share-aware plan included (only the attention's main launch skips
    them): on forked sequences its choices are bit-identical to the
    balanced plan's on a twin context, and so is the attention."""
    H, gqa, D, B, ng = 8, 4, 128, 6, 2
    rs = np.random.default_rng(33)
    L0 = rs.integers(300, 700, size=H)
    twins = [Case(H=H, Hq=H * gqa, D=D, ng=ng, B=B, num_pages=300, max_pages=64,
                  free_list_init=np.random.default_rng(33).permutation(300), num_workers=64,
                  plan_mode=mode, salt=33) for mode in (nup.PLAN_BALANCED, nup.PLAN_SHARED)]
    for c in twins:
        assert c.alloc([0], (L0 + 20)[None], L0[None]) == pg.OK
    goh = twins[0].spec.group_of_head
    most = _group_share(goh, L0, ng)
    forks = [1, 2, 3, 4]
    share = np.tile(most, (len(forks), 1))
    lens = share[:, goh] * 16 + 64 + rs.integers(0, 200, size=(len(forks), H))
    caps = lens + 16
    for c in twins:
        assert c.alias(forks, [0] * len(forks), share, caps, lens) == pg.OK
        c.commit()
    gangs, _ = nup.get_plan_gangs(twins[1].ctx)
    assert len(gangs) > 0                           # the shared plan has a gang launch
    K, window = 48, 8
    picks = []
    for c in twins:
        out = torch.full((B, H, K), -5, dtype=torch.int32, device=DEV)
        ws = torch.empty(nup.select_workspace_bytes(c.ctx), dtype=torch.uint8, device=DEV)
        nup.kv_select_topk(c.ctx, c.q, K, window, out, ws)
        torch.cuda.synchronize()
        picks.append(out.cpu().numpy())
    assert np.array_equal(picks[0], picks[1])
    assert (picks[0][:5] >= 0).all() and (picks[0][5] == -5).all()
    outs = [c.attend() for c in twins]
    ref, ref_lse = twins[1].oracle()
    for out, lse in outs:
        assert_attention_close(out, lse, ref, ref_lse, "twins")
