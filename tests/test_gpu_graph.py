"""A decode step captured once into a HIP graph and replayed while the pager
changes the mapping between replays (KV-RM, abstract and Fig 2: a
fixed-shape decoder reads one committed descriptor per step, so Reserve,
Alias and Trim need no new launch shapes).  The graph's outputs, pools and
lengths are compared bit for bit with the same calls made eagerly on a twin
context, and the last step with the oracle.  The graph holds either
kv_append + attn_decode_nonuniform or the fused
attn_decode_nonuniform_append; the twin always makes the separate calls."""
import numpy as np
import pytest
import torch

import non_uniform_paged_amd as nup
import oracle
import workloads as W
from oracle import pager as pg
from tests.gpu_common import DEV, Case, assert_attention_close, u16

pytestmark = pytest.mark.gpu

NL, H, GQA, D, NG, B = 2, 4, 2, 128, 2, 5
V = NL * H


def _dev_bf16(name, shape, salt):
    return torch.from_numpy(W.normal_bf16(name, shape, salt).view(np.int16)).to(DEV).view(torch.bfloat16)


def _twins(plan_mode, max_pages, num_pages, salt, merge_mode=0):
    perm = np.random.default_rng(salt).permutation(num_pages)
    kw = dict(H=H, Hq=H * GQA, D=D, ng=NG, B=B, num_pages=num_pages, max_pages=max_pages,
              free_list_init=perm, num_workers=37, plan_mode=plan_mode, uniform_splits=3, salt=salt,
              num_layers=NL, merge_mode=merge_mode)
    return Case(**kw), Case(**kw)


def _mirror_append(c, kn, vn, fk, fv, layer):
    """The oracle pager's view of one append of `layer`: rows written at each
    active head's length, lengths advanced (no head is at its budget)."""
    sp = c.spec
    for s in range(B):
        if not sp.active[s]:
            continue
        for h in range(H):
            v = layer * H + h
            row = sp.physical_row(s, v, int(sp.lengths[s, v]))
            fk[row], fv[row] = kn[s, h], vn[s, h]
            sp.lengths[s, v] += 1


def _step(c, layer, kn, vn, q, out, lse, fused):
    nup.set_layer(c.ctx, layer)
    if fused:
        nup.attn_decode_nonuniform_append(c.ctx, kn, vn, q, out, lse, c.scale, c.ws)
    else:
        nup.kv_append(c.ctx, kn, vn)
        nup.attn_decode_nonuniform(c.ctx, q, out, lse, c.scale, c.ws)


@pytest.mark.parametrize("plan_mode,fused", [(nup.PLAN_BALANCED, False), (nup.PLAN_UNIFORM, False),
                                             (nup.PLAN_SHARED, False), (nup.PLAN_BALANCED, True),
                                             (nup.PLAN_UNIFORM, True), (nup.PLAN_SHARED, True)])
def test_graph_replay_across_commits(plan_mode, fused):
    rs = np.random.default_rng(70 + plan_mode)
    steps = 8
    max_pages = 22
    num_pages = B * NG * max_pages + 9
    G, E = _twins(plan_mode, max_pages, num_pages, 70 + plan_mode)

    def caps_for(L):   # room for every remaining step
        return np.minimum(L + rs.integers(steps, 60, size=L.shape), max_pages * 16).astype(np.int32)

    L0 = rs.integers(1, 250, size=(3, V)).astype(np.int32)
    c0 = caps_for(L0)
    for c in (G, E):
        assert c.alloc([0, 1, 3], c0, L0) == pg.OK
        c.commit()
    torch.cuda.synchronize()

    # static buffers the graph reads and writes at every replay
    kn = [torch.empty((B, H, D), dtype=torch.bfloat16, device=DEV) for _ in range(NL)]
    vn = [torch.empty_like(kn[0]) for _ in range(NL)]
    qs = [torch.empty((B, H * GQA, D), dtype=torch.bfloat16, device=DEV) for _ in range(NL)]
    outs = [torch.empty((B, H * GQA, D), dtype=torch.float32, device=DEV) for _ in range(NL)]
    lses = [torch.empty((B, H * GQA), dtype=torch.float32, device=DEV) for _ in range(NL)]
    e_out = [torch.empty_like(outs[0]) for _ in range(NL)]
    e_lse = [torch.empty_like(lses[0]) for _ in range(NL)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l in range(NL):
            _step(G, l, kn[l], vn[l], qs[l], outs[l], lses[l], fused)
        # a commit is never captured
        assert nup.nup_commit(G.ctx, raise_on_error=False) == nup.NUP_E_STATE
    # capture recorded the appends without advancing the shadow
    assert np.array_equal(nup.get_lengths(G.ctx), E.spec.lengths)

    fk, fv = u16(G.kpool).copy().reshape(-1, D), u16(G.vpool).copy().reshape(-1, D)
    for i in range(steps):
        # the mapping changes between replays: Trim, Reserve, Alias, commit
        if i == 2:
            for c in (G, E):
                c.free([1])
        if i == 3:
            L = rs.integers(0, 200, size=(2, V)).astype(np.int32)
            cp = caps_for(L)
            for c in (G, E):
                assert c.alloc([1, 2], cp, L) == pg.OK
        if i == 5:
            lens = E.spec.lengths
            share = [min(int(lens[0, v]) // 16 for v in range(V) if E.spec.group_of_head[v] == gg) // 2
                     for gg in range(NG)]
            L = np.array([[16 * share[E.spec.group_of_head[v]] + 3 for v in range(V)]], np.int32)
            cp = caps_for(L)
            for c in (G, E):
                assert c.alias([4], [0], np.array([share], np.int32), cp, L) == pg.OK
            if plan_mode == nup.PLAN_SHARED:
                # the shared prefix is planned as gangs: a worker-ordered table
                for l in range(NL):
                    nup.set_layer(G.ctx, l)
                    hr = nup.get_plan_head_rows(G.ctx)
                    assert not np.array_equal(hr, np.arange(len(hr))), l
        if i == 6:
            for c in (G, E):
                c.free([0, 3])
        for c in (G, E):
            c.commit()
        fk, fv = u16(G.kpool).copy().reshape(-1, D), u16(G.vpool).copy().reshape(-1, D)
        for l in range(NL):
            kn[l].copy_(_dev_bf16("k", (B, H, D), 1000 * i + l))
            vn[l].copy_(_dev_bf16("v", (B, H, D), 1000 * i + l))
            qs[l].copy_(_dev_bf16("q", (B, H * GQA, D), 1000 * i + l))
        g.replay()
        nup.note_appends(G.ctx, 1)
        for l in range(NL):     # eager twin, same stream, between replays
            nup.set_layer(E.ctx, l)
            nup.kv_append(E.ctx, kn[l], vn[l])
            nup.attn_decode_nonuniform(E.ctx, qs[l], e_out[l], e_lse[l], E.scale, E.ws)
            _mirror_append(E, u16(kn[l]), u16(vn[l]), fk, fv, l)
        G.spec.lengths[:] = E.spec.lengths    # the twins' pagers stay identical
        torch.cuda.synchronize()
        for l in range(NL):
            assert torch.equal(outs[l], e_out[l]) and torch.equal(lses[l], e_lse[l]), (i, l)
        assert np.array_equal(nup.get_lengths(G.ctx), E.spec.lengths), i
        assert np.array_equal(nup.get_lengths(E.ctx), E.spec.lengths), i
        assert torch.equal(G.kpool, E.kpool) and torch.equal(G.vpool, E.vpool), i
    assert nup.device_errors(G.ctx) == nup.NUP_OK

    # the last replay against the oracle, from the oracle pager's own state
    assert np.array_equal(u16(G.kpool).reshape(-1, D), fk) and np.array_equal(u16(G.vpool).reshape(-1, D), fv)
    sp = E.spec
    assert np.array_equal(nup.get_page_table(G.ctx), sp.page_table)
    kp, vp = fk.reshape(u16(G.kpool).shape), fv.reshape(u16(G.vpool).shape)
    for l in range(NL):
        sl = slice(l * H, (l + 1) * H)
        ref, ref_lse = oracle.decode(u16(qs[l]), kp, vp, sp.page_table, sp.lengths[:, sl],
                                     sp.group_of_head[sl], sp.slot_of_head[sl], G.scale)
        assert_attention_close(outs[l].cpu().numpy().astype(np.float64),
                               lses[l].cpu().numpy().astype(np.float64), ref, ref_lse, f"graph layer {l}")


@pytest.mark.parametrize("fused,merge_mode", [(False, nup.MERGE_LAUNCH), (True, nup.MERGE_LAUNCH),
                                              (True, nup.MERGE_IN_SPLIT)])
def test_graph_append_stops_at_budget(fused, merge_mode):
    """A replayed append cannot be refused on the host: the kernel drops the
    token of a head at its budget, latches NUP_E_CAPACITY, and
    nup_note_appends mirrors exactly that (with the fused step, the length
    advance is the merge launch's or, merged in the split-K launch, the
    finishing wave's)."""
    rs = np.random.default_rng(75)
    max_pages = 12
    num_pages = B * NG * max_pages + 5
    c, _ = _twins(nup.PLAN_BALANCED, max_pages, num_pages, 75, merge_mode)
    L = rs.integers(20, 150, size=(2, V)).astype(np.int32)
    caps = (L + 5).astype(np.int32)
    caps[0, 1] = L[0, 1] + 1          # one append left
    caps[1, 6] = L[1, 6]              # already full
    assert c.alloc([0, 2], caps, L) == pg.OK
    c.commit()
    torch.cuda.synchronize()
    kn = torch.empty((B, H, D), dtype=torch.bfloat16, device=DEV)
    vn = torch.empty_like(kn)
    nup.set_layer(c.ctx, 1)      # eagerly, the full head refuses the whole step
    assert nup.kv_append(c.ctx, kn, vn, raise_on_error=False) == nup.NUP_E_CAPACITY
    assert nup.attn_decode_nonuniform_append(c.ctx, kn, vn, c.q, c.out, c.lse, c.scale, c.ws,
                                             raise_on_error=False) == nup.NUP_E_CAPACITY

    g = torch.cuda.CUDAGraph()
    ks = torch.empty((4096, D), dtype=torch.bfloat16, device=DEV)
    row_off = np.arange(B * H, dtype=np.int64) * 200
    row_off_dev = torch.from_numpy(row_off).to(DEV)
    with torch.cuda.graph(g):
        for l in range(NL):
            if fused:
                _step(c, l, kn, vn, c.q, c.out, c.lse, True)
            else:
                nup.set_layer(c.ctx, l)
                nup.kv_append(c.ctx, kn, vn)
        # the trains gathers are sized by the current trains: refused under capture
        assert nup.kv_gather_compact(c.ctx, 0, ks, ks, row_off=row_off_dev,
                                     raise_on_error=False) == nup.NUP_E_STATE
        assert nup.kv_gather_trains_dma(c.ctx, ks, ks, row_off, raise_on_error=False) == nup.NUP_E_STATE
    fk, fv = u16(c.kpool).copy().reshape(-1, D), u16(c.vpool).copy().reshape(-1, D)
    sp = c.spec
    for i in range(3):
        kn.copy_(_dev_bf16("k", (B, H, D), 900 + i))
        vn.copy_(_dev_bf16("v", (B, H, D), 900 + i))
        k_h, v_h = u16(kn), u16(vn)
        g.replay()
        for l in range(NL):
            for s in range(B):
                if not sp.active[s]:
                    continue
                for h in range(H):
                    v = l * H + h
                    if sp.lengths[s, v] < sp.caps[s, v]:
                        row = sp.physical_row(s, v, int(sp.lengths[s, v]))
                        fk[row], fv[row] = k_h[s, h], v_h[s, h]
                        sp.lengths[s, v] += 1
    torch.cuda.synchronize()
    assert np.array_equal(u16(c.kpool).reshape(-1, D), fk) and np.array_equal(u16(c.vpool).reshape(-1, D), fv)
    with pytest.raises(nup.NupError) as ei:
        nup.note_appends(c.ctx, 3)
    assert ei.value.status == nup.NUP_E_CAPACITY
    assert np.array_equal(nup.get_lengths(c.ctx), sp.lengths)
    assert nup.device_errors(c.ctx) == nup.NUP_E_CAPACITY
    assert nup.device_errors(c.ctx) == nup.NUP_OK      # read clears it

    # the next commit sends these lengths: attention agrees with the oracle
    c.free([2])
    c.commit()
    for l in range(NL):
        nup.set_layer(c.ctx, l)
        nup.attn_decode_nonuniform(c.ctx, c.q, c.out, c.lse, c.scale, c.ws)
        torch.cuda.synchronize()
        sl = slice(l * H, (l + 1) * H)
        ref, ref_lse = oracle.decode(u16(c.q), fk.reshape(u16(c.kpool).shape), fv.reshape(u16(c.vpool).shape),
                                     sp.page_table, sp.lengths[:, sl], sp.group_of_head[sl],
                                     sp.slot_of_head[sl], c.scale)
        assert_attention_close(c.out.cpu().numpy().astype(np.float64), c.lse.cpu().numpy().astype(np.float64),
                               ref, ref_lse, f"after replays, layer {l}")


def test_graph_select_then_attend_in_place():
    """The sparse decode step (KVDrive, Fig 1: choose critical entries, then
    attend to them) in a graph: append, exact top-K selection and in-place
    top-K attention, replayed across Trim / Reserve commits and compared bit
    for bit with the same calls made eagerly on a twin context."""
    rs = np.random.default_rng(77)
    H1, gqa, D1, B1, K, window, replays = 4, 4, 128, 3, 32, 8, 5
    max_pages = 40
    kw = dict(H=H1, Hq=H1 * gqa, D=D1, ng=2, B=B1, num_pages=B1 * 2 * max_pages + 3, max_pages=max_pages,
              free_list_init=rs.permutation(B1 * 2 * max_pages + 3), num_workers=50, salt=77)
    G, E = Case(**kw), Case(**kw)

    def lengths(n):
        return rs.integers(K + 1, 600, size=(n, H1)).astype(np.int32)

    L = lengths(2)
    for c in (G, E):
        assert c.alloc([0, 2], L + replays + 2, L) == pg.OK
        c.commit()
    kn = torch.empty((B1, H1, D1), dtype=torch.bfloat16, device=DEV)
    vn = torch.empty_like(kn)
    q = torch.empty((B1, H1 * gqa, D1), dtype=torch.bfloat16, device=DEV)
    bufs = {}
    for name, c in (("G", G), ("E", E)):
        bufs[name] = dict(idx=torch.full((B1, H1, K), -3, dtype=torch.int32, device=DEV),
                          out=torch.empty((B1, H1 * gqa, D1), dtype=torch.float32, device=DEV),
                          lse=torch.empty((B1, H1 * gqa), dtype=torch.float32, device=DEV),
                          sws=torch.empty(nup.select_workspace_bytes(c.ctx), dtype=torch.uint8, device=DEV),
                          aws=torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV))

    def step(c, b):
        nup.kv_append(c.ctx, kn, vn)
        nup.kv_select_topk(c.ctx, q, K, window, b["idx"], b["sws"])
        nup.attn_decode_topk_paged(c.ctx, q, b["idx"], K, b["out"], b["lse"], c.scale, b["aws"])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(G, bufs["G"])
    live = {0, 2}
    for i in range(replays):
        if i == 2:
            for c in (G, E):
                c.free([0])
            live.discard(0)
        if i == 3:
            L = lengths(2)
            for c in (G, E):
                assert c.alloc([0, 1], L + replays, L) == pg.OK
            live |= {0, 1}
        for c in (G, E):
            c.commit()
        kn.copy_(_dev_bf16("k", (B1, H1, D1), 3000 + i))
        vn.copy_(_dev_bf16("v", (B1, H1, D1), 3000 + i))
        q.copy_(_dev_bf16("q", (B1, H1 * gqa, D1), 3000 + i))
        g.replay()
        nup.note_appends(G.ctx, 1)
        step(E, bufs["E"])
        torch.cuda.synchronize()
        act = sorted(live)
        for key in ("idx", "out", "lse"):
            assert torch.equal(bufs["G"][key][act], bufs["E"][key][act]), (i, key)
        assert np.array_equal(nup.get_lengths(G.ctx), nup.get_lengths(E.ctx)), i
    assert torch.equal(G.kpool, E.kpool) and torch.equal(G.vpool, E.vpool)
    assert nup.device_errors(G.ctx) == nup.NUP_OK and nup.device_errors(E.ctx) == nup.NUP_OK


@pytest.mark.parametrize("fused", [False, True])
def test_graph_gang_launch_follows_commits(fused):
    """The share-aware plan's gang launch inside a captured graph: forks of
    one source are added (Alias) and removed (Trim) between replays, so the
    number of gang workgroups changes from commit to commit (the kernel
    reads it on the device).  Every replay equals the same calls made eagerly
    on a twin, bit for bit; the last one is checked against the oracle."""
    Hh, gq, Dd, Bb = 4, 4, 128, 8
    rs = np.random.default_rng(91)
    kw = dict(H=Hh, Hq=Hh * gq, D=Dd, ng=1, B=Bb, num_pages=Bb * 40 + 8, max_pages=40,
              free_list_init=np.random.default_rng(91).permutation(Bb * 40 + 8), num_workers=64,
              plan_mode=nup.PLAN_SHARED, salt=91)
    G, E = Case(**kw), Case(**kw)
    L0 = rs.integers(300, 500, size=(1, Hh)).astype(np.int32)
    for c in (G, E):
        assert c.alloc([0], L0 + 40, L0) == pg.OK
        c.commit()
    kn = torch.empty((Bb, Hh, Dd), dtype=torch.bfloat16, device=DEV)
    vn = torch.empty_like(kn)
    q = torch.empty((Bb, Hh * gq, Dd), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((Bb, Hh * gq, Dd), dtype=torch.float32, device=DEV)
    lse = torch.empty((Bb, Hh * gq), dtype=torch.float32, device=DEV)
    e_out, e_lse = torch.empty_like(out), torch.empty_like(lse)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(G, 0, kn, vn, q, out, lse, fused)
    counts = []
    fk, fv = u16(G.kpool).copy().reshape(-1, Dd), u16(G.vpool).copy().reshape(-1, Dd)
    for i in range(6):
        share = int(E.spec.lengths[0].min()) // 16 // 2
        if i in (1, 2):                      # four more sharers each time
            new = [1, 2, 3, 4] if i == 1 else [5, 6, 7]
            L = np.full((len(new), Hh), 16 * share + 20, np.int32)
            for c in (G, E):
                assert c.alias(new, [0] * len(new), np.full((len(new), 1), share, np.int32), L + 40, L) == pg.OK
        if i == 4:
            for c in (G, E):
                c.free([2, 5])
        for c in (G, E):
            c.commit()
        counts.append(len(nup.get_plan_gangs(G.ctx)[0]))
        fk, fv = u16(G.kpool).copy().reshape(-1, Dd), u16(G.vpool).copy().reshape(-1, Dd)
        kn.copy_(_dev_bf16("k", (Bb, Hh, Dd), 500 + i))
        vn.copy_(_dev_bf16("v", (Bb, Hh, Dd), 500 + i))
        q.copy_(_dev_bf16("q", (Bb, Hh * gq, Dd), 500 + i))
        g.replay()
        nup.note_appends(G.ctx, 1)
        nup.kv_append(E.ctx, kn, vn)
        nup.attn_decode_nonuniform(E.ctx, q, e_out, e_lse, E.scale, E.ws)
        sp = E.spec
        for s in range(Bb):
            if sp.active[s]:
                for h in range(Hh):
                    row = sp.physical_row(s, h, int(sp.lengths[s, h]))
                    fk[row], fv[row] = u16(kn)[s, h], u16(vn)[s, h]
                    sp.lengths[s, h] += 1
        G.spec.lengths[:] = sp.lengths
        torch.cuda.synchronize()
        assert torch.equal(out, e_out) and torch.equal(lse, e_lse), i
        assert torch.equal(G.kpool, E.kpool) and torch.equal(G.vpool, E.vpool), i
        assert np.array_equal(nup.get_lengths(G.ctx), sp.lengths), i
    assert counts[0] == 0 and max(counts) > 0 and len(set(counts)) > 2, counts
    assert nup.device_errors(G.ctx) == nup.NUP_OK
    kp, vp = fk.reshape(u16(G.kpool).shape), fv.reshape(u16(G.vpool).shape)
    ref, ref_lse = oracle.decode(u16(q), kp, vp, E.spec.page_table, E.spec.lengths,
                                 E.spec.group_of_head, E.spec.slot_of_head, G.scale)
    assert_attention_close(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                           ref, ref_lse, "gang graph, last replay")
