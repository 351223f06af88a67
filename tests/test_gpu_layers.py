"""Head groups that span layers (Tangram, Fig 11: group sizes beyond one
layer's heads): one pager over (layer, KV head) pairs, per-layer calls.
Each layer is checked against the oracle on that layer's slice of the
pager state."""
import numpy as np
import pytest
import torch

import non_uniform_paged_amd as nup
import oracle
import workloads as W
from oracle import pager as pg
from tests.gpu_common import DEV, Case, assert_attention_close, u16

pytestmark = pytest.mark.gpu


def _layer_oracle(c, layer, q, kp=None, vp=None, tokens=None):
    sl = slice(layer * c.H, (layer + 1) * c.H)
    sp = c.spec
    return oracle.decode(u16(q), u16(c.kpool) if kp is None else kp, u16(c.vpool) if vp is None else vp,
                         sp.page_table, sp.lengths[:, sl], sp.group_of_head[sl], sp.slot_of_head[sl],
                         c.scale, tokens=tokens)


def _q(c, layer, salt):
    return torch.from_numpy(W.normal_bf16("q", (c.B, c.Hq, c.D), salt + layer).view(np.int16)).to(DEV).view(torch.bfloat16)


@pytest.mark.parametrize("NL,H,gqa,ng", [(3, 4, 2, 3), (4, 8, 4, 2), (2, 2, 5, 1)])
def test_layers_decode_append_gather(NL, H, gqa, ng):
    D, B = 128, 3
    rs = np.random.default_rng(60 + NL)
    V = NL * H
    L = rs.integers(0, 400, size=(B, V)).astype(np.int32)
    L[0, 1] = 1
    caps = (L + rs.integers(4, 30, size=(B, V))).astype(np.int32)
    max_pages = int(np.ceil(caps.max() / 16))
    num_pages = B * ng * max_pages + 7
    c = Case(H=H, Hq=H * gqa, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages,
             free_list_init=rs.permutation(num_pages), num_workers=29, salt=60 + NL, num_layers=NL)
    assert c.alloc([0, 2], caps[[0, 2]], L[[0, 2]]) == pg.OK
    c.commit()
    goh = c.spec.group_of_head
    if ng > 1:   # the grouping does mix layers
        assert any(len({v // H for v in range(V) if goh[v] == g}) > 1 for g in range(ng))
    qs = [_q(c, l, 600) for l in range(NL)]
    for l in range(NL):
        nup.set_layer(c.ctx, l)
        nup.attn_decode_nonuniform(c.ctx, qs[l], c.out, c.lse, c.scale, c.ws)
        torch.cuda.synchronize()
        ref, ref_lse = _layer_oracle(c, l, qs[l])
        assert_attention_close(c.out.cpu().numpy().astype(np.float64), c.lse.cpu().numpy().astype(np.float64),
                               ref, ref_lse, f"layer {l}")

    # one decode step: every layer appends its own token
    kp, vp = u16(c.kpool).copy(), u16(c.vpool).copy()
    fk, fv = kp.reshape(-1, D), vp.reshape(-1, D)
    for l in range(NL):
        nup.set_layer(c.ctx, l)
        kn = W.normal_bf16("k", (B, H, D), 700 + l)
        vn = W.normal_bf16("v", (B, H, D), 700 + l)
        nup.kv_append(c.ctx, torch.from_numpy(kn.view(np.int16)).to(DEV), torch.from_numpy(vn.view(np.int16)).to(DEV))
        for s in range(B):
            if not c.spec.active[s]:
                continue
            for h in range(H):
                v = l * H + h
                row = c.spec.physical_row(s, v, int(c.spec.lengths[s, v]))
                fk[row], fv[row] = kn[s, h], vn[s, h]
                c.spec.lengths[s, v] += 1
    torch.cuda.synchronize()
    assert np.array_equal(nup.get_lengths(c.ctx), c.spec.lengths)
    assert np.array_equal(u16(c.kpool), kp) and np.array_equal(u16(c.vpool), vp)
    for l in range(NL):
        nup.set_layer(c.ctx, l)
        nup.attn_decode_nonuniform(c.ctx, qs[l], c.out, c.lse, c.scale, c.ws)
        torch.cuda.synchronize()
        ref, ref_lse = _layer_oracle(c, l, qs[l], kp, vp)
        assert_attention_close(c.out.cpu().numpy().astype(np.float64), c.lse.cpu().numpy().astype(np.float64),
                               ref, ref_lse, f"layer {l} after append")

    # trains gather of one layer: exactly that layer's rows
    l = NL - 1
    nup.set_layer(c.ctx, l)
    sl = slice(l * H, (l + 1) * H)
    lens = c.spec.lengths[:, sl].astype(np.int64).reshape(-1)
    row_off = np.concatenate([[0], np.cumsum(lens + 3)[:-1]]).astype(np.int64)
    total = int((lens + 3).sum())
    ks = torch.full((total, D), -7, dtype=torch.int16, device=DEV)
    vs = torch.full_like(ks, -7)
    nup.kv_gather_compact(c.ctx, 0, ks, vs, row_off=torch.from_numpy(row_off).to(DEV))
    torch.cuda.synchronize()
    gk, gv = ks.cpu().numpy(), vs.cpu().numpy()
    written = np.zeros(total, bool)
    for s in range(B):
        if not c.spec.active[s]:
            continue
        for h in range(H):
            n = int(c.spec.lengths[s, l * H + h])
            rows = [c.spec.physical_row(s, l * H + h, t) for t in range(n)]
            o = row_off[s * H + h]
            assert np.array_equal(gk[o:o + n].view(np.uint16), fk[rows]) and \
                np.array_equal(gv[o:o + n].view(np.uint16), fv[rows]), (s, h)
            written[o:o + n] = True
    assert (gk[~written] == -7).all() and (gv[~written] == -7).all()

    # in-place top-K attention of one layer against the oracle's token mode
    K = 16
    act_len = c.spec.lengths[[0, 2]]
    l = int(np.argmax([act_len[:, m * H:(m + 1) * H].min() for m in range(NL)]))
    nup.set_layer(c.ctx, l)
    sl = slice(l * H, (l + 1) * H)
    assert (act_len[:, sl] >= K).all()
    if True:
        idx = np.zeros((B, H, K), np.int32)
        for s in (0, 2):
            for h in range(H):
                idx[s, h] = np.sort(rs.choice(int(c.spec.lengths[s, l * H + h]), K, replace=False))
        ws = torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV)
        nup.attn_decode_topk_paged(c.ctx, qs[l], torch.from_numpy(idx).to(DEV), K, c.out, c.lse, c.scale, ws)
        torch.cuda.synchronize()
        ref, ref_lse = _layer_oracle(c, l, qs[l], kp, vp, tokens=idx)
        assert_attention_close(c.out.cpu().numpy().astype(np.float64)[[0, 2]],
                               c.lse.cpu().numpy().astype(np.float64)[[0, 2]], ref[[0, 2]], ref_lse[[0, 2]],
                               f"top-K in place, layer {l}")

    # selection on that layer: structure and membership against the oracle's
    # scores of the layer's heads
    from oracle import select as osel
    window = 4
    sel = torch.full((B, H, K), -5, dtype=torch.int32, device=DEV)
    ws_sel = torch.empty(nup.select_workspace_bytes(c.ctx), dtype=torch.uint8, device=DEV)
    nup.kv_select_topk(c.ctx, qs[l], K, window, sel, ws_sel)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    assert (got[1] == -5).all()
    view = pg.PagerSpec(H, ng, B, num_pages, max_pages, 16)   # the layer's heads over the same pages
    view.page_table, view.n_pages, view.active = c.spec.page_table, c.spec.n_pages, c.spec.active
    view.lengths = c.spec.lengths[:, sl].copy()
    view.group_of_head, view.slot_of_head = c.spec.group_of_head[sl], c.spec.slot_of_head[sl]
    view.g_h = c.gh
    for s in (0, 2):
        for h in range(H):
            Lh = int(view.lengths[s, h])
            g = got[s, h]
            assert (np.diff(g) > 0).all() and g[-window:].tolist() == list(range(Lh - window, Lh))
            sc = osel.scores(u16(qs[l]), kp, view, s, h)
            want = osel.select(sc, K, window)
            cand = sc[: Lh - window]
            thr = np.sort(cand)[::-1][K - window - 1]
            sure = np.abs(cand - thr) > 1e-3 * max(1.0, abs(thr))
            a_, b_ = np.zeros(Lh - window, bool), np.zeros(Lh - window, bool)
            a_[g[: K - window]] = True
            b_[want[: K - window]] = True
            assert np.array_equal(a_[sure], b_[sure]), (s, h)
