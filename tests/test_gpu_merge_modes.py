"""The two places split heads are merged (nupaged.h NUP_MERGE_LAUNCH and
NUP_MERGE_IN_SPLIT) on twin contexts: the same arithmetic in the same row
order, so outputs, lse, lengths and pools must agree bit for bit, and both
with the oracle.  Inputs change between launches, so a merge that read a
stale partial of an earlier launch would show."""
import math

import numpy as np
import pytest
import torch

import non_uniform_paged_amd as nup
import workloads as W
from oracle import pager as pg
from tests.gpu_common import DEV, Case, assert_attention_close, u16

pytestmark = pytest.mark.gpu


def _twins(seed, B, H, gqa, D, ng, maxL, workers, plan_mode=nup.PLAN_BALANCED, pad=40, minL=0):
    rs = np.random.default_rng(seed)
    L = rs.integers(max(minL, 1), maxL + 1, size=(B, H)).astype(np.int32)
    if minL == 0:
        L[rs.random((B, H)) < 0.1] = 0
    caps = (L + rs.integers(8, pad, size=(B, H))).astype(np.int32)
    max_pages = int(math.ceil(caps.max() / 16)) + 1
    num_pages = B * ng * max_pages + 9
    perm = rs.permutation(num_pages)
    kw = dict(H=H, Hq=H * gqa, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages,
              free_list_init=perm, num_workers=workers, plan_mode=plan_mode, uniform_splits=3, salt=seed)
    return Case(**kw, merge_mode=nup.MERGE_LAUNCH), Case(**kw, merge_mode=nup.MERGE_IN_SPLIT), L, caps


def _new_q(c, salt):
    q = W.normal_bf16("q", (c.B, c.Hq, c.D), salt)
    c.q.copy_(torch.from_numpy(q.view(np.int16)).to(DEV).view(torch.bfloat16))


@pytest.mark.parametrize("D,gqa,H,ng,workers,plan_mode,seed", [
    (128, 5, 8, 4, 2048, nup.PLAN_BALANCED, 1), (128, 4, 8, 2, 37, nup.PLAN_BALANCED, 2),
    (64, 1, 4, 2, 5, nup.PLAN_BALANCED, 3), (128, 8, 4, 1, 64, nup.PLAN_UNIFORM, 4),
    (64, 2, 8, 8, 300, nup.PLAN_UNIFORM, 5), (128, 5, 8, 4, 1, nup.PLAN_BALANCED, 6)])
def test_paged_merge_modes_agree(D, gqa, H, ng, workers, plan_mode, seed):
    print(f"merge modes: paged D{D} gqa{gqa} H{H} ng{ng} W{workers} plan{plan_mode}", flush=True)
    A, S, L, caps = _twins(seed, 5, H, gqa, D, ng, 1500, workers, plan_mode)
    for c in (A, S):
        assert c.alloc([0, 1, 3, 4], caps[[0, 1, 3, 4]], L[[0, 1, 3, 4]]) == pg.OK   # slot 2 inactive
        c.commit()
    for it in range(3):
        for c in (A, S):
            _new_q(c, 100 * seed + it)
        oa, la = A.attend()
        os_, ls = S.attend()
        assert np.array_equal(oa, os_) and np.array_equal(la, ls), f"launch {it}"
        ref, ref_lse = S.oracle()
        assert_attention_close(os_, ls, ref, ref_lse, f"in-split merge, launch {it}")


@pytest.mark.parametrize("K,gqa,seed", [(2048, 4, 11), (96, 5, 12), (37, 2, 13)])
def test_topk_merge_modes_agree(K, gqa, seed):
    print(f"merge modes: top-K {K} gqa{gqa}", flush=True)
    A, S, L, caps = _twins(seed, 3, 8, gqa, 128, 1, 3000, 0, minL=K)
    for c in (A, S):
        assert c.alloc([0, 2], caps[[0, 2]], L[[0, 2]]) == pg.OK                  # slot 1 inactive
        c.commit()
    lens = np.where(A.spec.active[:, None], A.spec.lengths, K)
    idx = W.topk_indices(lens, K, salt=seed)
    idx_d = torch.from_numpy(idx).to(DEV)
    ws = {id(c): torch.empty(nup.workspace_bytes(c.ctx, K), dtype=torch.uint8, device=DEV) for c in (A, S)}
    for it in range(3):
        res = []
        for c in (A, S):
            _new_q(c, 100 * seed + it)
            nup.attn_decode_topk_paged(c.ctx, c.q, idx_d, K, c.out, c.lse, c.scale, ws[id(c)])
            torch.cuda.synchronize()
            res.append((c.out.cpu().numpy().copy(), c.lse.cpu().numpy().copy()))
        assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1]), f"launch {it}"
        ref, ref_lse = S.oracle(tokens=idx)
        assert_attention_close(res[1][0].astype(np.float64), res[1][1].astype(np.float64), ref, ref_lse,
                               f"in-split top-K, launch {it}")


def test_fused_append_merge_modes_agree():
    """The fused step, three times: the in-split merge advances each head's
    length from the wave that finishes it; pools, lengths and outputs match
    the merge launch's bit for bit, and the oracle at the end."""
    print("merge modes: fused append", flush=True)
    A, S, L, caps = _twins(21, 6, 8, 5, 128, 4, 2500, 2048)
    for c in (A, S):
        assert c.alloc(list(range(6)), caps, L) == pg.OK
        c.commit()
    D = 128
    fk, fv = u16(S.kpool).reshape(-1, D), u16(S.vpool).reshape(-1, D)
    for step in range(3):
        kn = torch.from_numpy(W.normal_bf16("k", (6, 8, D), 600 + step).view(np.int16)).to(DEV).view(torch.bfloat16)
        vn = torch.from_numpy(W.normal_bf16("v", (6, 8, D), 600 + step).view(np.int16)).to(DEV).view(torch.bfloat16)
        for c in (A, S):
            _new_q(c, 700 + step)
            nup.attn_decode_nonuniform_append(c.ctx, kn, vn, c.q, c.out, c.lse, c.scale, c.ws)
        torch.cuda.synchronize()
        assert torch.equal(A.out, S.out) and torch.equal(A.lse, S.lse), step
        kh, vh = u16(kn), u16(vn)
        for c in (A, S):
            st, pos = c.spec.append_positions()
            assert st == pg.OK
        for s in range(6):
            for h in range(8):
                row = S.spec.physical_row(s, h, int(pos[s, h]))
                fk[row], fv[row] = kh[s, h], vh[s, h]
        assert np.array_equal(nup.get_lengths(S.ctx), S.spec.lengths)
    assert torch.equal(A.kpool, S.kpool) and torch.equal(A.vpool, S.vpool)
    assert nup.device_errors(S.ctx) == nup.NUP_OK
    # the device lengths: a commit after a Trim sends the shadow, and the
    # attention over them agrees with the oracle
    for c in (A, S):
        c.free([4])
        c.commit()
    out, lse = S.attend()
    import oracle
    ref, ref_lse = oracle.decode(u16(S.q), fk.reshape(u16(S.kpool).shape), fv.reshape(u16(S.vpool).shape),
                                 S.spec.page_table, S.spec.lengths, S.spec.group_of_head, S.spec.slot_of_head,
                                 S.scale)
    assert_attention_close(out, lse, ref, ref_lse, "in-split fused step")
    oa, la = A.attend()
    assert np.array_equal(oa, out) and np.array_equal(la, lse)


def test_full_size_merge_modes_agree():
    """The Qwen2.5-32B batch at the bench's launch: both merge places give the
    same bits."""
    print("merge modes: qwen25_32b full size", flush=True)
    w = W.qwen25_32b()
    out = []
    for mode in (nup.MERGE_LAUNCH, nup.MERGE_IN_SPLIT):
        c = Case(H=w.num_kv_heads, Hq=w.num_q_heads, D=w.head_dim, ng=w.num_groups, B=w.batch,
                 num_pages=w.num_pages, max_pages=int(math.ceil(w.caps.max() / 16)),
                 free_list_init=w.free_list_init, merge_mode=mode)
        c.alloc(list(range(w.batch)), w.caps, w.lengths)
        c.commit()
        out.append(c.attend())
        del c
        torch.cuda.empty_cache()
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][1], out[1][1])
