"""The fused decode step (attn_decode_nonuniform_append) at full size: the
Qwen2.5-32B-shaped batch and the mixed-length batch, three steps each,
compared bit for bit with kv_append + attn_decode_nonuniform on a twin
context, then sampled sessions against the oracle.  The oracle's pools are
the generator-filled pages copied before the steps with the appended rows
placed by the oracle pager's own addressing."""
import math

import numpy as np
import pytest
import torch

import non_uniform_paged_amd as nup
import oracle
import workloads as W
from oracle import pager as pg
from tests.gpu_common import DEV, Case, assert_attention_close, u16

pytestmark = pytest.mark.gpu


def _twin(w, max_pages):
    kw = dict(H=w.num_kv_heads, Hq=w.num_q_heads, D=w.head_dim, ng=w.num_groups, B=w.batch,
              num_pages=w.num_pages, max_pages=max_pages, free_list_init=w.free_list_init)
    return Case(**kw), Case(**kw)


@pytest.mark.parametrize("name", ["qwen25_32b", "mixed_churn"])
def test_fused_append_full_size(name):
    w = W.CONFIGS[name]()
    max_pages = int(math.ceil((w.caps.max() + 16) / 16))
    A, F = _twin(w, max_pages)
    caps = (w.caps + 16).astype(np.int32)     # room for the steps
    for c in (A, F):
        assert c.alloc(list(range(w.batch)), caps, w.lengths) == pg.OK
        c.commit()
    B, H, D = w.batch, w.num_kv_heads, w.head_dim
    seqs = [0, B // 3, B - 1]
    sp = F.spec
    # the sampled sessions' pages before any append (generator-filled)
    sub_pt = sp.page_table[:, seqs, :]
    used = np.unique(sub_pt[sub_pt >= 0])
    remap = np.full(sp.num_pages, -1, np.int64)
    remap[used] = np.arange(len(used))
    sel = torch.from_numpy(used.astype(np.int64)).to(DEV)
    pk, pv = u16(F.kpool.index_select(0, sel)).copy(), u16(F.vpool.index_select(0, sel)).copy()
    fk, fv = pk.reshape(-1, D), pv.reshape(-1, D)
    gh = sp.g_h
    for step in range(3):
        kn = torch.from_numpy(W.normal_bf16("k", (B, H, D), 500 + step).view(np.int16)).to(DEV).view(torch.bfloat16)
        vn = torch.from_numpy(W.normal_bf16("v", (B, H, D), 500 + step).view(np.int16)).to(DEV).view(torch.bfloat16)
        nup.kv_append(A.ctx, kn, vn)
        nup.attn_decode_nonuniform(A.ctx, A.q, A.out, A.lse, A.scale, A.ws)
        nup.attn_decode_nonuniform_append(F.ctx, kn, vn, F.q, F.out, F.lse, F.scale, F.ws)
        torch.cuda.synchronize()
        assert torch.equal(A.out, F.out) and torch.equal(A.lse, F.lse), step
        assert np.array_equal(nup.get_lengths(A.ctx), nup.get_lengths(F.ctx))
        kh, vh = u16(kn), u16(vn)
        for s in seqs:
            for h in range(H):
                t = int(sp.lengths[s, h])
                g = int(sp.group_of_head[h])
                pid = int(remap[sp.page_table[g, s, t // 16]])
                row = (pid * gh + int(sp.slot_of_head[h])) * 16 + t % 16
                fk[row], fv[row] = kh[s, h], vh[s, h]
        for c in (A, F):
            c.spec.lengths[c.spec.active] += 1
        assert np.array_equal(nup.get_lengths(F.ctx), sp.lengths)
    assert torch.equal(A.kpool, F.kpool) and torch.equal(A.vpool, F.vpool)
    assert nup.device_errors(F.ctx) == nup.NUP_OK

    pt = np.where(sub_pt >= 0, remap[np.maximum(sub_pt, 0)], -1).astype(np.int32)
    ref, ref_lse = oracle.decode(u16(F.q)[seqs], pk, pv, pt, sp.lengths[seqs], sp.group_of_head,
                                 sp.slot_of_head, F.scale)
    out = F.out.cpu().numpy().astype(np.float64)[seqs]
    lse = F.lse.cpu().numpy().astype(np.float64)[seqs]
    assert_attention_close(out, lse, ref, ref_lse, f"{name} fused, sampled")
