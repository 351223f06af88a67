"""The fused decode step (attn_decode_nonuniform_append) at full size: the
Qwen2.5-32B-shaped batch and the mixed-length batch, three steps each,
compared bit for bit with kv_append + attn_decode_nonuniform on a twin
context, then every session against the oracle.  The oracle's pools are
the generator-filled pools copied before the steps, with the appended rows
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
    sp = F.spec
    # the whole pools before any append (generator-filled)
    pk, pv = u16(F.kpool), u16(F.vpool)
    fk, fv = pk.reshape(-1, D), pv.reshape(-1, D)
    active = np.nonzero(sp.active)[0]
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
        for c in (A, F):                       # the oracle pager's positions, then L += 1
            st, pos = c.spec.append_positions()
            assert st == pg.OK
        for s in active:
            for h in range(H):
                row = sp.physical_row(int(s), h, int(pos[s, h]))
                fk[row], fv[row] = kh[s, h], vh[s, h]
        assert np.array_equal(nup.get_lengths(F.ctx), sp.lengths)
    assert torch.equal(A.kpool, F.kpool) and torch.equal(A.vpool, F.vpool)
    assert nup.device_errors(F.ctx) == nup.NUP_OK

    ref, ref_lse = oracle.decode(u16(F.q), pk, pv, sp.page_table, sp.lengths, sp.group_of_head,
                                 sp.slot_of_head, F.scale)
    out = F.out.cpu().numpy().astype(np.float64)
    lse = F.lse.cpu().numpy().astype(np.float64)
    assert_attention_close(out, lse, ref, ref_lse, f"{name} fused, every session")
