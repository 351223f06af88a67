"""Copy-engine trains (KV-RM, Fig 2): kv_gather_trains_dma must deliver the
same rows as the oracle's page gather, bit for bit, and write nothing else."""
import numpy as np
import pytest
import torch

import non_uniform_paged_amd as nup
from oracle import pager as pg
from tests.gpu_common import DEV, Case, u16

pytestmark = pytest.mark.gpu

SENTINEL = -12345


def _check_dma_gather(c, gap=5):
    lens = c.spec.lengths.astype(np.int64).reshape(-1)
    row_off = np.concatenate([[0], np.cumsum(lens + gap)[:-1]]).astype(np.int64)
    total = int((lens + gap).sum())
    ks = torch.full((total, c.D), SENTINEL, dtype=torch.int16, device=DEV)
    vs = torch.full_like(ks, SENTINEL)
    n = nup.kv_gather_trains_dma(c.ctx, ks, vs, row_off)
    torch.cuda.synchronize()
    gk, gv = ks.cpu().numpy(), vs.cpu().numpy()
    written = np.zeros(total, bool)
    want = pg.gather_pages(c.spec, u16(c.kpool), u16(c.vpool), row_off)
    for (s, h), (kr, vr, _) in want.items():
        o, m = row_off[s * c.H + h], len(kr)
        assert np.array_equal(gk[o:o + m].view(np.uint16), kr), (s, h)
        assert np.array_equal(gv[o:o + m].view(np.uint16), vr), (s, h)
        written[o:o + m] = True
    assert (gk[~written] == SENTINEL).all() and (gv[~written] == SENTINEL).all()
    return n


@pytest.mark.parametrize("ng", [1, 2, 8])
def test_dma_trains_fragmented(ng):
    H, D, B = 8, 128, 5
    rs = np.random.default_rng(40 + ng)
    L = rs.integers(0, 500, size=(B, H)).astype(np.int32)
    L[0, 0], L[1, 1] = 16, 1                     # exactly one page; a lone row
    caps = L + rs.integers(0, 40, size=(B, H)).astype(np.int32)
    num_pages = B * ng * 40
    c = Case(H=H, Hq=H * 2, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=40,
             free_list_init=rs.permutation(num_pages), salt=40 + ng)
    c.alloc([0, 1, 3], caps[[0, 1, 3]], L[[0, 1, 3]])
    c.free([1])
    c.alloc([2, 4], caps[[2, 4]], L[[2, 4]])     # reuses freed pages: trains break up
    c.commit()
    n = _check_dma_gather(c)
    assert n > 0


def test_dma_trains_over_shared_pages():
    H, D, B, ng = 8, 64, 4, 2
    rs = np.random.default_rng(44)
    L0 = rs.integers(100, 300, size=H)
    c = Case(H=H, Hq=H, D=D, ng=ng, B=B, num_pages=200, max_pages=30,
             free_list_init=rs.permutation(200), salt=44)
    c.alloc([0], (L0 + 10)[None], L0[None])
    goh = c.spec.group_of_head
    share = np.array([[min(L0[h] for h in range(H) if goh[h] == g) // 16 for g in range(ng)]] * 2)
    lens = share[:, goh] * 16 + rs.integers(0, 90, size=(2, H))
    assert c.alias([1, 3], [0, 0], share, lens + 3, lens) == pg.OK
    c.commit()
    _check_dma_gather(c)


def test_dma_trains_refuses_pending_edits():
    H, D, B = 4, 64, 2
    c = Case(H=H, Hq=H, D=D, ng=1, B=B, num_pages=16, max_pages=4, salt=45)
    c.alloc([0], np.full((1, H), 40), np.full((1, H), 33))
    ks = torch.zeros((4 * 64, D), dtype=torch.int16, device=DEV)
    row_off = np.arange(B * H, dtype=np.int64) * 64
    assert nup.kv_gather_trains_dma(c.ctx, ks, ks, row_off, raise_on_error=False) == nup.NUP_E_STATE
    c.commit()
    c.free([0])
    assert nup.kv_gather_trains_dma(c.ctx, ks, ks, row_off, raise_on_error=False) == nup.NUP_E_STATE
