"""The allocation-free decode attention (attn_decode_nonuniform_noalloc)
against the workspace call it varies (attn_decode_nonuniform), bit for bit,
and against the oracle, on two calls in a row on one GPU, the second with a
smaller input, so the second runs over what the first left in the scratch."""
import math

import numpy as np
import pytest
import torch

import non_uniform_paged_amd as nup
from tests.gpu_common import DEV, Case, assert_attention_close

pytestmark = pytest.mark.gpu


def _ragged_case(seed, B, H, gqa, D, ng, maxL, workers=0):
    rs = np.random.default_rng(seed)
    L = rs.integers(1, maxL + 1, size=(B, H)).astype(np.int32)
    L[rs.random((B, H)) < 0.1] = 0
    caps = (L + rs.integers(0, 40, size=(B, H))).astype(np.int32)
    max_pages = int(math.ceil(caps.max() / 16)) + 1
    num_pages = B * ng * max_pages + 11
    c = Case(H=H, Hq=H * gqa, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages,
             free_list_init=rs.permutation(num_pages), num_workers=workers, salt=seed)
    return c, L, caps


def _both(c):
    """(workspace call, allocation-free call) outputs on the same context."""
    ref_out = torch.full_like(c.out, float("nan"))
    ref_lse = torch.full_like(c.lse, float("nan"))
    nup.attn_decode_nonuniform(c.ctx, c.q, ref_out, ref_lse, c.scale, c.ws)
    out = torch.full_like(c.out, float("nan"))
    lse = torch.full_like(c.lse, float("nan"))
    nup.attn_decode_nonuniform_noalloc(c.ctx, c.q, out, lse, c.scale)
    torch.cuda.synchronize()
    return (ref_out, ref_lse), (out, lse)


def test_noalloc_two_calls_second_smaller():
    print("noalloc: call 1, B 6, 8 KV heads, gqa 5, D 128, lengths to 4000", flush=True)
    c1, L, caps = _ragged_case(90, B=6, H=8, gqa=5, D=128, ng=4, maxL=4000)
    c1.alloc(list(range(6)), caps, L)
    c1.commit()
    (ro, rl), (o, l) = _both(c1)
    assert torch.equal(o, ro) and torch.equal(l, rl), "call 1: differs from the workspace call"
    ref, ref_lse = c1.oracle()
    assert_attention_close(o.cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64),
                           ref, ref_lse, "call 1")
    # call 2: a smaller input on another context of the same GPU (fewer,
    # shorter heads; other head dim and GQA), over the scratch call 1 left
    print("noalloc: call 2, B 3, 4 KV heads, gqa 2, D 64, lengths to 300", flush=True)
    c2, L2, caps2 = _ragged_case(91, B=3, H=4, gqa=2, D=64, ng=2, maxL=300, workers=37)
    c2.alloc([0, 2], caps2[[0, 2]], L2[[0, 2]])       # slot 1 inactive
    c2.commit()
    (ro, rl), (o, l) = _both(c2)
    assert torch.equal(o, ro) and torch.equal(l, rl), "call 2: differs from the workspace call"
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(l[1]))
    ref, ref_lse = c2.oracle()
    assert_attention_close(o.cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64),
                           ref, ref_lse, "call 2")
    # and the first context again, after a Trim: smaller than its first call
    c1.free([1, 4])
    c1.commit()
    (ro, rl), (o, l) = _both(c1)
    assert torch.equal(o, ro) and torch.equal(l, rl), "call 3: differs from the workspace call"
    ref, ref_lse = c1.oracle()
    assert_attention_close(o.cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64),
                           ref, ref_lse, "call 3")


def test_noalloc_refuses_partials_beyond_the_scratch():
    """A context whose split-K partials exceed the scratch is refused before
    anything is launched; the output is left alone."""
    print("noalloc: 65536 workers (partials > 32 MiB) must be refused", flush=True)
    c, L, caps = _ragged_case(92, B=2, H=8, gqa=8, D=128, ng=2, maxL=200, workers=65536)
    assert nup.workspace_bytes(c.ctx) > nup.NOALLOC_SCRATCH_BYTES
    c.alloc([0, 1], caps, L)
    c.commit()
    out = torch.full_like(c.out, float("nan"))
    lse = torch.full_like(c.lse, float("nan"))
    st = nup.attn_decode_nonuniform_noalloc(c.ctx, c.q, out, lse, c.scale, raise_on_error=False)
    torch.cuda.synchronize()
    assert st == nup.NUP_E_ARG
    assert torch.isnan(out).all() and torch.isnan(lse).all()
