"""Randomised parity: shapes, grouping, layers, plan sizes, page orders,
Reserve / Trim / append sequences and lengths drawn by hypothesis, with the
append made by kv_append or by the fused append + attention call; every
example is checked against the oracle at the acceptance bar (attention)
and bit for bit (pool after appends)."""
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


# NUP_FUZZ_EXAMPLES raises the count for a longer soak of passing code
@settings(max_examples=int(os.environ.get("NUP_FUZZ_EXAMPLES", "60")), deadline=None, derandomize=True,
          suppress_health_check=list(HealthCheck))
@given(st.data())
def test_random_shapes_and_edits(data):
    D = data.draw(st.sampled_from([64, 128]))
    gqa = data.draw(st.sampled_from([1, 2, 4, 5, 8]))
    H = data.draw(st.sampled_from([1, 2, 4, 8]))
    NL = data.draw(st.sampled_from([1, 1, 2, 3]))
    V = NL * H
    ng = data.draw(st.sampled_from([g for g in range(1, V + 1) if V % g == 0]))
    B = data.draw(st.integers(1, 5))
    maxL = data.draw(st.sampled_from([20, 200, 1500]))
    max_pages = (maxL + 40) // 16 + 1
    num_pages = B * ng * max_pages + data.draw(st.integers(0, 20))
    workers = data.draw(st.sampled_from([1, 7, 64, 300, 0]))
    seed = data.draw(st.integers(0, 2 ** 16))
    rs = np.random.default_rng(seed)
    c = Case(H=H, Hq=H * gqa, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages,
             free_list_init=rs.permutation(num_pages), num_workers=workers, salt=seed % 97 + 1,
             num_layers=NL)
    live = np.zeros(B, bool)
    for step in range(data.draw(st.integers(1, 4))):
        if step == 0 or data.draw(st.booleans()):
            idle = np.nonzero(~live)[0]
            if len(idle):
                slots = rs.choice(idle, size=int(rs.integers(1, len(idle) + 1)), replace=False)
                L = rs.integers(0, maxL + 1, size=(len(slots), V))
                L[rs.random(L.shape) < 0.15] = 0
                L[rs.random(L.shape) < 0.15] = 1
                caps = L + rs.integers(0, 40, size=L.shape)
                assert c.alloc(slots.tolist(), caps, L) == pg.OK
                live[slots] = True
        elif live.any():
            slots = rs.choice(np.nonzero(live)[0], size=1)
            c.free(slots.tolist())
            live[slots] = False
    c.commit()
    qs = [torch.from_numpy(W.normal_bf16("q", (B, H * gqa, D), seed + l).view(np.int16)).to(DEV)
          .view(torch.bfloat16) for l in range(NL)]
    # one append per layer where every live head has room: kv_append, or
    # (drawn) the fused append + attention call, checked as it goes
    fused = data.draw(st.booleans())
    kp, vp = u16(c.kpool).copy(), u16(c.vpool).copy()
    fk, fv = kp.reshape(-1, D), vp.reshape(-1, D)
    tag = f"seed {seed} D{D} gqa{gqa} H{H} NL{NL} ng{ng} B{B} W{workers} fused {fused}"

    def check(l):
        torch.cuda.synchronize()
        sl = slice(l * H, (l + 1) * H)
        ref, ref_lse = oracle.decode(u16(qs[l]), kp, vp, c.spec.page_table, c.spec.lengths[:, sl],
                                     c.spec.group_of_head[sl], c.spec.slot_of_head[sl], c.scale)
        assert_attention_close(c.out.cpu().numpy().astype(np.float64),
                               c.lse.cpu().numpy().astype(np.float64), ref, ref_lse, f"{tag} layer {l}")

    for l in range(NL):
        sl = slice(l * H, (l + 1) * H)
        room = (c.spec.lengths[live][:, sl] < c.spec.caps[live][:, sl]).all()
        nup.set_layer(c.ctx, l)
        if room:
            kn = W.normal_bf16("k", (B, H, D), seed + 100 + l)
            vn = W.normal_bf16("v", (B, H, D), seed + 100 + l)
            kd, vd = torch.from_numpy(kn.view(np.int16)).to(DEV), torch.from_numpy(vn.view(np.int16)).to(DEV)
            if fused:
                nup.attn_decode_nonuniform_append(c.ctx, kd, vd, qs[l], c.out, c.lse, c.scale, c.ws)
            else:
                nup.kv_append(c.ctx, kd, vd)
            for s in np.nonzero(live)[0]:
                for h in range(H):
                    v = l * H + h
                    row = c.spec.physical_row(s, v, int(c.spec.lengths[s, v]))
                    fk[row], fv[row] = kn[s, h], vn[s, h]
                    c.spec.lengths[s, v] += 1
        if fused:
            if not room:
                nup.attn_decode_nonuniform(c.ctx, qs[l], c.out, c.lse, c.scale, c.ws)
            check(l)
    torch.cuda.synchronize()
    assert np.array_equal(nup.get_lengths(c.ctx), c.spec.lengths)
    assert np.array_equal(u16(c.kpool), kp) and np.array_equal(u16(c.vpool), vp)
    assert nup.device_errors(c.ctx) == nup.NUP_OK
    if not fused:
        for l in range(NL):
            nup.set_layer(c.ctx, l)
            nup.attn_decode_nonuniform(c.ctx, qs[l], c.out, c.lse, c.scale, c.ws)
            check(l)
