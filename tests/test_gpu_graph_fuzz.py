"""Randomised graph replays: shapes, layers, grouping, plan mode and the
Reserve / Trim edits between replays are drawn by hypothesis.  A decode
step (fused or separate append + attention in every layer) is captured once
on one context and replayed; a twin context makes the same calls eagerly.
Outputs, pools and lengths must agree bit for bit after every replay."""
import os

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import non_uniform_paged_amd as nup
import workloads as W
from oracle import pager as pg
from tests.gpu_common import DEV, Case

pytestmark = pytest.mark.gpu


@settings(max_examples=int(os.environ.get("NUP_FUZZ_EXAMPLES", "25")), deadline=None, derandomize=True,
          suppress_health_check=list(HealthCheck))
@given(st.data())
def test_random_graph_replays(data):
    D = data.draw(st.sampled_from([64, 128]))
    gqa = data.draw(st.sampled_from([1, 2, 4, 5, 8]))
    H = data.draw(st.sampled_from([1, 2, 4, 8]))
    NL = data.draw(st.sampled_from([1, 2, 3]))
    V = NL * H
    ng = data.draw(st.sampled_from([g for g in range(1, V + 1) if V % g == 0]))
    B = data.draw(st.integers(1, 5))
    plan_mode = data.draw(st.sampled_from([nup.PLAN_BALANCED, nup.PLAN_UNIFORM, nup.PLAN_SHARED]))
    workers = data.draw(st.sampled_from([1, 7, 64, 0]))
    fused = data.draw(st.booleans())
    replays = data.draw(st.integers(1, 5))
    seed = data.draw(st.integers(0, 2 ** 16))
    rs = np.random.default_rng(seed)
    maxL = 300
    max_pages = (maxL + 60) // 16 + 1
    num_pages = B * ng * max_pages + 5
    perm = rs.permutation(num_pages)
    kw = dict(H=H, Hq=H * gqa, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages,
              free_list_init=perm, num_workers=workers, plan_mode=plan_mode, uniform_splits=3,
              salt=seed % 89 + 1, num_layers=NL)
    G, E = Case(**kw), Case(**kw)
    live = np.zeros(B, bool)

    def reserve():
        idle = np.nonzero(~live)[0]
        if not len(idle):
            return
        slots = rs.choice(idle, size=int(rs.integers(1, len(idle) + 1)), replace=False)
        L = rs.integers(0, maxL + 1, size=(len(slots), V)).astype(np.int32)
        caps = (L + replays + rs.integers(0, 30, size=L.shape)).astype(np.int32)   # room for the replays
        for c in (G, E):
            assert c.alloc(slots.tolist(), caps, L) == pg.OK
        live[slots] = True

    reserve()
    for c in (G, E):
        c.commit()
    kn = [torch.empty((B, H, D), dtype=torch.bfloat16, device=DEV) for _ in range(NL)]
    vn = [torch.empty_like(kn[0]) for _ in range(NL)]
    qs = [torch.empty((B, H * gqa, D), dtype=torch.bfloat16, device=DEV) for _ in range(NL)]
    outs = [torch.empty((B, H * gqa, D), dtype=torch.float32, device=DEV) for _ in range(NL)]
    lses = [torch.empty((B, H * gqa), dtype=torch.float32, device=DEV) for _ in range(NL)]
    e_out = [torch.empty_like(outs[0]) for _ in range(NL)]
    e_lse = [torch.empty_like(lses[0]) for _ in range(NL)]

    def step(c, out, lse):
        for l in range(NL):
            nup.set_layer(c.ctx, l)
            if fused:
                nup.attn_decode_nonuniform_append(c.ctx, kn[l], vn[l], qs[l], out[l], lse[l], c.scale, c.ws)
            else:
                nup.kv_append(c.ctx, kn[l], vn[l])
                nup.attn_decode_nonuniform(c.ctx, qs[l], out[l], lse[l], c.scale, c.ws)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(G, outs, lses)
    for i in range(replays):
        if i > 0 and rs.random() < 0.5:         # the mapping changes between replays
            if live.any() and rs.random() < 0.5:
                s = int(rs.choice(np.nonzero(live)[0]))
                for c in (G, E):
                    c.free([s])
                live[s] = False
            else:
                reserve()
            for c in (G, E):
                c.commit()
        for l in range(NL):
            kn[l].copy_(torch.from_numpy(W.normal_bf16("k", (B, H, D), seed + 10 * i + l).view(np.int16)).to(DEV).view(torch.bfloat16))
            vn[l].copy_(torch.from_numpy(W.normal_bf16("v", (B, H, D), seed + 10 * i + l).view(np.int16)).to(DEV).view(torch.bfloat16))
            qs[l].copy_(torch.from_numpy(W.normal_bf16("q", (B, H * gqa, D), seed + 10 * i + l).view(np.int16)).to(DEV).view(torch.bfloat16))
        g.replay()
        nup.note_appends(G.ctx, 1)
        step(E, e_out, e_lse)
        torch.cuda.synchronize()
        tag = f"seed {seed} replay {i} D{D} gqa{gqa} H{H} NL{NL} ng{ng} B{B} plan{plan_mode} fused {fused}"
        for l in range(NL):
            assert torch.equal(outs[l], e_out[l]) and torch.equal(lses[l], e_lse[l]), f"{tag} layer {l}"
        for c in (G, E):                      # one token per (layer, KV head) of every live slot
            c.spec.lengths[c.spec.active] += 1
        assert np.array_equal(nup.get_lengths(G.ctx), G.spec.lengths), tag
        assert np.array_equal(nup.get_lengths(E.ctx), E.spec.lengths), tag
        assert torch.equal(G.kpool, E.kpool) and torch.equal(G.vpool, E.vpool), tag
    assert nup.device_errors(G.ctx) == nup.NUP_OK
