"""Shared set-up for the GPU parity tests: device pools drawn by the input
generators, a library context, and the oracle's own pager state for the same
inputs (the oracle never sees anything the HIP path produced)."""
import math

import numpy as np
import torch

import non_uniform_paged_amd as nup
import oracle
from oracle import pager as pg
from workloads import fill_normal_bf16_torch, normal_bf16

DEV = "cuda"
MAX_ABS, REL_L2 = 1e-2, 5e-3          # acceptance bar
REL_L2_BUG = 1e-4                     # fp32 accumulation lands far below this


def u16(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 numpy (raw bits)."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class Case:
    def __init__(self, *, H, Hq, D, ng, B, num_pages, max_pages, free_list_init=None,
                 num_workers=0, plan_mode=0, uniform_splits=0, salt=0, num_layers=1, merge_mode=0):
        self.H, self.Hq, self.D, self.ng, self.B = H, Hq, D, ng, B
        self.NL, self.V = num_layers, num_layers * H      # the pager's (layer, head) pairs
        self.gh = self.V // ng
        self.num_pages, self.max_pages = num_pages, max_pages
        self.kpool = torch.empty((num_pages, self.gh, 16, D), dtype=torch.bfloat16, device=DEV)
        self.vpool = torch.empty_like(self.kpool)
        fill_normal_bf16_torch(self.kpool, "k", salt)
        fill_normal_bf16_torch(self.vpool, "v", salt)
        cfg = dict(num_kv_heads=H, num_q_heads=Hq, head_dim=D, num_groups=ng, max_batch=B,
                   num_pages=num_pages, max_pages=max_pages, num_workers=num_workers,
                   plan_mode=plan_mode, uniform_splits=uniform_splits, num_layers=num_layers,
                   merge_mode=merge_mode)
        self.desc = torch.empty(nup.desc_bytes(**cfg), dtype=torch.uint8, device=DEV)
        self.ctx = nup.Context(**cfg, k_pool=self.kpool, v_pool=self.vpool, desc=self.desc,
                               free_list_init=free_list_init)
        self.spec = pg.PagerSpec(self.V, ng, B, num_pages, max_pages, 16, free_list_init)
        self.q = torch.from_numpy(normal_bf16("q", (B, Hq, D), salt).view(np.int16)).to(DEV).view(torch.bfloat16)
        self.ws = torch.empty(nup.workspace_bytes(self.ctx), dtype=torch.uint8, device=DEV)
        self.out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        self.lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
        self.scale = 1.0 / math.sqrt(D)

    def alloc(self, slots, caps, lengths=None):
        a = self.spec.alloc(slots, caps, lengths)
        b = nup.kv_alloc_groups(self.ctx, slots, caps, lengths, raise_on_error=False)
        assert a == b
        return a

    def alias(self, slots, src_slots, share_pages, caps, lengths):
        a = self.spec.alias(slots, src_slots, share_pages, caps, lengths)
        b = nup.kv_alias(self.ctx, slots, src_slots, share_pages, caps, lengths, raise_on_error=False)
        assert a == b
        return a

    def free(self, slots):
        a = self.spec.free_seqs(slots)
        b = nup.kv_free_seqs(self.ctx, slots, raise_on_error=False)
        assert a == b

    def commit(self):
        nup.nup_commit(self.ctx)

    def attend(self):
        nup.attn_decode_nonuniform(self.ctx, self.q, self.out, self.lse, self.scale, self.ws)
        torch.cuda.synchronize()
        return self.out.cpu().numpy().astype(np.float64), self.lse.cpu().numpy().astype(np.float64)

    def oracle(self, slots=None, tokens=None):
        """fp64 reference from the oracle's own pager state (full pools)."""
        assert np.array_equal(nup.get_page_table(self.ctx), self.spec.page_table)
        return oracle.decode(u16(self.q), u16(self.kpool), u16(self.vpool), self.spec.page_table,
                             self.spec.lengths, self.spec.group_of_head, self.spec.slot_of_head,
                             self.scale, tokens=tokens)


def assert_attention_close(out, lse, ref_out, ref_lse, what=""):
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    diff = np.abs(out - ref_out)
    max_abs = float(diff.max()) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref_out))
    rel = float(np.linalg.norm(out - ref_out)) / nrm if nrm > 0 else float(np.linalg.norm(out))
    assert max_abs <= MAX_ABS, f"{what}: max-abs {max_abs}"
    assert rel <= REL_L2, f"{what}: rel-L2 {rel}"
    assert rel <= REL_L2_BUG, f"{what}: rel-L2 {rel} (passes the bar but fp32 should do better)"
    neg = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), neg), f"{what}: -inf pattern of lse differs"
    if (~neg).any():
        assert float(np.abs(lse[~neg] - ref_lse[~neg]).max()) <= 1e-3, f"{what}: lse"
    return max_abs, rel
