"""Pins for the fp64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: a pure-Python
brute force over logically stored rows, torch's own attention routine in fp64
(full budget = dense attention; uniform budget with one group = standard paged
attention), closed forms, and invariants of the definition (page placement,
merging of split token lists).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from workloads import bf16_bits_to_f64, f32_to_bf16_bits


def _scatter_pool(k_log, v_log, lengths, page_table, group_of_head, slot_of_head,
                  num_pages, P):
    """Place logical rows into a [num_pages][G_h][P][D] pool with numpy's
    multi-dimensional indexing (the layout definition, stated independently
    of the oracle's address arithmetic)."""
    B, H = lengths.shape
    D = k_log[0][0].shape[-1] if k_log[0][0].size else k_log[0][1].shape[-1]
    n_g = page_table.shape[0]
    G_h = H // n_g
    rs = np.random.default_rng(7)
    pk = f32_to_bf16_bits(rs.standard_normal((num_pages, G_h, P, D), dtype=np.float32))
    pv = f32_to_bf16_bits(rs.standard_normal((num_pages, G_h, P, D), dtype=np.float32))
    for s in range(B):
        for h in range(H):
            g, j = group_of_head[h], slot_of_head[h]
            for t in range(lengths[s, h]):
                page = page_table[g, s, t // P]
                pk[page, j, t % P] = k_log[s][h][t]
                pv[page, j, t % P] = v_log[s][h][t]
    return pk, pv


def _random_case(seed, B=2, H=4, n_g=2, gqa=2, D=16, P=4, maxL=40, num_pages=None):
    rs = np.random.default_rng(seed)
    G_h = H // n_g
    lengths = rs.integers(0, maxL + 1, size=(B, H)).astype(np.int32)
    group_of_head = rs.permutation(np.repeat(np.arange(n_g), G_h)).astype(np.int32)
    slot_of_head = np.zeros(H, np.int32)
    for g in range(n_g):
        hs = np.nonzero(group_of_head == g)[0]
        slot_of_head[hs] = rs.permutation(len(hs))
    max_pages = math.ceil(maxL / P)
    need = B * n_g * max_pages
    num_pages = num_pages or need + 5
    perm = rs.permutation(num_pages)
    page_table = perm[:need].reshape(n_g, B, max_pages).astype(np.int32)
    k_log = [[f32_to_bf16_bits(rs.standard_normal((lengths[s, h], D), dtype=np.float32))
              for h in range(H)] for s in range(B)]
    v_log = [[f32_to_bf16_bits(rs.standard_normal((lengths[s, h], D), dtype=np.float32))
              for h in range(H)] for s in range(B)]
    pk, pv = _scatter_pool(k_log, v_log, lengths, page_table, group_of_head,
                           slot_of_head, num_pages, P)
    q = f32_to_bf16_bits(rs.standard_normal((B, H * gqa, D), dtype=np.float32))
    return dict(q=q, pk=pk, pv=pv, pt=page_table, L=lengths, goh=group_of_head,
                soh=slot_of_head, k_log=k_log, v_log=v_log, gqa=gqa, D=D)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    c = _random_case(seed)
    scale = 1.0 / math.sqrt(c["D"])
    out, lse = oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], c["L"], c["goh"],
                             c["soh"], scale, num_threads=2)
    B, Hq, D = c["q"].shape
    for s in range(B):
        for r in range(Hq):
            h = r // c["gqa"]
            keys = [list(bf16_bits_to_f64(row)) for row in c["k_log"][s][h]]
            vals = [list(bf16_bits_to_f64(row)) for row in c["v_log"][s][h]]
            o_ref, lse_ref = brute.attend(list(bf16_bits_to_f64(c["q"][s, r])), keys, vals, scale)
            np.testing.assert_allclose(out[s, r], o_ref, rtol=0, atol=1e-12)
            if math.isinf(lse_ref):
                assert math.isinf(lse[s, r]) and lse[s, r] < 0
            else:
                assert abs(lse[s, r] - lse_ref) <= 1e-12


def test_full_budget_equals_dense_sdpa():
    """Every head keeps its whole context: the result is dense softmax
    attention, computed here by torch's scaled_dot_product_attention in fp64."""
    rs = np.random.default_rng(11)
    B, H, gqa, D, P, ctx, n_g = 2, 4, 3, 32, 8, 50, 2
    lengths = np.full((B, H), ctx, np.int32)
    c = _random_case(11, B=B, H=H, n_g=n_g, gqa=gqa, D=D, P=P, maxL=ctx)
    # rebuild with every head at full context
    k_log = [[f32_to_bf16_bits(rs.standard_normal((ctx, D), dtype=np.float32)) for _ in range(H)]
             for _ in range(B)]
    v_log = [[f32_to_bf16_bits(rs.standard_normal((ctx, D), dtype=np.float32)) for _ in range(H)]
             for _ in range(B)]
    pk, pv = _scatter_pool(k_log, v_log, lengths, c["pt"], c["goh"], c["soh"],
                           c["pk"].shape[0], P)
    scale = 1.0 / math.sqrt(D)
    out, lse = oracle.decode(c["q"], pk, pv, c["pt"], lengths, c["goh"], c["soh"], scale)
    q = torch.from_numpy(bf16_bits_to_f64(c["q"])).view(B, H * gqa, 1, D)
    K = torch.from_numpy(np.stack([[bf16_bits_to_f64(k_log[s][h]) for h in range(H)] for s in range(B)]))
    V = torch.from_numpy(np.stack([[bf16_bits_to_f64(v_log[s][h]) for h in range(H)] for s in range(B)]))
    K = K.repeat_interleave(gqa, dim=1)
    V = V.repeat_interleave(gqa, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=scale)
    np.testing.assert_allclose(out, ref.view(B, H * gqa, D).numpy(), rtol=0, atol=1e-12)
    ref_lse = torch.logsumexp(scale * (q @ K.transpose(-1, -2)), dim=-1).view(B, H * gqa)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=0, atol=1e-12)


def test_uniform_budget_one_group_equals_standard_paged():
    """One group holding every head and the same budget for all heads is the
    standard paged cache: gather pages with index_select, then attend."""
    rs = np.random.default_rng(12)
    B, H, gqa, D, P, L, num_pages = 3, 4, 2, 16, 16, 70, 40
    max_pages = math.ceil(L / P)
    pool_k = f32_to_bf16_bits(rs.standard_normal((num_pages, H, P, D), dtype=np.float32))
    pool_v = f32_to_bf16_bits(rs.standard_normal((num_pages, H, P, D), dtype=np.float32))
    pt = rs.permutation(num_pages)[:B * max_pages].reshape(1, B, max_pages).astype(np.int32)
    lengths = np.full((B, H), L, np.int32)
    goh = np.zeros(H, np.int32)
    soh = np.arange(H, dtype=np.int32)
    q = f32_to_bf16_bits(rs.standard_normal((B, H * gqa, D), dtype=np.float32))
    scale = 1.0 / math.sqrt(D)
    out, _ = oracle.decode(q, pool_k, pool_v, pt, lengths, goh, soh, scale)
    tk = torch.from_numpy(bf16_bits_to_f64(pool_k))
    tv = torch.from_numpy(bf16_bits_to_f64(pool_v))
    for s in range(B):
        idx = torch.from_numpy(pt[0, s].astype(np.int64))
        Ks = tk.index_select(0, idx).permute(1, 0, 2, 3).reshape(H, -1, D)[:, :L]
        Vs = tv.index_select(0, idx).permute(1, 0, 2, 3).reshape(H, -1, D)[:, :L]
        Ks = Ks.repeat_interleave(gqa, dim=0)
        Vs = Vs.repeat_interleave(gqa, dim=0)
        qs = torch.from_numpy(bf16_bits_to_f64(q[s])).view(H * gqa, 1, D)
        ref = torch.nn.functional.scaled_dot_product_attention(qs, Ks, Vs, scale=scale)
        np.testing.assert_allclose(out[s], ref.view(H * gqa, D).numpy(), rtol=0, atol=1e-12)


def test_length_one_returns_v_exactly():
    c = _random_case(3, maxL=1)
    c["L"][:] = 1
    out, lse = oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], c["L"], c["goh"], c["soh"], 0.3)
    B, Hq, D = c["q"].shape
    for s in range(B):
        for r in range(Hq):
            h = r // c["gqa"]
            page = c["pt"][c["goh"][h], s, 0]
            v0 = bf16_bits_to_f64(c["pv"][page, c["soh"][h], 0])
            assert np.array_equal(out[s, r], v0)


def test_zero_query_gives_mean_and_log_length():
    c = _random_case(4, maxL=37)
    c["L"][0, 0] = 0
    c["q"][:] = 0
    out, lse = oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], c["L"], c["goh"], c["soh"], 0.25)
    B, Hq, D = c["q"].shape
    for s in range(B):
        for r in range(Hq):
            h = r // c["gqa"]
            L = c["L"][s, h]
            if L == 0:
                assert np.all(out[s, r] == 0) and lse[s, r] == -np.inf
                continue
            mean = np.mean([bf16_bits_to_f64(v) for v in c["v_log"][s][h]], axis=0)
            np.testing.assert_allclose(out[s, r], mean, rtol=0, atol=1e-13)
            assert abs(lse[s, r] - math.log(L)) < 1e-13


def test_constant_values():
    c = _random_case(5, maxL=33)
    c["pv"][:] = f32_to_bf16_bits(np.full(1, 1.375, np.float32))[0]
    out, _ = oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], c["L"], c["goh"], c["soh"], 0.25)
    mask = np.repeat(c["L"] > 0, c["gqa"], axis=1)
    assert np.all(np.abs(out[mask] - 1.375) <= 1.375 * 1e-14 * 33)


def test_page_permutation_bit_identical():
    """Moving pages to other physical places (data moved with them) leaves
    the result bit-identical: the definition never looks at placement."""
    c = _random_case(6, maxL=60)
    out1, lse1 = oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], c["L"], c["goh"], c["soh"], 0.2)
    num_pages = c["pk"].shape[0]
    perm = np.random.default_rng(99).permutation(num_pages)
    pk2 = np.empty_like(c["pk"])
    pv2 = np.empty_like(c["pv"])
    pk2[perm] = c["pk"]
    pv2[perm] = c["pv"]
    pt2 = perm[c["pt"]].astype(np.int32)
    out2, lse2 = oracle.decode(c["q"], pk2, pv2, pt2, c["L"], c["goh"], c["soh"], 0.2)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_split_token_lists_merge_to_whole():
    """Attention over two halves of the token list, merged by log-sum-exp,
    equals attention over the whole list (Flash-Decoding's split-K identity)."""
    c = _random_case(8, maxL=64)
    c["L"][:] = np.maximum(c["L"], 2)
    B, H = c["L"].shape
    L = 2 * (int(c["L"].min()) // 2)
    toks = np.tile(np.arange(L, dtype=np.int32), (B, H, 1))
    out_all, lse_all = oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], c["L"], c["goh"], c["soh"],
                                     0.3, tokens=toks)
    o1, l1 = oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], c["L"], c["goh"], c["soh"], 0.3,
                           tokens=toks[..., : L // 2])
    o2, l2 = oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], c["L"], c["goh"], c["soh"], 0.3,
                           tokens=toks[..., L // 2:])
    M = np.maximum(l1, l2)
    w1 = np.exp(l1 - M)
    w2 = np.exp(l2 - M)
    merged = (w1[..., None] * o1 + w2[..., None] * o2) / (w1 + w2)[..., None]
    np.testing.assert_allclose(merged, out_all, rtol=0, atol=1e-12)
    np.testing.assert_allclose(M + np.log(w1 + w2), lse_all, rtol=0, atol=1e-12)


def test_token_list_of_all_positions_equals_length_mode():
    c = _random_case(9, maxL=48)
    c["L"][:] = np.maximum(c["L"], 1)
    B, H = c["L"].shape
    # use the common minimum so the list is valid for every head
    L = int(c["L"].min())
    lengths = np.full_like(c["L"], L)
    toks = np.tile(np.arange(L, dtype=np.int32), (B, H, 1))
    a = oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], lengths, c["goh"], c["soh"], 0.3)
    b = oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], lengths, c["goh"], c["soh"], 0.3, tokens=toks)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_out_of_range_token_rejected():
    c = _random_case(10, maxL=20)
    c["L"][:] = 5
    toks = np.full((2, 4, 2), 5, np.int32)
    with pytest.raises(ValueError):
        oracle.decode(c["q"], c["pk"], c["pv"], c["pt"], c["L"], c["goh"], c["soh"], 0.3, tokens=toks)
