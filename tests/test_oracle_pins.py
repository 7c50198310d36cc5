"""Pins of the fp64 oracle against things other than itself.

Each test names what fixes the expected value: brute force, a library
routine (torch SDPA in float64), a closed form or special case of the
definition, or a property the definition implies.  Together they are chosen
so that a plausible mistake in the oracle (dropped rope term, wrong scale,
transposed weight, wrong head->group map, off-by-one causal mask, wrong page
slot, lse in the wrong base) fails at least one of them.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from decode_attention_gqla_amd.inputs import make_case, random_partials
from oracle import brute
from oracle.gqla_ref import (Dims, bf16_round, combine, decode_absorb_form, decode_gqa_expanded,
                             decode_literal, decode_partials, decode_partials_latent, expand_pages, expanded_offset_k,
                             expanded_offset_rope, expanded_offset_v, expanded_page_elems,
                             _expanded_group_views, _expanded_rope_view, gather_latent)
from tests.oracle_util import dims_of, oracle_args

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")

TINY = dict(h_q=4, g=2, r=8, d_R=4, d_nope=4, d_v=6)


def tiny_case(ctx, s_q, seed, table="random", bs=8, **kw):
    dims = dict(TINY)
    dims.update(kw)
    return make_case(batch=len(ctx), ctx=list(ctx), s_q=s_q, seed=seed, table=table,
                     dtype=torch.float64, bs=bs, **dims)


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --- brute force -----------------------------------------------------------
@pytest.mark.parametrize("s_q", [1, 2])
@pytest.mark.parametrize("ctx", [(2, 3), (63, 64), (65, 130), (8, 9)])
def test_literal_matches_pure_python_brute_force(ctx, s_q):
    case = tiny_case(ctx, s_q, seed=11 + sum(ctx) + s_q)
    d = dims_of(case)
    args = oracle_args(case)
    out, lse = decode_literal(*args, d)
    q_nope, q_rope, pages, bt, sl, w_uk, w_uv = args
    bo, bl = brute.decode(q_nope.tolist(), q_rope.tolist(), pages.tolist(), bt.tolist(),
                          sl.tolist(), w_uk.tolist(), w_uv.tolist(), d.h_q, d.g, d.r, d.d_R,
                          d.d_nope, d.d_v, d.s_q, d.bs)
    assert rel(out, bo) < 1e-12
    assert np.max(np.abs(lse - np.array(bl))) < 1e-12


def test_length_one_context_returns_the_single_value_vector():
    # L = 1, s_q = 1: softmax over one token is 1, so out = c_0 W_UV[G] exactly.
    case = tiny_case((1, 1), 1, seed=5)
    d = dims_of(case)
    args = oracle_args(case)
    out, lse = decode_literal(*args, d)
    _, _, pages, bt, _, _, w_uv = args
    for b in range(2):
        c0 = pages[bt[b, 0], 0, : d.r]
        for h in range(d.h_q):
            G = h // (d.h_q // d.g)
            assert np.allclose(out[b, 0, h], c0 @ w_uv[G], rtol=0, atol=1e-15)


def test_zero_query_gives_mean_of_values():
    case = tiny_case((37, 50), 2, seed=6)
    case.q_nope.zero_()
    case.q_rope.zero_()
    d = dims_of(case)
    args = oracle_args(case)
    out, lse = decode_literal(*args, d)
    _, _, pages, bt, sl, _, w_uv = args
    for b in range(2):
        C, _ = gather_latent(pages, bt[b], int(sl[b]), d)
        for i in range(d.s_q):
            n = int(sl[b]) - d.s_q + i + 1
            for h in range(d.h_q):
                G = h // (d.h_q // d.g)
                assert rel(out[b, i, h], (C[:n] @ w_uv[G]).mean(axis=0)) < 1e-13
                assert abs(lse[b, i, h] - math.log(n)) < 1e-13      # natural log, logits 0


def test_dominant_rope_logit_selects_one_token_and_scale_is_inverse_sqrt():
    # q_nope = 0 and a rope query aligned with one token's rope key: that
    # token's logit dominates by > 700, so out = V of that token, and
    # lse = its logit = |k_rope|^2 * big / sqrt(d_nope + d_R).
    case = tiny_case((20,), 1, seed=7, table="identity")
    d = dims_of(case)
    q_nope, q_rope, pages, bt, sl, w_uk, w_uv = oracle_args(case)
    q_nope[:] = 0
    t_star = 13
    kr = pages[bt[0, t_star // d.bs], t_star % d.bs, d.r:]
    big = 4000.0 / float(kr @ kr)
    q_rope[0, 0, :] = big * kr
    out, lse = decode_literal(q_nope, q_rope, pages, bt, sl, w_uk, w_uv, d)
    c = pages[bt[0, t_star // d.bs], t_star % d.bs, : d.r]
    for h in range(d.h_q):
        G = h // (d.h_q // d.g)
        assert rel(out[0, 0, h], c @ w_uv[G]) < 1e-12
        assert abs(lse[0, 0, h] - big * float(kr @ kr) / math.sqrt(d.d_nope + d.d_R)) < 1e-9


def test_selection_w_uv_picks_latent_coordinates():
    # W_UV[G] a 0/1 selection matrix (column j picks latent coordinate sel[G][j]):
    # out must equal those coordinates of softmax-weighted C.  A transposed or
    # wrongly indexed W_UV (r x d_v with r != d_v) cannot pass.
    case = tiny_case((30, 41), 2, seed=8)
    d = dims_of(case)
    q_nope, q_rope, pages, bt, sl, w_uk, w_uv = oracle_args(case)
    rng = np.random.default_rng(0)
    sel = [rng.choice(d.r, size=d.d_v, replace=False) for _ in range(d.g)]
    w_uv = np.zeros_like(w_uv)
    for G in range(d.g):
        w_uv[G, sel[G], np.arange(d.d_v)] = 1.0
    out, _ = decode_literal(q_nope, q_rope, pages, bt, sl, w_uk, w_uv, d)
    ident = np.stack([np.eye(d.r)] * d.g)
    # same attention with V = C itself (W_UV = identity, d_v = r)
    d_lat = Dims(**{**d.__dict__, "d_v": d.r})
    o_lat, _ = decode_literal(q_nope, q_rope, pages, bt, sl, w_uk, ident, d_lat)
    for h in range(d.h_q):
        G = h // (d.h_q // d.g)
        assert rel(out[:, :, h], o_lat[:, :, h][..., sel[G]]) < 1e-13


# --- library routine: torch SDPA in float64 -------------------------------
@pytest.mark.parametrize("s_q", [1, 2])
def test_literal_matches_torch_sdpa_fp64(s_q):
    case = tiny_case((70, 97), s_q, seed=21 + s_q, h_q=8, g=2)
    d = dims_of(case)
    q_nope, q_rope, pages, bt, sl, w_uk, w_uv = oracle_args(case)
    out, _ = decode_literal(q_nope, q_rope, pages, bt, sl, w_uk, w_uv, d)
    for b in range(case.batch):
        L = int(sl[b])
        C, KR = gather_latent(pages, bt[b], L, d)
        C, KR = torch.from_numpy(C), torch.from_numpy(KR)
        k = torch.stack([torch.cat([C @ torch.from_numpy(w_uk[G]), KR], dim=1) for G in range(d.g)])
        v = torch.stack([C @ torch.from_numpy(w_uv[G]) for G in range(d.g)])
        q = torch.cat([torch.from_numpy(q_nope[b]), torch.from_numpy(q_rope[b])], dim=-1)
        q = q.permute(1, 0, 2)                                  # [h_q, s_q, E]
        pos = torch.arange(L)
        mask = pos[None, :] <= (L - s_q + torch.arange(s_q))[:, None]   # [s_q, L]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None], v[None], attn_mask=mask, enable_gqa=True)[0]  # default scale 1/sqrt(E)
        assert rel(out[b], ref.permute(1, 0, 2).numpy()) < 1e-12


# --- the pages' algebraic equivalence of the two paths ------------------------
@pytest.mark.parametrize("s_q", [1, 2])
def test_absorb_form_equals_literal_form(s_q):
    case = tiny_case((45, 129), s_q, seed=31 + s_q)
    d = dims_of(case)
    args = oracle_args(case)
    o1, l1 = decode_literal(*args, d)
    o2, l2 = decode_absorb_form(*args, d)
    assert rel(o2, o1) < 1e-12
    assert np.max(np.abs(l2 - l1)) < 1e-12


def test_absorb_equals_literal_on_tiny_workload_fp32_values():
    # The tiny workload (16 heads, 2 groups, latent 64 + rope 16, nope/v 32)
    # with fp32-drawn values: the two forms agree to fp64 rounding.
    case = make_case(16, 2, 64, 16, 32, 32, batch=2, ctx=256, s_q=2, seed=1000,
                     dtype=torch.float32)
    d = dims_of(case)
    args = oracle_args(case)
    o1, _ = decode_literal(*args, d)
    o2, _ = decode_absorb_form(*args, d)
    assert rel(o2, o1) < 1e-12


# --- MTP causal mask ---------------------------------------------------------
def test_mtp_rows_equal_single_row_decodes_at_shifted_lengths():
    # Row s_q-1 of an s_q = 2 step at length L equals an s_q = 1 decode at L;
    # row 0 equals an s_q = 1 decode at L - 1 (same cache, same query row).
    case = tiny_case((33, 64), 2, seed=41)
    d2 = dims_of(case)
    q_nope, q_rope, pages, bt, sl, w_uk, w_uv = oracle_args(case)
    out2, lse2 = decode_literal(q_nope, q_rope, pages, bt, sl, w_uk, w_uv, d2)
    d1 = dims_of(case, s_q=1)
    for row, shift in ((1, 0), (0, 1)):
        o1, l1 = decode_literal(q_nope[:, row:row + 1], q_rope[:, row:row + 1], pages, bt,
                                sl - shift, w_uk, w_uv, d1)
        assert rel(out2[:, row], o1[:, 0]) < 1e-14
        assert np.max(np.abs(lse2[:, row] - l1[:, 0])) < 1e-14


# --- paging -------------------------------------------------------------------
def test_random_page_table_equals_identity_table_after_gather():
    c_rand = tiny_case((50, 77), 2, seed=51, table="random")
    c_id = tiny_case((50, 77), 2, seed=51, table="identity")
    d = dims_of(c_rand)
    # rebuild an identity-table pool holding the same token rows as the random one
    q_nope, q_rope, pages_r, bt_r, sl, w_uk, w_uv = oracle_args(c_rand)
    pages_i = np.full_like(pages_r, np.nan)
    bt_i = c_id.block_table.numpy()
    for b in range(2):
        for j in range((int(sl[b]) + d.bs - 1) // d.bs):
            pages_i[bt_i[b, j]] = pages_r[bt_r[b, j]]
    o_r, l_r = decode_literal(q_nope, q_rope, pages_r, bt_r, sl, w_uk, w_uv, d)
    o_i, l_i = decode_literal(q_nope, q_rope, pages_i, bt_i, sl, w_uk, w_uv, d)
    assert np.array_equal(o_r, o_i) and np.array_equal(l_r, l_i)


def test_poisoned_unused_slots_never_reach_the_output():
    case = make_case(batch=2, ctx=[37, 70], s_q=2, seed=52, table="random", poison=True,
                     dtype=torch.float64, bs=8, **TINY)
    out, lse = decode_literal(*oracle_args(case), dims_of(case))
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


# --- split partials and their merge --------------------------------------------
@pytest.mark.parametrize("split_tokens", [8, 16, 64])
def test_merge_of_partials_equals_unsplit(split_tokens):
    case = tiny_case((47, 130), 2, seed=61)
    d = dims_of(case)
    args = oracle_args(case)
    ref_o, ref_l = decode_literal(*args, d)
    po, pl, off = decode_partials(*args, d, split_tokens)
    o, l = combine(po, pl, off)
    assert rel(o, ref_o) < 1e-13
    assert np.max(np.abs(l - ref_l)) < 1e-13


@pytest.mark.parametrize("s_q", [1, 2])
def test_latent_partials_up_project_to_the_literal_partials(s_q):
    # the absorb path's split partials are taken in the latent space; by
    # linearity o_lat W_UV[G] must be the literal form's split output, with the
    # same lse, and merging in the latent space before the up-projection must
    # give the unsplit result
    case = tiny_case((47, 130, 17), s_q, seed=64)
    d = dims_of(case)
    args = oracle_args(case)
    q_nope, q_rope, pages, bt, sl, w_uk, w_uv = args
    pl_lat, pl_lse, off = decode_partials_latent(q_nope, q_rope, pages, bt, sl, w_uk, d, 16)
    po, pl, off2 = decode_partials(*args, d, 16)
    assert list(off) == list(off2)
    w_uv = np.asarray(w_uv, np.float64)
    G_of_h = np.arange(d.h_q) // d.heads_per_group
    up = np.einsum("sihr,hrv->sihv", pl_lat, w_uv[G_of_h])
    assert rel(up, po) < 1e-12
    fin = np.isfinite(pl)
    assert np.array_equal(fin, np.isfinite(pl_lse))
    assert np.max(np.abs(pl_lse[fin] - pl[fin])) < 1e-12
    assert np.all(pl_lat[~fin] == 0)
    o_lat, l = combine(pl_lat, pl_lse, off)
    ref_o, ref_l = decode_literal(*args, d)
    assert rel(np.einsum("bihr,hrv->bihv", o_lat, w_uv[G_of_h]), ref_o) < 1e-12
    assert np.max(np.abs(l - ref_l)) < 1e-12


def test_partial_with_no_visible_token_is_empty():
    # L = 17, s_q = 2, splits of 8 tokens: row 0 sees tokens 0..15, so the
    # third split [16, 17) is empty for row 0 but not for row 1.
    case = tiny_case((17,), 2, seed=62)
    d = dims_of(case)
    po, pl, off = decode_partials(*oracle_args(case), d, 8)
    assert list(off) == [0, 3]
    assert np.all(pl[2, 0] == -np.inf) and np.all(po[2, 0] == 0)
    assert np.all(np.isfinite(pl[2, 1]))


def test_combine_single_split_is_identity_and_merge_is_order_free():
    po, pl, off = random_partials([1, 1], 2, 3, 5, seed=63)
    o, l = combine(po.numpy(), pl.numpy(), off.numpy())
    assert np.allclose(o, po.numpy(), rtol=0, atol=1e-15)
    assert np.allclose(l, pl.numpy(), rtol=0, atol=1e-15)
    po, pl, off = random_partials([4], 2, 3, 5, seed=64)
    perm = [2, 0, 3, 1]
    o1, l1 = combine(po.numpy(), pl.numpy(), off.numpy())
    o2, l2 = combine(po.numpy()[perm], pl.numpy()[perm], off.numpy())
    assert rel(o2, o1) < 1e-14 and np.max(np.abs(l2 - l1)) < 1e-13


def test_combine_closed_form_two_splits_and_empty_rows():
    # two splits with lse a, b: weights e^a, e^b -> out = (e^a o1 + e^b o2)/(e^a + e^b)
    po = np.array([[[[1.0, 2.0]]], [[[3.0, -4.0]]]])          # [2 splits][1][1][2]
    pl = np.array([[[0.5]], [[math.log(3.0) + 0.5]]])
    o, l = combine(po, pl, [0, 2])
    assert np.allclose(o[0, 0, 0], [(1 + 9) / 4, (2 - 12) / 4], rtol=0, atol=1e-15)
    assert abs(l[0, 0, 0] - (0.5 + math.log(4.0))) < 1e-15
    pl_empty = np.full_like(pl, -np.inf)
    o, l = combine(np.zeros_like(po), pl_empty, [0, 2])
    assert np.all(o == 0) and np.all(l == -np.inf)
    pl_half = pl.copy()
    pl_half[0] = -np.inf
    o, l = combine(po, pl_half, [0, 2])
    assert np.array_equal(o[0, 0, 0], po[1, 0, 0]) and l[0, 0, 0] == pl[1, 0, 0]


# --- bf16 rounding ---------------------------------------------------------------
def test_bf16_round_matches_torch_conversion_of_float32_values():
    # torch's float32 -> bfloat16 conversion is round-to-nearest-even; on values
    # that are exact in float32 the oracle's direct float64 rounding must agree.
    g = torch.Generator().manual_seed(71)
    x = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 20)
    specials = torch.tensor([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38,
                             1e-39, -1e-39, 1e-45, 9.2e-41, float("inf"), float("-inf")])
    x = torch.cat([x, specials])
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    got = bf16_round(x.to(torch.float64).numpy())
    assert np.array_equal(got, ref)


def test_bf16_round_ties_to_even_and_no_double_rounding():
    one = 1.0
    ulp = 2.0 ** -7
    assert bf16_round(one + ulp / 2) == one                 # tie -> even (1.0)
    assert bf16_round(one + 3 * ulp / 2) == one + 2 * ulp    # tie -> even (1 + 2ulp)
    # just above a tie in float64 but a tie after rounding to float32:
    x = one + ulp / 2 + 2.0 ** -40
    assert bf16_round(x) == one + ulp
    assert np.isnan(bf16_round(np.nan))


# --- expanded cache layout and expansion ----------------------------------------
def test_expanded_layout_views_match_offset_definitions():
    d = Dims(h_q=4, g=3, r=8, d_R=4, d_nope=4, d_v=6, s_q=1, bs=8)
    page = np.arange(expanded_page_elems(d), dtype=np.float64)
    assert expanded_page_elems(d) == d.bs * (2 * 0 + d.g * (d.d_nope + d.d_v) + d.d_R)
    for G in range(d.g):
        kv, vv = _expanded_group_views(page, d, G)
        for s in range(d.bs):
            for j in range(d.d_nope):
                assert kv[s, j] == expanded_offset_k(d, G, s, j)
            for j in range(d.d_v):
                assert vv[s, j] == expanded_offset_v(d, G, s, j)
    rv = _expanded_rope_view(page, d)
    for s in range(d.bs):
        for j in range(d.d_R):
            assert rv[s, j] == expanded_offset_rope(d, s, j)
    # every element is covered exactly once
    seen = set()
    for G in range(d.g):
        for s in range(d.bs):
            seen.update(expanded_offset_k(d, G, s, j) for j in range(d.d_nope))
            seen.update(expanded_offset_v(d, G, s, j) for j in range(d.d_v))
    for s in range(d.bs):
        seen.update(expanded_offset_rope(d, s, j) for j in range(d.d_R))
    assert seen == set(range(expanded_page_elems(d)))


def test_expansion_with_selection_weights_is_a_pure_gather():
    case = tiny_case((20, 9), 1, seed=81)
    d = dims_of(case)
    _, _, pages, _, _, w_uk, w_uv = oracle_args(case)
    rng = np.random.default_rng(3)
    sk = [rng.choice(d.r, d.d_nope, replace=False) for _ in range(d.g)]
    sv = [rng.choice(d.r, d.d_v, replace=False) for _ in range(d.g)]
    w_uk = np.zeros_like(w_uk)
    w_uv = np.zeros_like(w_uv)
    for G in range(d.g):
        w_uk[G, sk[G], np.arange(d.d_nope)] = 1.0
        w_uv[G, sv[G], np.arange(d.d_v)] = 1.0
    pages_bf = bf16_round(pages)
    E = expand_pages(pages_bf, w_uk, w_uv, d)
    for p in range(pages.shape[0]):
        for G in range(d.g):
            for s in range(d.bs):
                for j in range(d.d_nope):
                    assert E[p, expanded_offset_k(d, G, s, j)] == pages_bf[p, s, sk[G][j]]
                for j in range(d.d_v):
                    assert E[p, expanded_offset_v(d, G, s, j)] == pages_bf[p, s, sv[G][j]]
        for s in range(d.bs):
            for j in range(d.d_R):
                assert E[p, expanded_offset_rope(d, s, j)] == pages_bf[p, s, d.r + j]


def test_expanded_values_are_bf16_within_half_an_ulp_of_the_exact_product():
    # The expansion stores each K and V element once in bf16: every stored value must be a bf16
    # number (its 8 significant bits and nothing below), and it must lie within half a bf16 ulp
    # of the exact product c_t . W[G][:, j], summed here term by term.
    case = tiny_case((20, 9), 1, seed=85)
    d = dims_of(case)
    _, _, pages, _, _, w_uk, w_uv = oracle_args(case)
    E = expand_pages(pages, w_uk, w_uv, d)
    for p in range(pages.shape[0]):
        for G in range(d.g):
            for s in range(d.bs):
                for w, off, n in ((w_uk, expanded_offset_k, d.d_nope), (w_uv, expanded_offset_v, d.d_v)):
                    for j in range(n):
                        got = E[p, off(d, G, s, j)]
                        exact = math.fsum(pages[p, s, k] * w[G, k, j] for k in range(d.r))
                        m, e = math.frexp(got)                      # got = m * 2**e, |m| in [0.5, 1)
                        assert m * 256 == int(m * 256)               # 8 significant bits
                        half_ulp = math.ldexp(1.0, math.frexp(exact)[1] - 9) if exact else 0.0
                        assert abs(got - exact) <= half_ulp


@pytest.mark.parametrize("s_q", [1, 2])
def test_gqa_over_expanded_cache_equals_literal_up_to_bf16_storage(s_q):
    case = tiny_case((40, 66), s_q, seed=91 + s_q)
    d = dims_of(case)
    q_nope, q_rope, pages, bt, sl, w_uk, w_uv = oracle_args(case)
    E = expand_pages(pages, w_uk, w_uv, d)
    o_e, l_e = decode_gqa_expanded(q_nope, q_rope, E, bt, sl, d)
    o_l, l_l = decode_literal(q_nope, q_rope, pages, bt, sl, w_uk, w_uv, d)
    assert rel(o_e, o_l) < 2e-2          # bf16 storage of K and V only
    # without the storage rounding the two are the same function
    E_exact = np.zeros_like(E)
    for p in range(pages.shape[0]):
        for G in range(d.g):
            kv, vv = _expanded_group_views(E_exact[p], d, G)
            kv[...] = pages[p, :, : d.r] @ w_uk[G]
            vv[...] = pages[p, :, : d.r] @ w_uv[G]
        _expanded_rope_view(E_exact[p], d)[...] = pages[p, :, d.r:]
    o_x, l_x = decode_gqa_expanded(q_nope, q_rope, E_exact, bt, sl, d)
    assert rel(o_x, o_l) < 1e-12 and np.max(np.abs(l_x - l_l)) < 1e-12
