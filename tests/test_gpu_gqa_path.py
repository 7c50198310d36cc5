"""GPU parity of the GQA path: one-shot expansion, GQA decode, split-KV merge.

Every expected value comes from the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import decode_attention_gqla_amd as G
from decode_attention_gqla_amd.inputs import config_case, make_case, random_partials
from oracle.gqla_ref import (bf16_round, combine, decode_gqa_expanded, decode_literal,
                             expand_pages, expanded_offset_k, expanded_offset_rope,
                             expanded_offset_v)
from tests.gpu_util import GpuCase, assert_close, assert_lse_close, f64, log
from tests.oracle_util import dims_of, oracle_args

pytestmark = pytest.mark.gpu


def _expected_ulp_bound(ref):
    """One bf16 ulp at each reference value (spacing of bf16 numbers there)."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(int))


# --- expansion ----------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "llama3_8b", "dsv3"])
def test_expand_selection_weights_is_bit_exact(name):
    log(f"expand/selection {name}")
    case = config_case(name, 1, batch=2, ctx=200 if name == "tiny" else 300)
    d = dims_of(case)
    rng = np.random.default_rng(5)
    w_uk = torch.zeros_like(case.w_uk)
    w_uv = torch.zeros_like(case.w_uv)
    for g in range(d.g):
        w_uk[g, torch.from_numpy(rng.choice(d.r, d.d_nope, replace=False)), torch.arange(d.d_nope)] = 1
        w_uv[g, torch.from_numpy(rng.choice(d.r, d.d_v, replace=False)), torch.arange(d.d_v)] = 1
    case.w_uk, case.w_uv = w_uk, w_uv
    gc = GpuCase(case)
    E = gc.expand()
    torch.cuda.synchronize()
    ref = expand_pages(f64(case.pages), f64(w_uk), f64(w_uv), d)
    got = f64(E)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("name", ["tiny", "dsv3"])
def test_expand_random_weights_within_one_bf16_ulp(name):
    log(f"expand/random {name}")
    case = config_case(name, 1, batch=3, ctx=(64, 130, 257))
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    torch.cuda.synchronize()
    pages = list(range(case.pages.shape[0] - 1))          # skip the spare page
    ref = expand_pages(f64(case.pages), f64(case.w_uk), f64(case.w_uv), d, page_ids=pages)
    # sum_k |c_k w_k| per output element (the scale of fp32 accumulation error)
    mag = expand_pages(np.abs(f64(case.pages)), np.abs(f64(case.w_uk)), np.abs(f64(case.w_uv)), d,
                       page_ids=pages)
    got = f64(E)[pages]
    diff = np.abs(got - ref)
    # bf16(fp32 sum) vs bf16(exact sum): one bf16 ulp plus the fp32 accumulation
    # error bound gamma_r * sum|c w| (gamma_r ~ r * 2^-24)
    bound = _expected_ulp_bound(ref) + d.r * 2.0 ** -24 * mag * 1.01
    assert np.all(diff <= bound), float(np.max(diff / bound))
    assert np.mean(diff == 0) > 0.95
    # the rope key is copied bit-exactly (checked inside the comparison above, here explicitly)
    assert np.array_equal(got[:, -d.bs * d.d_R:], ref[:, -d.bs * d.d_R:])


def test_expand_full_pool_whole_quads_and_pieces_agree():
    # 1025 pages: on a 256-CU GPU, 256 workgroups expand whole page quads and the
    # leftover quad's passes are spread over 32 more; the same pages expanded by a
    # call with a short page list (pass pieces only) must be identical bit for bit,
    # and sampled pages (the last quad's included) meet the oracle's bound
    log("expand/full pool (1025 pages)")
    case = config_case("dsv3", 1, batch=16, ctx=4096)
    d = dims_of(case)
    gc = GpuCase(case)
    n = case.pages.shape[0]
    assert n == 1025
    E = gc.expand()
    ids = [0, 1, 511, 1021, 1022, 1023, 1024]
    E_sub = torch.full_like(E, 3.0)
    G.gqla_expand_cache(gc.d, gc.pages, gc.w_uk, gc.w_uv, E_sub,
                        page_ids=torch.tensor(ids, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for p in ids:
        assert torch.equal(E_sub[p], E[p]), p
    sample = [0, 511, 1023]                                  # 1024 is the spare (zero) page
    ref = expand_pages(f64(case.pages), f64(case.w_uk), f64(case.w_uv), d, page_ids=sample)
    mag = expand_pages(np.abs(f64(case.pages)), np.abs(f64(case.w_uk)), np.abs(f64(case.w_uv)), d,
                       page_ids=sample)
    got = f64(E)[sample]
    bound = _expected_ulp_bound(ref) + d.r * 2.0 ** -24 * mag * 1.01
    assert np.all(np.abs(got - ref) <= bound)
    assert torch.all(E[1024] == 0)


def test_expand_page_list_touches_only_listed_pages():
    log("expand/page_ids")
    case = config_case("tiny", 1, batch=2, ctx=256)
    gc = GpuCase(case)
    n = case.pages.shape[0]
    E = torch.full((n, G.expanded_page_elems(gc.d)), 7.0, dtype=torch.bfloat16, device="cuda")
    ids = torch.tensor([5, 1, 3], dtype=torch.int32, device="cuda")
    G.gqla_expand_cache(gc.d, gc.pages, gc.w_uk, gc.w_uv, E, page_ids=ids)
    full = gc.expand()
    torch.cuda.synchronize()
    for p in range(n):
        if p in (5, 1, 3):
            assert torch.equal(E[p], full[p])
        else:
            assert torch.all(E[p] == 7.0)


# --- GQA decode ---------------------------------------------------------------------
CASES = [
    ("tiny", 1, dict()), ("tiny", 2, dict()),
    ("llama3_8b", 1, dict(batch=4)), ("llama3_8b", 2, dict(batch=4)),
    ("dsv3", 2, dict(batch=3, ctx=(4096, 1000, 77))),
    ("dsv3", 1, dict(batch=2, ctx=(129, 2))),
    ("dsv3_g4", 1, dict(batch=3, ctx=(4096, 1000, 77))),
    ("dsv3_g4", 2, dict(batch=2, ctx=(1500, 33))),
    # the smallest contexts the precondition s_q <= L allows (MTP row 0 of
    # L = 2 sees one token), one page plus a token, and a batch of one
    ("dsv3", 2, dict(batch=3, ctx=(2, 3, 65))),
    ("dsv3", 1, dict(batch=1, ctx=1)),
]


@pytest.mark.parametrize("name,s_q,kw", CASES)
def test_gqa_decode_matches_oracle(name, s_q, kw):
    log(f"gqa/unsplit {name} s_q={s_q} {kw}")
    case = config_case(name, s_q, poison=True, table="random", **kw)
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    out, lse = gc.gqa(E)
    torch.cuda.synchronize()
    ref_o, ref_l = decode_literal(*oracle_args(case), d)
    assert_close(f64(out), ref_o, "out vs literal oracle")
    assert_lse_close(f64(lse), ref_l, "lse vs literal oracle")
    # against the exact decode of the expanded cache the GPU itself produced:
    # only P and the output are rounded to bf16 here
    ex_o, ex_l = decode_gqa_expanded(f64(case.q_nope), f64(case.q_rope), f64(E),
                                     case.block_table.numpy(), case.seqlens.numpy(), d)
    assert_close(f64(out), ex_o, "out vs oracle over GPU-expanded cache", max_rel=8e-3, rel_l2=4e-3)


def test_gqa_bench_launch_configuration_full_context():
    # the bench's GQA call: DeepSeek-V3 shape, batch 64, context 4096, s_q = 2,
    # unsplit (512 workgroups); sampled sequences against the oracle
    log("gqa/full size dsv3 B=64 ctx=4096 (sampled sequences)")
    case = config_case("dsv3", 2)
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    out, lse = gc.gqa(E)
    torch.cuda.synchronize()
    seqs = [0, 31, 63]
    ref_o, ref_l = decode_literal(*oracle_args(case), d, seqs=seqs)
    assert_close(f64(out)[seqs], ref_o, "out vs literal oracle")
    assert_lse_close(f64(lse)[seqs], ref_l, "lse vs literal oracle")


@pytest.mark.parametrize("split_tokens", [64, 128, 1024])
def test_gqa_split_kv_matches_oracle(split_tokens):
    log(f"gqa/split {split_tokens}")
    case = config_case("dsv3", 2, batch=3, ctx=(1500, 64, 2049), poison=True, table="random")
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    out, lse = gc.gqa(E, split=gc.split(split_tokens))
    torch.cuda.synchronize()
    ref_o, ref_l = decode_literal(*oracle_args(case), d)
    assert_close(f64(out), ref_o, "split out vs oracle")
    assert_lse_close(f64(lse), ref_l, "split lse vs oracle")


def test_gqa_ragged_long_context_sampled():
    log("gqa/ragged dsv3_ragged (sampled sequences)")
    case = config_case("dsv3_ragged", 2, poison=True)
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    out, lse = gc.gqa(E, split=gc.split(1024))
    torch.cuda.synchronize()
    seqs = [int(np.argmax(case.seqlens.numpy())), int(np.argmin(case.seqlens.numpy())), 7]
    ref_o, ref_l = decode_literal(*oracle_args(case), d, seqs=seqs)
    assert_close(f64(out)[seqs], ref_o, "ragged out (sampled)")
    assert_lse_close(f64(lse)[seqs], ref_l, "ragged lse (sampled)")


def test_gqa_is_deterministic_and_writes_only_its_outputs():
    log("gqa/determinism+canary")
    case = config_case("dsv3", 2, batch=4, ctx=(300, 4096, 65, 1024), poison=True)
    gc = GpuCase(case)
    E = gc.expand()
    d = gc.d
    B = 4
    n_out = B * d.s_q * d.num_heads * d.d_v
    buf = torch.full((n_out + 4096,), 3.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * d.s_q * d.num_heads + 1024,), 5.0, dtype=torch.float32, device="cuda")
    out = buf[:n_out].view(B, d.s_q, d.num_heads, d.d_v)
    lse = lbuf[: B * d.s_q * d.num_heads].view(B, d.s_q, d.num_heads)
    G.gqla_decode_gqa(d, gc.q_nope, gc.q_rope, E, gc.block_table, gc.seqlens, out=out, lse=lse)
    first = out.clone()
    G.gqla_decode_gqa(d, gc.q_nope, gc.q_rope, E, gc.block_table, gc.seqlens, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert torch.all(buf[n_out:] == 3.0) and torch.all(lbuf[B * d.s_q * d.num_heads:] == 5.0)


# --- split-KV merge ---------------------------------------------------------------------
@pytest.mark.parametrize("empty_frac", [0.0, 0.3])
def test_combine_matches_oracle_on_the_same_partials(empty_frac):
    log(f"combine empty_frac={empty_frac}")
    d = G.Dims.make(128, 8, 512, 64, 128, 128, 2)
    counts = [1, 3, 7, 32, 2]
    po, pl, offs = random_partials(counts, 2, 128, 128, seed=11, empty_frac=empty_frac)
    out = torch.empty(len(counts), 2, 128, 128, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(len(counts), 2, 128, dtype=torch.float32, device="cuda")
    G.gqla_splitkv_combine(d, offs.cuda(), po.cuda(), pl.cuda(), out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = combine(po.double().numpy(), pl.double().numpy(), offs.numpy())
    got_o, got_l = f64(out), f64(lse)
    full = np.isfinite(ref_l)
    # the merge is done in fp32 and rounded once to bf16
    assert np.all(np.abs(got_o - bf16_round(ref_o)) <= _expected_ulp_bound(ref_o) + 1e-6)
    assert np.max(np.abs(got_l[full] - ref_l[full])) < 1e-4
    assert np.array_equal(got_l[~full], ref_l[~full])            # all-empty rows: -inf
    assert np.all(got_o[~full] == 0)


# --- incremental append ---------------------------------------------------------------
@pytest.mark.parametrize("n_new", [1, 2])
@pytest.mark.parametrize("name", ["tiny", "dsv3"])
def test_append_then_both_caches_equal_a_full_build(name, n_new):
    """Appending each sequence's last n_new tokens to a cache that lacks them gives, bit for
    bit, the latent pages of the full case and the full expansion of those pages, and writes
    nothing else (the new tokens of the 65-token sequence straddle a page boundary when
    n_new = 2)."""
    log(f"append {name} n_new={n_new}")
    ctx = (65, 300, 64, 128) if name == "tiny" else (65, 4096, 1000, 129)
    case = config_case(name, 1, batch=4, ctx=ctx, poison=True, table="random")
    d = dims_of_gpu(case)
    dev = "cuda"
    full = case.pages.to(dev)
    bt, sl = case.block_table.to(dev), case.seqlens.to(dev)
    w_uk, w_uv = case.w_uk.to(dev), case.w_uv.to(dev)
    E_full = G.expand_cache(d, full, w_uk, w_uv)
    # the state before the step: new-token slots hold something else
    start = full.clone()
    rows = []
    for b in range(case.batch):
        L = int(case.seqlens[b])
        r_b = []
        for j in range(n_new):
            t = L - n_new + j
            pg, slot = int(case.block_table[b, t // case.bs]), t % case.bs
            r_b.append(full[pg, slot].clone())
            start[pg, slot] = 3.0
        rows.append(torch.stack(r_b))
    new_rows = torch.stack(rows).contiguous()
    E = G.expand_cache(d, start, w_uk, w_uv)
    G.gqla_append_tokens(d, new_rows, start, bt, sl, w_uk, w_uv, expanded_pages=E)
    torch.cuda.synchronize()
    assert torch.equal(start.view(torch.int16), full.view(torch.int16))
    assert torch.equal(E.view(torch.int16), E_full.view(torch.int16))
    # latent-only append (the absorb path's cache)
    start2 = full.clone()
    for b in range(case.batch):
        L = int(case.seqlens[b])
        for j in range(n_new):
            t = L - n_new + j
            start2[int(case.block_table[b, t // case.bs]), t % case.bs] = -5.0
    G.gqla_append_tokens(d, new_rows, start2, bt, sl)
    torch.cuda.synchronize()
    assert torch.equal(start2.view(torch.int16), full.view(torch.int16))


def _selection_weights(case, seed):
    """W_UK / W_UV with one 1.0 per column: the expansion becomes a pure gather."""
    d = dims_of(case)
    rng = np.random.default_rng(seed)
    w_uk = torch.zeros_like(case.w_uk)
    w_uv = torch.zeros_like(case.w_uv)
    for g in range(d.g):
        w_uk[g, torch.from_numpy(rng.choice(d.r, d.d_nope, replace=False)), torch.arange(d.d_nope)] = 1
        w_uv[g, torch.from_numpy(rng.choice(d.r, d.d_v, replace=False)), torch.arange(d.d_v)] = 1
    return w_uk, w_uv


@pytest.mark.parametrize("weights", ["selection", "random"])
def test_appended_slots_match_the_oracle_expansion(weights):
    """The K, V and rope slots gqla_append_tokens writes for each sequence's last two tokens,
    against oracle.expand_pages of the updated latent pages: bit-exact with selection weights
    (a pure gather), within one bf16 ulp plus the fp32 accumulation bound with random weights.
    Every other element of the expanded pool keeps its sentinel."""
    n_new = 2
    log(f"append vs oracle expansion, {weights} weights")
    case = config_case("dsv3", 1, batch=4, ctx=(65, 4096, 1000, 129), poison=True, table="random")
    if weights == "selection":
        case.w_uk, case.w_uv = _selection_weights(case, seed=9)
    d = dims_of(case)
    dg = G.Dims.of(case)
    dev = "cuda"
    full = case.pages.to(dev)
    bt, sl = case.block_table.to(dev), case.seqlens.to(dev)
    w_uk, w_uv = case.w_uk.to(dev), case.w_uv.to(dev)
    slots, rows = [], []
    for b in range(case.batch):
        L = int(case.seqlens[b])
        for j in range(n_new):
            t = L - n_new + j
            slots.append((int(case.block_table[b, t // case.bs]), t % case.bs))
            rows.append(full[slots[-1][0], slots[-1][1]].clone())
    new_rows = torch.stack(rows).view(case.batch, n_new, -1).contiguous()
    E = torch.full((full.shape[0], G.expanded_page_elems(dg)), 7.0, dtype=torch.bfloat16, device=dev)
    G.gqla_append_tokens(dg, new_rows, full.clone(), bt, sl, w_uk, w_uv, expanded_pages=E)
    torch.cuda.synchronize()
    touched = sorted({pg for pg, _ in slots})
    ref = expand_pages(f64(case.pages), f64(case.w_uk), f64(case.w_uv), d, page_ids=touched)
    mag = expand_pages(np.abs(f64(case.pages)), np.abs(f64(case.w_uk)), np.abs(f64(case.w_uv)), d,
                       page_ids=touched)
    got = f64(E)
    written = np.zeros(got.shape, dtype=bool)
    for pg, slot in slots:
        idx = []
        for Gi in range(d.g):
            idx += [expanded_offset_k(d, Gi, slot, j) for j in range(d.d_nope)]
            idx += [expanded_offset_v(d, Gi, slot, j) for j in range(d.d_v)]
        idx_rope = [expanded_offset_rope(d, slot, j) for j in range(d.d_R)]
        r_pg = ref[touched.index(pg)]
        g_pg = got[pg]
        if weights == "selection":
            assert np.array_equal(g_pg[idx], r_pg[idx]), (pg, slot)
        else:
            bound = _expected_ulp_bound(r_pg[idx]) + d.r * 2.0 ** -24 * mag[touched.index(pg)][idx] * 1.01
            assert np.all(np.abs(g_pg[idx] - r_pg[idx]) <= bound), (pg, slot)
        assert np.array_equal(g_pg[idx_rope], r_pg[idx_rope]), (pg, slot)
        written[pg, idx + idx_rope] = True
    assert np.all(got[~written] == 7.0)


def test_append_skips_positions_outside_the_sequence_or_the_block_table():
    """Tokens whose position falls before 0 (cache_seqlens < n_new) or past the block table
    write nothing, in both modes; the one valid token rewrites its own row, so no slot of
    either cache changes."""
    n_new = 2
    log("append with invalid positions")
    case = config_case("dsv3", 1, batch=2, ctx=(1, 128), poison=True, table="random")
    dg = G.Dims.of(case)
    dev = "cuda"
    assert case.max_blocks == 2
    full = case.pages.to(dev)
    bt = case.block_table.to(dev)
    w_uk, w_uv = case.w_uk.to(dev), case.w_uv.to(dev)
    E_full = G.expand_cache(dg, full, w_uk, w_uv)
    # sequence 0: L = 1, so new token 0 sits at t = -1 (invalid) and token 1 at t = 0;
    # sequence 1: L = 192 with a two-page table, so both new tokens sit on page index 2
    sl = torch.tensor([1, 192], dtype=torch.int32, device=dev)
    new_rows = torch.full((2, n_new, dg.d_latent + dg.d_rope), 9.0, dtype=torch.bfloat16, device=dev)
    new_rows[0, 1] = full[int(case.block_table[0, 0]), 0]
    lat = full.clone()
    E = E_full.clone()
    G.gqla_append_tokens(dg, new_rows, lat, bt, sl, w_uk, w_uv, expanded_pages=E)
    lat2 = full.clone()
    G.gqla_append_tokens(dg, new_rows, lat2, bt, sl)
    torch.cuda.synchronize()
    assert torch.equal(lat.view(torch.int16), full.view(torch.int16))
    assert torch.equal(E.view(torch.int16), E_full.view(torch.int16))
    assert torch.equal(lat2.view(torch.int16), full.view(torch.int16))


def dims_of_gpu(case):
    return G.Dims.of(case)
