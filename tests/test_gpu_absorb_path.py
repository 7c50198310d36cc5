"""GPU parity of the MQA-absorb path, the cross-path identity, and bit-exact
page/slot indexing of both paths.  Expected values come from the fp64 oracle
on the same seeded inputs (or, for the indexing test, from the inputs
themselves)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import decode_attention_gqla_amd as G
from decode_attention_gqla_amd.inputs import config_case
from oracle.gqla_ref import decode_literal, error_stats
from tests.gpu_util import GpuCase, assert_close, assert_lse_close, f64, log
from tests.oracle_util import dims_of, oracle_args

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", 1, dict()), ("tiny", 2, dict()),
    ("llama3_8b", 1, dict(batch=4)), ("llama3_8b", 2, dict(batch=3, ctx=(2048, 300, 64))),
    ("dsv3", 1, dict(batch=3, ctx=(4096, 1000, 77))),
    ("dsv3", 2, dict(batch=2, ctx=(1500, 33))),
    ("dsv3_g4", 1, dict(batch=3, ctx=(4096, 1000, 77))),
    ("dsv3_g4", 2, dict(batch=2, ctx=(1500, 33))),
    # the smallest contexts the precondition s_q <= L allows (MTP row 0 of
    # L = 2 sees one token), one page plus a token, and a batch of one
    ("dsv3", 2, dict(batch=3, ctx=(2, 3, 65))),
    ("dsv3", 1, dict(batch=1, ctx=1)),
]


@pytest.mark.parametrize("name,s_q,kw", CASES)
def test_absorb_decode_matches_oracle(name, s_q, kw):
    log(f"absorb/unsplit {name} s_q={s_q} {kw}")
    case = config_case(name, s_q, poison=True, table="random", **kw)
    gc = GpuCase(case)
    out, lse = gc.absorb()
    torch.cuda.synchronize()
    ref_o, ref_l = decode_literal(*oracle_args(case), dims_of(case))
    assert_close(f64(out), ref_o, "out vs literal oracle")
    assert_lse_close(f64(lse), ref_l, "lse vs literal oracle")


@pytest.mark.parametrize("split_tokens", [64, 1024, 2048])
def test_absorb_split_kv_matches_oracle(split_tokens):
    log(f"absorb/split {split_tokens}")
    case = config_case("dsv3", 1, batch=3, ctx=(1500, 64, 2049), poison=True, table="random")
    gc = GpuCase(case)
    out, lse = gc.absorb(split=gc.split(split_tokens))
    torch.cuda.synchronize()
    ref_o, ref_l = decode_literal(*oracle_args(case), dims_of(case))
    assert_close(f64(out), ref_o, "split out vs oracle")
    assert_lse_close(f64(lse), ref_l, "split lse vs oracle")


def test_absorb_bench_launch_configuration_full_context():
    """The configuration the bench times: DeepSeek-V3 shape at context 4096 in 2048-token
    splits, here over 8 sequences (every output row compared with the oracle)."""
    log("absorb/dsv3 batch 8 ctx 4096 split 2048")
    case = config_case("dsv3", 1, batch=8, poison=True, table="random")
    gc = GpuCase(case)
    out, lse = gc.absorb(split=gc.split(2048))
    torch.cuda.synchronize()
    ref_o, ref_l = decode_literal(*oracle_args(case), dims_of(case))
    assert_close(f64(out), ref_o, "out vs literal oracle")
    assert_lse_close(f64(lse), ref_l, "lse vs literal oracle")


def test_absorb_ragged_long_context_sampled():
    log("absorb/ragged dsv3_ragged (sampled sequences)")
    case = config_case("dsv3_ragged", 1, poison=True)
    gc = GpuCase(case)
    out, lse = gc.absorb(split=gc.split(1024))
    torch.cuda.synchronize()
    seqs = [int(np.argmax(case.seqlens.numpy())), int(np.argmin(case.seqlens.numpy())), 5]
    ref_o, ref_l = decode_literal(*oracle_args(case), dims_of(case), seqs=seqs)
    assert_close(f64(out)[seqs], ref_o, "ragged out (sampled)")
    assert_lse_close(f64(lse)[seqs], ref_l, "ragged lse (sampled)")


@pytest.mark.parametrize("s_q", [1, 2])
def test_cross_path_identity_on_gpu(s_q):
    # The pages' claim: the two paths compute the same function.  On the GPU
    # they differ only by bf16 rounding at different points.
    log(f"cross-path dsv3 s_q={s_q}")
    case = config_case("dsv3", s_q, batch=4, ctx=(4096, 2500, 129, 64), poison=True, table="random")
    gc = GpuCase(case)
    o_abs, l_abs = gc.absorb()
    E = gc.expand()
    o_gqa, l_gqa = gc.gqa(E)
    torch.cuda.synchronize()
    assert_close(f64(o_abs), f64(o_gqa), "absorb vs gqa (GPU)")
    assert_lse_close(f64(l_abs), f64(l_gqa), "absorb vs gqa lse (GPU)")


def _one_hot_case(name, s_q, seed):
    """Inputs whose softmax puts all weight on one chosen token per row group,
    with a selection W_UV: both paths must return that token's latent
    coordinates exactly (every step is exact: q_abs = 0, p in {0, 1}, the
    selected coordinate is a bf16 value copied through fp32)."""
    case = config_case(name, s_q, table="random", poison=True, seed=seed)
    d = dims_of(case)
    rng = np.random.default_rng(seed)
    case.q_nope.zero_()
    w_uv = torch.zeros_like(case.w_uv)
    sel = [rng.choice(d.r, d.d_v, replace=False) for _ in range(d.g)]
    for gi in range(d.g):
        w_uv[gi, torch.from_numpy(sel[gi]), torch.arange(d.d_v)] = 1
    case.w_uv = w_uv
    # rope keys: small random; one chosen token per sequence gets a large key
    # aligned with every query's rope part
    B = case.batch
    t_star = []
    pages = case.pages.float()
    for b in range(B):
        L = int(case.seqlens[b])
        t = int(rng.integers(0, L - s_q + 1))          # visible to every MTP row
        t_star.append(t)
    key = torch.ones(d.d_R)
    for b in range(B):
        L = int(case.seqlens[b])
        nblk = (L + d.bs - 1) // d.bs
        for j in range(nblk):
            pg = int(case.block_table[b, j])
            pages[pg, :, d.r:] = torch.where(torch.isnan(pages[pg, :, d.r:]), pages[pg, :, d.r:],
                                             0.01 * pages[pg, :, d.r:])
        pg = int(case.block_table[b, t_star[b] // d.bs])
        pages[pg, t_star[b] % d.bs, d.r:] = key
    case.pages = pages.to(torch.bfloat16)
    case.q_rope = (torch.ones_like(case.q_rope.float()) * 40.0).to(torch.bfloat16)
    return case, d, sel, t_star


@pytest.mark.parametrize("path", ["absorb", "gqa"])
def test_one_hot_attention_reads_exactly_the_chosen_page_slot(path):
    log(f"one-hot indexing {path}")
    case, d, sel, t_star = _one_hot_case("dsv3_ragged", 2 if path == "gqa" else 1, seed=77)
    gc = GpuCase(case)
    if path == "absorb":
        out, _ = gc.absorb(split=gc.split(1024))
    else:
        out, _ = gc.gqa(gc.expand(), split=gc.split(1024))
    torch.cuda.synchronize()
    got = f64(out)
    pages = f64(case.pages)
    for b in range(case.batch):
        pg = int(case.block_table[b, t_star[b] // d.bs])
        c_row = pages[pg, t_star[b] % d.bs, : d.r]
        for h in range(d.h_q):
            Gi = h // (d.h_q // d.g)
            exp = c_row[sel[Gi]]
            for i in range(d.s_q):
                assert np.array_equal(got[b, i, h], exp), (b, i, h, t_star[b])


def test_absorb_is_deterministic_and_writes_only_its_outputs():
    log("absorb/determinism+canary")
    case = config_case("dsv3", 1, batch=4, ctx=(300, 4096, 65, 1024), poison=True)
    gc = GpuCase(case)
    d = gc.d
    B = 4
    n_out = B * d.s_q * d.num_heads * d.d_v
    buf = torch.full((n_out + 4096,), 3.0, dtype=torch.bfloat16, device="cuda")
    nl = B * d.s_q * d.num_heads
    lbuf = torch.full((nl + 1024,), 5.0, dtype=torch.float32, device="cuda")
    out = buf[:n_out].view(B, d.s_q, d.num_heads, d.d_v)
    lse = lbuf[:nl].view(B, d.s_q, d.num_heads)
    ws = G.absorb_workspace(d, B)
    G.gqla_decode_mqa_absorb(d, gc.q_nope, gc.q_rope, gc.pages, gc.block_table, gc.seqlens,
                             gc.w_uk, gc.w_uv, out=out, lse=lse, workspace=ws)
    first = out.clone()
    G.gqla_decode_mqa_absorb(d, gc.q_nope, gc.q_rope, gc.pages, gc.block_table, gc.seqlens,
                             gc.w_uk, gc.w_uv, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert torch.all(buf[n_out:] == 3.0) and torch.all(lbuf[nl:] == 5.0)


def test_absorb_partials_match_oracle_partials():
    # the per-split latent outputs o_lat and their lse, as the decode kernel
    # leaves them in the workspace before the merge and the up-projection
    from oracle.gqla_ref import decode_partials_latent
    log("absorb/latent partials")
    case = config_case("dsv3", 2, batch=2, ctx=(700, 130), poison=True, table="random")
    gc = GpuCase(case)
    d = gc.d
    offs, total, st = gc.split(256)
    ws = G.absorb_workspace(d, 2, total_splits=total)
    out = torch.empty(2, d.s_q, d.num_heads, d.d_v, dtype=torch.bfloat16, device="cuda")
    G.gqla_decode_mqa_absorb(d, gc.q_nope, gc.q_rope, gc.pages, gc.block_table, gc.seqlens,
                             gc.w_uk, gc.w_uv, out=out, split_offsets=offs, split_tokens=st,
                             total_splits=total, workspace=ws)
    torch.cuda.synchronize()
    o0, o1, o2, o3 = G.gqla_mqa_absorb_workspace_offsets(d, 2, total)
    rows = d.s_q * d.num_heads
    lat = ws[o2:o2 + total * rows * d.d_latent * 2].view(torch.bfloat16)
    lat = lat.view(total, d.s_q, d.num_heads, d.d_latent)
    lse = ws[o3:o3 + total * rows * 4].view(torch.float32).view(total, d.s_q, d.num_heads)
    q_nope, q_rope, pages, bt, sl, w_uk, _ = oracle_args(case)
    ref_lat, ref_lse, ref_off = decode_partials_latent(q_nope, q_rope, pages, bt, sl, w_uk,
                                                       dims_of(case), 256)
    assert list(ref_off) == offs.cpu().tolist()
    got_lat, got_lse = f64(lat), f64(lse)
    empty = ~np.isfinite(ref_lse)            # rows that see no token of a split (MTP row 0)
    assert np.array_equal(empty, ~np.isfinite(got_lse))
    assert np.all(got_lat[empty] == 0)
    assert_close(got_lat[~empty], ref_lat[~empty], "latent partials")
    assert_lse_close(got_lse[~empty], ref_lse[~empty], "partial lse")


@pytest.mark.parametrize("name,s_q,split", [("dsv3", 2, 256), ("dsv3", 1, 1024), ("llama3_8b", 1, 64),
                                            ("tiny", 2, None)])
def test_merge_entry_point_on_oracle_latent_partials(name, s_q, split):
    """gqla_mqa_absorb_merge on latent partials computed by the oracle (rounded to bf16, the
    entry point's input type): against the oracle's log-sum-exp combine of the same rounded
    partials followed by the up-projection by W_UV[G], and against the literal decode."""
    from oracle.gqla_ref import combine, decode_partials_latent
    log(f"absorb/merge entry {name} s_q={s_q} split={split}")
    kw = dict(batch=3, ctx=(700, 130, 65)) if name != "tiny" else dict()
    case = config_case(name, s_q, poison=True, table="random", **kw)
    d = dims_of(case)
    gd = G.Dims.of(case)
    args = oracle_args(case)
    q_nope, q_rope, pages, bt, sl, w_uk, w_uv = args
    lens = [int(x) for x in case.seqlens]
    B = len(lens)
    split_tokens = split if split else max(lens) + 64 - max(lens) % 64
    ref_lat, ref_lse, ref_off = decode_partials_latent(q_nope, q_rope, pages, bt, sl, w_uk, d, split_tokens)
    lat_bf = torch.from_numpy(ref_lat).to(torch.bfloat16)
    lse_f = torch.from_numpy(ref_lse).to(torch.float32)
    total = int(ref_off[-1])
    out = torch.empty(B, s_q, case.h_q, case.d_v, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, s_q, case.h_q, dtype=torch.float32, device="cuda")
    offs = torch.tensor(ref_off, dtype=torch.int32, device="cuda") if split else None
    G.gqla_mqa_absorb_merge(gd, lat_bf.cuda(), lse_f.cuda(), case.w_uv.cuda(), out, lse=lse,
                            split_offsets=offs, total_splits=total if split else 0)
    torch.cuda.synchronize()
    # oracle: combine the rounded partials, then o W_UV[G] per group
    m_lat, m_lse = combine(lat_bf.double().numpy(), lse_f.double().numpy(), ref_off)
    hpg = case.h_q // case.g
    w = np.repeat(w_uv, hpg, axis=0)                     # [h_q][d_latent][d_v], head h -> group h // hpg
    ref_out = np.einsum("bihl,hlv->bihv", m_lat, w)
    assert_close(f64(out), ref_out, "merge vs oracle combine + up-projection")
    fin = np.isfinite(m_lse)
    assert np.array_equal(fin, np.isfinite(f64(lse)))
    assert_lse_close(f64(lse)[fin], m_lse[fin], "merge lse vs oracle combine")
    lit_o, _ = decode_literal(*args, d)
    assert_close(f64(out), lit_o, "merge vs literal decode")


def test_merge_entry_point_remerges_the_decode_workspace():
    """The partials a decode call leaves in its workspace, merged again by the entry point,
    give the decode call's own output bit for bit (the same merge kernel)."""
    log("absorb/merge entry over the decode workspace")
    case = config_case("dsv3", 1, batch=3, ctx=(1500, 64, 2049), poison=True, table="random")
    gc = GpuCase(case)
    d = gc.d
    offs, total, st = gc.split(1024)
    ws = G.absorb_workspace(d, 3, total_splits=total)
    out = torch.empty(3, 1, d.num_heads, d.d_v, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(3, 1, d.num_heads, dtype=torch.float32, device="cuda")
    G.gqla_decode_mqa_absorb(d, gc.q_nope, gc.q_rope, gc.pages, gc.block_table, gc.seqlens, gc.w_uk, gc.w_uv,
                             out=out, lse=lse, split_offsets=offs, split_tokens=st, total_splits=total,
                             workspace=ws)
    o0, o1, o2, o3 = G.gqla_mqa_absorb_workspace_offsets(d, 3, total)
    rows = d.s_q * d.num_heads
    lat = ws[o2:o2 + total * rows * d.d_latent * 2].view(torch.bfloat16).view(total, 1, d.num_heads, d.d_latent)
    plse = ws[o3:o3 + total * rows * 4].view(torch.float32).view(total, 1, d.num_heads)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    G.gqla_mqa_absorb_merge(d, lat.clone(), plse.clone(), gc.w_uv, out2, lse=lse2, split_offsets=offs,
                            total_splits=total)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
