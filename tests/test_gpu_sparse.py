"""GPU parity of the sparse GQA decode (per-group token selections).

Every expected value comes from the fp64 oracle on the same seeded inputs and
the same index lists; caches carry NaN in every unused slot, so an entry that
is ignored or masked must really contribute nothing."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import decode_attention_gqla_amd as G
from decode_attention_gqla_amd.inputs import config_case, sparse_indices
from oracle.gqla_ref import decode_gqa_sparse, expand_pages
from tests.gpu_util import GpuCase, assert_close, f64, log
from tests.oracle_util import dims_of

pytestmark = pytest.mark.gpu


def run_sparse(gc, E, idx_host, split=0):
    d, B = gc.d, gc.q_nope.shape[0]
    idx = idx_host.to("cuda")
    out = torch.empty(B, d.s_q, d.num_heads, d.d_v, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, d.s_q, d.num_heads, dtype=torch.float32, device="cuda")
    ws = G.sparse_workspace(d, B, idx.shape[2], split)
    G.gqla_decode_gqa_sparse(d, gc.q_nope, gc.q_rope, E, gc.block_table, gc.seqlens, idx, out,
                             lse=lse, workspace=ws, split_entries=split)
    return out, lse


def check(out, lse, ref_o, ref_l, what, max_rel=1e-2, rel_l2=5e-3):
    """Rows the oracle leaves empty must be exactly 0 / -inf; the rest meet the bar."""
    got_o, got_l = f64(out), f64(lse)
    empty = np.isneginf(ref_l)
    log(f"  {what}: {int(empty.sum())} empty rows of {empty.size}")
    assert np.all(got_o[empty] == 0.0) and np.all(np.isneginf(got_l[empty]))
    full = ~empty
    assert_close(got_o[full], ref_o[full], what, max_rel=max_rel, rel_l2=rel_l2)
    err = float(np.max(np.abs(got_l[full] - ref_l[full]))) if full.any() else 0.0
    log(f"  {what}: max|lse err|={err:.3e}")
    assert np.all(np.isfinite(got_l[full])) and err <= 2e-2


CASES = [
    ("tiny", 1, dict(batch=2, ctx=256), 40, 0.0, 0.0),
    ("tiny", 2, dict(batch=2, ctx=(256, 70)), 64, 0.2, 0.1),
    ("llama3_8b", 1, dict(batch=4, ctx=(2048, 600, 33, 1000)), 257, 0.05, 0.0),
    ("dsv3", 2, dict(batch=3, ctx=(4096, 1000, 77)), 2048, 0.05, 0.05),
    ("dsv3", 1, dict(batch=2, ctx=(129, 2)), 31, 0.0, 0.0),
    ("dsv3_g4", 2, dict(batch=2, ctx=(1500, 33)), 100, 0.1, 0.0),
]


@pytest.mark.parametrize("name,s_q,kw,topk,invalid,dup", CASES)
def test_sparse_matches_oracle(name, s_q, kw, topk, invalid, dup):
    log(f"sparse {name} s_q={s_q} {kw} topk={topk} invalid={invalid} dup={dup}")
    case = config_case(name, s_q, poison=True, table="random", **kw)
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    idx = sparse_indices(gc.seqlens_host, d.g, topk, seed=301 + topk, invalid_frac=invalid,
                         dup_frac=dup)
    out, lse = run_sparse(gc, E, idx)
    torch.cuda.synchronize()
    bt, sl = case.block_table.numpy(), case.seqlens.numpy()
    # exact decode of the expanded cache the GPU produced: only P and the output are rounded
    ex_o, ex_l = decode_gqa_sparse(f64(case.q_nope), f64(case.q_rope), f64(E), bt, sl,
                                   idx.numpy(), d)
    check(out, lse, ex_o, ex_l, "out vs oracle over GPU-expanded cache", max_rel=8e-3, rel_l2=4e-3)
    # the whole chain against the oracle's own expansion
    Eo = expand_pages(f64(case.pages), f64(case.w_uk), f64(case.w_uv), d)
    ref_o, ref_l = decode_gqa_sparse(f64(case.q_nope), f64(case.q_rope), Eo, bt, sl, idx.numpy(), d)
    check(out, lse, ref_o, ref_l, "out vs oracle over oracle-expanded cache")


@pytest.mark.parametrize("name,s_q", [("tiny", 2), ("dsv3", 2), ("dsv3", 1)])
def test_every_position_in_order_equals_the_dense_decode_bitwise(name, s_q):
    # the same tokens land in the same tiles in the same order, and padding
    # entries are masked exactly as tokens past the end are (40 sequences:
    # more workgroups than CUs, as at the bench's batch)
    log(f"sparse=dense {name} s_q={s_q}")
    B = 40
    case = config_case(name, s_q, poison=True, table="random", batch=B,
                       ctx=tuple((300, 64, 97)[i % 3] for i in range(B)))
    gc = GpuCase(case)
    E = gc.expand()
    L = gc.seqlens_host
    topk = max(L)
    idx = torch.full((B, gc.d.num_groups, topk), -1, dtype=torch.int32)
    for b in range(B):
        idx[b, :, : L[b]] = torch.arange(L[b], dtype=torch.int32)
    out, lse = run_sparse(gc, E, idx)
    dense_o, dense_l = gc.gqa(E)
    torch.cuda.synchronize()
    assert torch.equal(out, dense_o)
    assert torch.equal(lse, dense_l)


def test_rows_that_see_no_entry_are_empty():
    log("sparse/empty rows")
    case = config_case("dsv3", 2, poison=True, table="random", batch=2, ctx=(500, 64))
    gc = GpuCase(case)
    E = gc.expand()
    d = dims_of(case)
    # only the second new token's position: query row 0 cannot see it;
    # group 1 lists nothing valid at all
    idx = torch.full((2, d.g, 3), -1, dtype=torch.int32)
    for b, L in enumerate(gc.seqlens_host):
        idx[b, :, 0] = L - 1
        idx[b, 1, 0] = L + 5
    out, lse = run_sparse(gc, E, idx)
    torch.cuda.synchronize()
    ex_o, ex_l = decode_gqa_sparse(f64(case.q_nope), f64(case.q_rope), f64(E),
                                   case.block_table.numpy(), case.seqlens.numpy(), idx.numpy(), d)
    assert np.all(np.isneginf(ex_l[:, 0]))
    check(out, lse, ex_o, ex_l, "empty-row case", max_rel=8e-3, rel_l2=4e-3)


def test_full_size_bench_configuration_sampled():
    # DeepSeek-V3 shape, batch 64, context 4096, s_q = 2, 2048 entries per group
    log("sparse/full size dsv3 B=64 ctx=4096 topk=2048 (sampled sequences)")
    case = config_case("dsv3", 2)
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    idx = sparse_indices(gc.seqlens_host, d.g, 2048, seed=2048)
    out, lse = run_sparse(gc, E, idx)
    torch.cuda.synchronize()
    seqs = [0, 37, 63]
    ex_o, ex_l = decode_gqa_sparse(f64(case.q_nope), f64(case.q_rope), f64(E),
                                   case.block_table.numpy(), case.seqlens.numpy(), idx.numpy(), d,
                                   seqs=seqs)
    check(out[seqs], lse[seqs], ex_o, ex_l, "full-size sampled", max_rel=8e-3, rel_l2=4e-3)


def test_sparse_is_deterministic_and_writes_only_its_outputs():
    log("sparse/determinism+canary")
    case = config_case("dsv3", 2, batch=4, ctx=(300, 4096, 65, 1024), poison=True)
    gc = GpuCase(case)
    E = gc.expand()
    d, B = gc.d, 4
    idx = sparse_indices(gc.seqlens_host, d.num_groups, 333, seed=5, invalid_frac=0.1).to("cuda")
    n_out = B * d.s_q * d.num_heads * d.d_v
    n_lse = B * d.s_q * d.num_heads
    n_ws = G.gqla_sparse_workspace_bytes(d, B, 333)
    assert n_ws == B * d.num_groups * 352 * 4
    buf = torch.full((n_out + 4096,), 3.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((n_lse + 1024,), 5.0, dtype=torch.float32, device="cuda")
    wbuf = torch.full((n_ws + 4096,), 9, dtype=torch.uint8, device="cuda")
    out = buf[:n_out].view(B, d.s_q, d.num_heads, d.d_v)
    lse = lbuf[:n_lse].view(B, d.s_q, d.num_heads)
    G.gqla_decode_gqa_sparse(d, gc.q_nope, gc.q_rope, E, gc.block_table, gc.seqlens, idx, out,
                             lse=lse, workspace=wbuf[:n_ws])
    first = out.clone()
    G.gqla_decode_gqa_sparse(d, gc.q_nope, gc.q_rope, E, gc.block_table, gc.seqlens, idx, out,
                             lse=lse, workspace=wbuf[:n_ws])
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert torch.all(buf[n_out:] == 3.0) and torch.all(lbuf[n_lse:] == 5.0)
    assert torch.all(wbuf[n_ws:] == 9)


SPLIT_CASES = [
    ("tiny", 2, dict(batch=2, ctx=(256, 70)), 100, 32, 0.1),     # 4 ranges, the last ragged
    ("dsv3", 2, dict(batch=3, ctx=(4096, 1000, 77)), 2048, 512, 0.05),   # ranges of padding only
    ("dsv3_g4", 1, dict(batch=2, ctx=(1500, 33)), 300, 64, 0.0),
]


@pytest.mark.parametrize("name,s_q,kw,topk,split,invalid", SPLIT_CASES)
def test_split_sparse_matches_oracle_and_the_unsplit_call(name, s_q, kw, topk, split, invalid):
    log(f"sparse/split {name} s_q={s_q} {kw} topk={topk} split={split}")
    case = config_case(name, s_q, poison=True, table="random", **kw)
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    idx = sparse_indices(gc.seqlens_host, d.g, topk, seed=401 + topk, invalid_frac=invalid)
    out, lse = run_sparse(gc, E, idx, split=split)
    ref_u, _ = run_sparse(gc, E, idx)
    torch.cuda.synchronize()
    ex_o, ex_l = decode_gqa_sparse(f64(case.q_nope), f64(case.q_rope), f64(E),
                                   case.block_table.numpy(), case.seqlens.numpy(), idx.numpy(), d)
    check(out, lse, ex_o, ex_l, "split out vs oracle over GPU-expanded cache", max_rel=8e-3,
          rel_l2=4e-3)
    assert_close(f64(out), f64(ref_u), "split vs unsplit", max_rel=8e-3, rel_l2=4e-3)


def test_split_sparse_writes_only_its_workspace():
    log("sparse/split canary")
    case = config_case("dsv3", 2, batch=2, ctx=(700, 2000), poison=True)
    gc = GpuCase(case)
    E = gc.expand()
    d, B = gc.d, 2
    idx = sparse_indices(gc.seqlens_host, d.num_groups, 600, seed=6).to("cuda")
    n_ws = G.gqla_sparse_workspace_bytes(d, B, 600, 128)
    off = G.gqla_sparse_workspace_offsets(d, B, 600, 128)
    assert off[4] == n_ws
    wbuf = torch.full((n_ws + 4096,), 9, dtype=torch.uint8, device="cuda")
    out = torch.empty(B, d.s_q, d.num_heads, d.d_v, dtype=torch.bfloat16, device="cuda")
    G.gqla_decode_gqa_sparse(d, gc.q_nope, gc.q_rope, E, gc.block_table, gc.seqlens, idx, out,
                             workspace=wbuf[:n_ws], split_entries=128)
    torch.cuda.synchronize()
    assert torch.all(wbuf[n_ws:] == 9)
    plan = wbuf[off[1]: off[1] + 4 * (B + 1)].view(torch.int32).cpu().tolist()
    assert plan == [0, 5, 10]                                   # 608 padded entries -> 5 ranges


@pytest.mark.parametrize("name,s_q,topk,split,seed", [
    ("dsv3_ragged", 2, 2048, 512, 2048 + 1),     # the bench's small-batch ragged call, in ranges of 512
    ("dsv3_ragged", 2, 2048, 1024, 2048 + 1),    # and in ranges of 1024
    ("dsv3_ragged", 2, 2048, 0, 2048 + 1),       # and unsplit
    ("dsv3", 2, 512, 0, 512),                    # the bench's batch-64 call at 512 entries per group
])
def test_sparse_bench_launches_sampled(name, s_q, topk, split, seed):
    log(f"sparse/bench launch {name} topk={topk} split={split} (sampled sequences)")
    case = config_case(name, s_q)
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    idx = sparse_indices(gc.seqlens_host, d.g, topk, seed=seed)
    out, lse = run_sparse(gc, E, idx, split=split)
    torch.cuda.synchronize()
    L = case.seqlens.numpy()
    seqs = sorted({0, int(np.argmax(L)), int(np.argmin(L)), len(L) - 1})
    ex_o, ex_l = decode_gqa_sparse(f64(case.q_nope), f64(case.q_rope), f64(E),
                                   case.block_table.numpy(), case.seqlens.numpy(), idx.numpy(), d,
                                   seqs=seqs)
    check(out[seqs], lse[seqs], ex_o, ex_l, "bench launch sampled", max_rel=8e-3, rel_l2=4e-3)
