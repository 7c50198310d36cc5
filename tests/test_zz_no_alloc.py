"""The allocation-free absorb entry point: through the C ABI, two calls in a row
(the second on a smaller input) against the workspace entry point on the same
inputs, and against the oracle within the floating-point bar."""
from __future__ import annotations

import pytest
import torch

import decode_attention_gqla_amd as G
from decode_attention_gqla_amd.inputs import config_case
from oracle.gqla_ref import decode_literal
from tests.gpu_util import GpuCase, assert_close, assert_lse_close, f64, log
from tests.oracle_util import dims_of, oracle_args

pytestmark = pytest.mark.gpu


def _run_pair(case, split):
    gc = GpuCase(case)
    offs, total, st = gc.split(split)
    out_ref, lse_ref = gc.absorb(split=(offs, total, st))
    torch.cuda.synchronize()
    out = torch.full_like(out_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    before = torch.cuda.memory_allocated()
    G.gqla_decode_mqa_absorb_noalloc(gc.d, gc.q_nope, gc.q_rope, gc.pages, gc.block_table, gc.seqlens,
                                     gc.w_uk, gc.w_uv, out=out, lse=lse, split_offsets=offs,
                                     split_tokens=st, total_splits=total)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return out, lse, out_ref, lse_ref


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    for batch, ctx, split in ((4, (4096, 3000, 1000, 65), 1024), (2, (700, 130), 256)):
        log(f"absorb/noalloc batch {batch} ctx {ctx} split {split}")
        case = config_case("dsv3", 1, batch=batch, ctx=ctx, poison=True, table="random")
        out, lse, out_ref, lse_ref = _run_pair(case, split)
        assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
        ref_o, ref_l = decode_literal(*oracle_args(case), dims_of(case))
        assert_close(f64(out), ref_o, "noalloc out vs oracle")
        assert_lse_close(f64(lse), ref_l, "noalloc lse vs oracle")


def test_noalloc_rejects_a_call_beyond_its_scratch():
    # 64 sequences of 4096 tokens in 64-token splits need about 145 MB of workspace
    log("absorb/noalloc over the scratch limit")
    d = G.Dims.make(128, 8, 512, 64, 128, 128, 1)
    need = G.gqla_mqa_absorb_workspace_bytes(d, 64, 64 * 64)
    assert need > G.NOALLOC_SCRATCH_BYTES
    case = config_case("dsv3", 1, batch=2, ctx=(128, 64))
    gc = GpuCase(case)
    out = torch.empty(2, 1, 128, 128, dtype=torch.bfloat16, device="cuda")
    offs = torch.zeros(3, dtype=torch.int32, device="cuda")
    with pytest.raises(G.GqlaError) as e:
        # a split plan claiming 5000 splits: the workspace it implies is over the limit
        G.gqla_decode_mqa_absorb_noalloc(gc.d, gc.q_nope, gc.q_rope, gc.pages, gc.block_table, gc.seqlens,
                                         gc.w_uk, gc.w_uv, out=out, split_offsets=offs, split_tokens=64,
                                         total_splits=5000)
    assert e.value.status == -6
