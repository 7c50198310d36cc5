"""GPU parity at the size limits of the launches.

Past the block-table entries kept in LDS: the main absorb decode kernel copies
a unit's block-table entries into LDS when they are at most 1024 (65536
tokens at 64-token pages) and reads them with scalar loads otherwise.  An
unsplit call over a sequence of 70000 tokens (1094 pages) takes the second
form; a 100-token sequence in the same batch takes the first-tile-only edge.

Past one round of workgroups: a batch of 600 short sequences gives thousands
of workgroups on both paths.

Both paths are compared with the fp64 oracle in its absorb form (pinned to
the literal definition on the CPU)."""
from __future__ import annotations

import pytest
import torch

from decode_attention_gqla_amd.inputs import config_case
from oracle.gqla_ref import decode_absorb_form
from tests.gpu_util import GpuCase, assert_close, assert_lse_close, f64, log
from tests.oracle_util import dims_of, oracle_args

pytestmark = pytest.mark.gpu


def test_both_paths_past_the_block_table_kept_in_lds():
    log("long context: dsv3 s_q=1, contexts (70000, 100), unsplit")
    case = config_case("dsv3", 1, batch=2, ctx=(70000, 100), poison=True, table="random")
    assert case.block_table.shape[1] > 1024
    d = dims_of(case)
    gc = GpuCase(case)
    out_a, lse_a = gc.absorb()
    E = gc.expand()
    out_g, lse_g = gc.gqa(E)
    torch.cuda.synchronize()
    ref_o, ref_l = decode_absorb_form(*oracle_args(case), d)
    assert_close(f64(out_a), ref_o, "absorb out")
    assert_lse_close(f64(lse_a), ref_l, "absorb lse")
    assert_close(f64(out_g), ref_o, "gqa out")
    assert_lse_close(f64(lse_g), ref_l, "gqa lse")


def test_both_paths_on_a_batch_of_many_workgroup_rounds():
    # 600 short sequences: the GQA launch has 4800 workgroups (two resident per CU at a time), the
    # absorb decode 2400 (256 query rows per sequence in blocks of 64, one resident per CU)
    log("many rounds: dsv3 s_q=2, batch 600, contexts 2..200")
    batch = 600
    ctx = tuple(2 + (37 * i) % 199 for i in range(batch))
    case = config_case("dsv3", 2, batch=batch, ctx=ctx, poison=True, table="random")
    d = dims_of(case)
    gc = GpuCase(case)
    out_a, lse_a = gc.absorb()
    E = gc.expand()
    out_g, lse_g = gc.gqa(E)
    torch.cuda.synchronize()
    seqs = [0, 1, 2, 255, 256, 311, 598, 599]
    ref_o, ref_l = decode_absorb_form(*oracle_args(case), d, seqs=seqs)
    assert_close(f64(out_a)[seqs], ref_o, "absorb out (sampled)")
    assert_lse_close(f64(lse_a)[seqs], ref_l, "absorb lse (sampled)")
    assert_close(f64(out_g)[seqs], ref_o, "gqa out (sampled)")
    assert_lse_close(f64(lse_g)[seqs], ref_l, "gqa lse (sampled)")
