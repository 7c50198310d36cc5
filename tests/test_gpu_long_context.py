"""GPU parity beyond the longest split the kernels keep in LDS.

The main absorb decode kernel copies a unit's block-table entries into LDS
when they are at most 1024 (65536 tokens at 64-token pages) and reads them
with scalar loads otherwise.  An unsplit call over a sequence of 70000 tokens
(1094 pages) takes the second form; a 100-token sequence in the same batch
takes the first-tile-only edge.  Both paths are compared with the fp64 oracle
in its absorb form (pinned to the literal definition on the CPU)."""
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
