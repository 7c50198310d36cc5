"""GPU parity of every GQA decode launch form against the fp64 oracle.

The GQA launcher picks the tile ring and the number of wave groups (waves
taking alternate tiles, their softmax states merged in LDS at the end) from
the shape and the grid: one-wave row sets in an eight-buffer ring and two-wave
row sets in a six-buffer ring when the grid has at most one workgroup per CU,
a four-buffer ring with two groups beyond that, one group for four-wave row
sets.  Each case below runs one of those forms on contexts whose tile counts
are odd and even, down to the smallest legal context (s_q tokens: one group
then sees no tile at all), and compares sampled sequences, every output row
and lse, with the literal oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from decode_attention_gqla_amd.inputs import config_case
from oracle.gqla_ref import decode_literal
from tests.gpu_util import GpuCase, assert_close, assert_lse_close, f64, log
from tests.oracle_util import dims_of, oracle_args

pytestmark = pytest.mark.gpu

# context lengths: 1, 2, 3, 4, 10 and 32 tiles of 32 tokens, and the smallest legal one
CTX = (33, 64, 65, 97, 300, 1000)


# (config, s_q, batch): a small batch gives at most one workgroup per CU, a large one more
# than one (the GPU has 256 CUs; the grid is 8 * ceil(batch / 8) * g workgroups)
CASES = [
    ("tiny", 1, 3), ("tiny", 2, 200),
    ("llama3_8b", 1, 3), ("llama3_8b", 2, 40),
    ("dsv3", 1, 3), ("dsv3", 2, 3), ("dsv3", 1, 40), ("dsv3", 2, 40),
    ("dsv3_g4", 1, 3), ("dsv3_g4", 1, 72), ("dsv3_g4", 2, 3),
]


@pytest.mark.parametrize("name,s_q,batch", CASES)
def test_gqa_launch_forms_match_oracle(name, s_q, batch):
    ctx = tuple(s_q if i % 7 == 6 else CTX[i % 7 % 6] for i in range(batch))
    log(f"gqa launch form {name} s_q={s_q} batch={batch}")
    case = config_case(name, s_q, batch=batch, ctx=ctx, table="random", poison=True)
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    out, lse = gc.gqa(E)
    torch.cuda.synchronize()
    seqs = sorted(set(range(min(batch, 7))) | {batch - 1})
    ref_o, ref_l = decode_literal(*oracle_args(case), d, seqs=seqs)
    assert_close(f64(out)[seqs], ref_o, f"{name} out")
    assert_lse_close(f64(lse)[seqs], ref_l, f"{name} lse")


@pytest.mark.parametrize("split_tokens", [64, 192])
def test_gqa_split_units_with_wave_groups_match_oracle(split_tokens):
    # split units of up to 2 or 6 tiles, the last unit of a sequence shorter (down to one tile, so
    # that one group sees none), more workgroups than CUs, merged by the combine
    log(f"gqa wave groups, split {split_tokens}")
    batch = 24
    ctx = tuple(CTX[i % 6] for i in range(batch))
    case = config_case("dsv3", 2, batch=batch, ctx=ctx, table="random", poison=True)
    d = dims_of(case)
    gc = GpuCase(case)
    E = gc.expand()
    out, lse = gc.gqa(E, split=gc.split(split_tokens))
    torch.cuda.synchronize()
    seqs = list(range(6)) + [batch - 1]
    ref_o, ref_l = decode_literal(*oracle_args(case), d, seqs=seqs)
    assert_close(f64(out)[seqs], ref_o, "split out")
    assert_lse_close(f64(lse)[seqs], ref_l, "split lse")
