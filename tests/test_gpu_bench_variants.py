"""GPU parity at the launches the bench measures for its variants.

Each case runs both decode paths at the batch, context mix and split sizes that
bench.py times (the (g, s_q) = (4, 1) regrouping, the LLaMA-3-8B shape at s_q 1
and 2, the ragged long-context mix), and compares sampled sequences with the
fp64 literal oracle: every output row and lse of those sequences."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from decode_attention_gqla_amd.inputs import config_case
from oracle.gqla_ref import decode_literal
from tests.gpu_util import GpuCase, assert_close, assert_lse_close, f64, log
from tests.oracle_util import dims_of, oracle_args

pytestmark = pytest.mark.gpu

# (config, s_q, absorb split tokens, GQA split tokens (0: unsplit), seed) as bench.py's variants
# run them; their GQA calls have at most two workgroups per CU and run two wave groups over alternate
# tiles
CASES = [
    ("dsv3_g4", 1, 2048, 0, None),
    ("llama3_8b", 1, 512, 0, 1001 + 10),
    ("llama3_8b", 2, 512, 0, 1001 + 10),
    ("dsv3_ragged", 1, 1280, 2560, 1004 + 10),
    ("dsv3_ragged", 2, 1280, 2560, 1004 + 10),
]


@pytest.mark.parametrize("name,s_q,a_split,g_split,seed", CASES)
def test_bench_variant_launch_matches_oracle(name, s_q, a_split, g_split, seed):
    log(f"bench variant {name} s_q={s_q}: absorb split {a_split}, GQA split {g_split}")
    case = config_case(name, s_q, seed=seed) if seed is not None else config_case(name, s_q)
    d = dims_of(case)
    gc = GpuCase(case)
    out_a, lse_a = gc.absorb(split=gc.split(a_split))
    E = gc.expand()
    out_g, lse_g = gc.gqa(E, split=gc.split(g_split) if g_split else None)
    torch.cuda.synchronize()
    L = case.seqlens.numpy()
    seqs = sorted({0, int(np.argmax(L)), int(np.argmin(L)), len(L) - 1})
    ref_o, ref_l = decode_literal(*oracle_args(case), d, seqs=seqs)
    assert_close(f64(out_a)[seqs], ref_o, "absorb out (sampled)")
    assert_lse_close(f64(lse_a)[seqs], ref_l, "absorb lse (sampled)")
    assert_close(f64(out_g)[seqs], ref_o, "gqa out (sampled)")
    assert_lse_close(f64(lse_g)[seqs], ref_l, "gqa lse (sampled)")
