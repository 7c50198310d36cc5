"""The path selector (roofline advisor) of the C ABI, on the CPU.

Pinned to the step times and throughputs the GQLA pages print for H100 and H20
(tests/golden/pages_numbers.json, each entry citing where it is printed), and
to the package's closed-form per-call work (decode_attention_gqla_amd.roofline,
itself pinned in test_roofline_closed_forms.py)."""
import json
import os

import numpy as np
import pytest

import decode_attention_gqla_amd as G
from decode_attention_gqla_amd import roofline as rf

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
DSV3 = G.Dims.make(128, 8, 512, 64, 128, 128, 1)


def near(key, got):
    e = GOLD[key]
    assert abs(got - e["value"]) <= e.get("tol", 0), (key, got, e)


def hw_of(peaks, frac_a=1.0, frac_g=1.0, cache_only=1):
    return G.Hw(peaks["tbps"] * 1000.0, peaks["tflops"], frac_a, frac_g, cache_only)


def test_pages_h100_prefers_absorb():
    # one sequence, one layer, context 8192 (the reading that reproduces the pages' step times)
    st, ea, eg = G.gqla_select_path(DSV3, [8192], 1, 2, hw_of(rf.H100))
    assert st == G.PATH_ABSORB
    near("h100_absorb_sq1_us", ea.t_expected_us)
    near("h100_absorb_tok_s", ea.tokens_per_s)
    _, ea2, _ = G.gqla_select_path(DSV3, [8192], 2, 2, hw_of(rf.H100))
    near("h100_absorb_sq2_us", ea2.t_expected_us)
    near("h100_mtp_speedup", ea2.tokens_per_s / ea.tokens_per_s)


def test_pages_h20_prefers_gqa():
    st, ea, eg = G.gqla_select_path(DSV3, [8192], 1, 2, hw_of(rf.H20))
    assert st == G.PATH_GQA
    near("h20_mla_us", ea.t_expected_us)
    near("h20_mla_tok_s", ea.tokens_per_s)
    near("h20_gqa_g8_sq2_us", eg.t_expected_us)
    near("h20_gqa_tok_s", eg.tokens_per_s)
    near("h20_speedup_gqa_over_mla", eg.tokens_per_s / ea.tokens_per_s)
    # the other ridge-optimal GQA configuration, (g, s_q) = (4, 1)
    g4 = G.Dims.make(128, 4, 512, 64, 128, 128, 1)
    st4, _, eg4 = G.gqla_select_path(g4, [8192], 1, 1, hw_of(rf.H20))
    assert st4 == G.PATH_GQA
    near("h20_gqa_tok_s", eg4.tokens_per_s)


@pytest.mark.parametrize("lens,shape", [
    ([4096] * 64, (128, 8)),                                 # the DSV3 bench batch
    ([1000, 4096, 33, 32768, 2], (128, 8)),                  # ragged
    ([2048] * 32, (32, 8)),                                  # LLaMA-3-8B-shaped
])
@pytest.mark.parametrize("s_q", [(1, 2), (2, 1), (1, 1)])
def test_counts_equal_the_closed_form_work(lens, shape, s_q):
    h_q, g = shape
    d = G.Dims.make(h_q, g, 512, 64, 128, 128, 1)
    st, ea, eg = G.gqla_select_path(d, lens, s_q[0], s_q[1], G.Hw(8000.0, 2500.0, 1.0, 1.0, 0))
    wa = rf.work_absorb(lens, h_q, g, 512, 64, 128, 128, s_q[0])
    wg = rf.work_gqa(lens, h_q, g, 64, 128, 128, s_q[1])
    assert ea.bytes == wa.bytes and ea.flops == wa.flops
    assert eg.bytes == wg.bytes and eg.flops == wg.flops
    assert ea.t_roofline_us == pytest.approx(wa.roofline_us(), rel=1e-12)
    assert eg.t_roofline_us == pytest.approx(wg.roofline_us(), rel=1e-12)
    # the choice is the higher tokens/s, ties to absorb
    ta = len(lens) * s_q[0] / wa.roofline_us()
    tg = len(lens) * s_q[1] / wg.roofline_us()
    assert st == (G.PATH_GQA if tg > ta else G.PATH_ABSORB)


def test_fractions_scale_the_expected_time_and_can_flip_the_choice():
    lens = [4096] * 64
    st1, ea1, eg1 = G.gqla_select_path(DSV3, lens, 1, 2, G.Hw(8000.0, 2500.0, 1.0, 1.0, 0))
    assert st1 == G.PATH_ABSORB                    # at the roofline the absorb path wins on MI355X
    st2, ea2, eg2 = G.gqla_select_path(DSV3, lens, 1, 2, G.Hw(8000.0, 2500.0, 0.25, 0.75, 0))
    assert ea2.t_expected_us == pytest.approx(ea1.t_roofline_us / 0.25)
    assert eg2.t_expected_us == pytest.approx(eg1.t_roofline_us / 0.75)
    assert st2 == G.PATH_GQA
    # equal tokens/s -> absorb (no expanded cache needed)
    fa = ea1.t_roofline_us / (eg1.t_roofline_us / 2)
    st3, ea3, eg3 = G.gqla_select_path(DSV3, lens, 1, 2, G.Hw(8000.0, 2500.0, fa, 1.0, 0))
    assert ea3.tokens_per_s == pytest.approx(eg3.tokens_per_s, rel=1e-12)
    if eg3.tokens_per_s <= ea3.tokens_per_s:
        assert st3 == G.PATH_ABSORB


@pytest.mark.parametrize("bad", [
    dict(lens=[], s=(1, 2)), dict(lens=[4096], s=(0, 2)), dict(lens=[4096], s=(1, 3)),
    dict(lens=[1], s=(1, 2)), dict(lens=[4096], s=(1, 2), hw=(0.0, 2500.0, 1.0, 1.0)),
    dict(lens=[4096], s=(1, 2), hw=(8000.0, -1.0, 1.0, 1.0)),
    dict(lens=[4096], s=(1, 2), hw=(8000.0, 2500.0, 0.0, 1.0)),
    dict(lens=[4096], s=(1, 2), hw=(8000.0, 2500.0, 1.0, 1.5)),
    dict(lens=[4096], s=(1, 2), hw=(8000.0, 2500.0, float("nan"), 1.0)),
])
def test_invalid_arguments(bad):
    hw = G.Hw(*(bad.get("hw", (8000.0, 2500.0, 1.0, 1.0))), 0)
    if not bad["lens"]:
        with pytest.raises(G.GqlaError):
            _call_empty(hw)
        return
    with pytest.raises(G.GqlaError):
        G.gqla_select_path(DSV3, bad["lens"], bad["s"][0], bad["s"][1], hw)


def _call_empty(hw):
    import ctypes
    lens = (ctypes.c_int32 * 1)(4096)
    st = G.lib().gqla_select_path(ctypes.byref(DSV3), 0, lens, 1, 2, ctypes.byref(hw), None, None)
    if st < 0:
        raise G.GqlaError(st, "gqla_select_path")
