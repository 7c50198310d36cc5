"""The closed forms behind the bench's algorithmic bytes and FLOPs, pinned to
the numbers the GQLA pages print (tests/golden/pages_numbers.json, each entry
citing where it is printed)."""
import json
import os

import pytest

from decode_attention_gqla_amd import roofline as rf

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
DSV3 = dict(h_q=128, g=8, r=512, d_R=64, d_h=128)
L = 8192


def near(key, got):
    e = GOLD[key]
    assert abs(got - e["value"]) <= e.get("tol", 0), (key, got, e)


def test_cache_sizes():
    near("latent_elems_per_token", rf.latent_elems_per_token(512, 64))
    near("latent_bytes_per_token", 2 * rf.latent_elems_per_token(512, 64))
    near("expanded_bytes_per_token_g8", 2 * rf.expanded_elems_per_token(8, 128, 64))
    near("expanded_bytes_per_token_g4", 2 * rf.expanded_elems_per_token(4, 128, 64))
    near("llama_gqa_elems_per_token", 2 * 8 * 128)
    near("latent_fraction_of_gqa", rf.latent_elems_per_token(512, 64) / (2 * 8 * 128))


def test_intensities():
    near("intensity_absorb_sq1", rf.intensity_absorb(128, 1, 512, 64))
    near("intensity_absorb_sq2", rf.intensity_absorb(128, 2, 512, 64))
    near("intensity_gqa_g8_sq2", rf.intensity_gqa(128, 2, 8, 128, 64))
    near("intensity_gqa_g4_sq1", rf.intensity_gqa(128, 1, 4, 128, 64))
    near("ridge_h100", rf.H100["tflops"] / rf.H100["tbps"])
    near("ridge_h20", rf.H20["tflops"] / rf.H20["tbps"])


def _step(path, s_q, hw, g=8):
    if path == "absorb":
        by = L * 2 * rf.latent_elems_per_token(512, 64)
        fl = L * rf.flops_per_token_absorb(128, s_q, 512, 64)
    else:
        by = L * 2 * rf.expanded_elems_per_token(g, 128, 64)
        fl = L * rf.flops_per_token_gqa(128, s_q, 128, 64)
    return rf.model_step_us(by, fl, hw["tbps"], hw["tflops"])


def test_pages_step_time_predictions():
    t1 = _step("absorb", 1, rf.H100)
    t2 = _step("absorb", 2, rf.H100)
    near("h100_absorb_sq1_us", t1)
    near("h100_absorb_sq2_us", t2)
    near("h100_mtp_speedup", (2 / t2) / (1 / t1))
    near("h100_absorb_tok_s", 1e6 / t1)
    t_mla = _step("absorb", 1, rf.H20)
    near("h20_mla_us", t_mla)
    near("h20_mla_tok_s", 1e6 / t_mla)
    t_gqa = _step("gqa", 2, rf.H20)
    near("h20_gqa_g8_sq2_us", t_gqa)
    near("h20_gqa_tok_s", 2e6 / t_gqa)
    near("h20_gqa_tok_s", 1e6 / _step("gqa", 1, rf.H20, g=4))
    near("h20_speedup_gqa_over_mla", (2e6 / t_gqa) / (1e6 / t_mla))


def test_per_launch_work_matches_hand_count_for_the_dsv3_batch():
    w = rf.work_absorb([4096] * 64, 128, 8, 512, 64, 128, 128, 1)
    assert w.cache_bytes == 64 * 4096 * 1152
    assert w.bytes == 64 * 4096 * 1152 + 2 * 64 * 128 * 192 + 2 * 8 * 512 * 256 + 2 * 64 * 128 * 128
    assert w.flops == 64 * 4096 * 278528 + 2 * 64 * 128 * 512 * 256
    g = rf.work_gqa([4096] * 64, 128, 8, 64, 128, 128, 2)
    assert g.cache_bytes == 64 * 4096 * 4224
    # two MTP rows see 4095 and 4096 tokens
    assert g.flops == 64 * (4095 + 4096) * 128 * 2 * 320
    assert g.bound() == "hbm" and w.bound() == "hbm"


def test_sparse_work_with_every_position_listed_relates_to_the_dense_count():
    # every position listed once: the same (row, token) pairs as the dense decode, and the
    # rope row read once per group instead of once per token
    lens = [100, 37]
    idx = [[list(range(L)) + [-1, L + 3] for _ in range(8)] for L in lens]
    sp = rf.work_gqa_sparse(idx, lens, 128, 8, 64, 128, 128, 2)
    de = rf.work_gqa(lens, 128, 8, 64, 128, 128, 2)
    assert sp.flops == de.flops
    assert sp.cache_bytes == de.cache_bytes + sum(lens) * 7 * 64 * 2
    # queries and output as for the dense call, plus 4 bytes per listed index
    assert sp.bytes - sp.cache_bytes == de.bytes - de.cache_bytes + sum(8 * (L + 2) * 4 for L in lens)


def test_sparse_work_hand_count_for_the_bench_configuration():
    # batch 64, 8 groups, 2048 distinct entries per group, all older than the new tokens
    lens = [4096] * 64
    idx = [[list(range(0, 4096, 2))] * 8] * 64
    w = rf.work_gqa_sparse(idx, lens, 128, 8, 64, 128, 128, 2)
    assert w.cache_bytes == 64 * 8 * 2048 * 640
    assert w.bytes == 64 * 8 * 2048 * 640 + 64 * 2 * 128 * 192 * 2 + 64 * 2 * 128 * 128 * 2 \
        + 64 * 8 * 2048 * 4
    assert w.flops == 64 * 8 * 2048 * 2 * 16 * 2 * 320
