"""Helpers for the GPU parity tests: move seeded cases to the GPU, run the
oracle on sampled sequences, and apply the acceptance bar."""
from __future__ import annotations

import sys

import numpy as np
import torch

import decode_attention_gqla_amd as G
from oracle.gqla_ref import error_stats

# Acceptance bar for floating-point outputs (bf16 inputs, fp32 accumulation):
MAX_REL = 1e-2      # max |err| <= 1e-2 * max |ref|
REL_L2 = 5e-3       # ||err||_2 <= 5e-3 * ||ref||_2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


class GpuCase:
    """A seeded ``inputs.Case`` with every tensor copied to the GPU."""

    def __init__(self, case, device="cuda"):
        self.case = case
        self.d = G.Dims.of(case)
        self.q_nope = case.q_nope.to(device)
        self.q_rope = case.q_rope.to(device)
        self.pages = case.pages.to(device)
        self.block_table = case.block_table.to(device)
        self.seqlens = case.seqlens.to(device)
        self.w_uk = case.w_uk.to(device)
        self.w_uv = case.w_uv.to(device)
        self.seqlens_host = [int(x) for x in case.seqlens]

    def split(self, split_tokens):
        offs, total = G.make_split_plan(self.seqlens_host, split_tokens)
        return offs, total, split_tokens

    def expand(self):
        return G.expand_cache(self.d, self.pages, self.w_uk, self.w_uv)

    def gqa(self, E, split=None):
        return G.decode_gqa(self.d, self.q_nope, self.q_rope, E, self.block_table, self.seqlens,
                            split=split)

    def absorb(self, split=None):
        return G.decode_mqa_absorb(self.d, self.q_nope, self.q_rope, self.pages, self.block_table,
                                   self.seqlens, self.w_uk, self.w_uv, split=split)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def assert_close(got, ref, what: str, max_rel=MAX_REL, rel_l2=REL_L2):
    st = error_stats(got, ref)
    log(f"  {what}: max_rel={st['max_rel']:.3e} rel_l2={st['rel_l2']:.3e} finite={st['finite']}")
    assert st["finite"], f"{what}: non-finite output"
    assert st["max_rel"] <= max_rel, f"{what}: max_rel {st['max_rel']:.3e} > {max_rel}"
    assert st["rel_l2"] <= rel_l2, f"{what}: rel_l2 {st['rel_l2']:.3e} > {rel_l2}"
    return st


def assert_lse_close(got, ref, what: str, tol=2e-2):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = float(np.max(np.abs(got - ref)))
    log(f"  {what}: max|lse err|={err:.3e}")
    assert np.all(np.isfinite(got)) and err <= tol, f"{what}: lse err {err}"
