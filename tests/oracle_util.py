"""Helpers that hand seeded cases to the oracle (tests only)."""
from __future__ import annotations

import numpy as np
import torch

from oracle.gqla_ref import Dims


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def dims_of(case, s_q=None) -> Dims:
    return Dims(h_q=case.h_q, g=case.g, r=case.r, d_R=case.d_R, d_nope=case.d_nope,
                d_v=case.d_v, s_q=case.s_q if s_q is None else s_q, bs=case.bs)


def oracle_args(case):
    """(q_nope, q_rope, pages, block_table, seqlens, w_uk, w_uv) as float64 / int numpy."""
    return (to64(case.q_nope), to64(case.q_rope), to64(case.pages),
            case.block_table.numpy().astype(np.int64), case.seqlens.numpy().astype(np.int64),
            to64(case.w_uk), to64(case.w_uv))
