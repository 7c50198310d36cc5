"""Algorithmic bytes / FLOPs of the GQLA decode paths and the roofline model.

Counting convention (the one that reproduces every number the GQLA pages
print; paperlayer.ai section 4 "Roofline analysis"): 2 FLOPs per
multiply-accumulate, QK and PV only, bf16 cache (2 bytes per element), each
cache byte read once.

* Cache per token: latent r + d_R elements; expanded 2*g*d_h + d_R elements
  (paperlayer.ai section 5 "Conversion setup"; section 4 "GQA path" quotes
  4224 B per token for g = 8).
* Intensity of the absorb path: h_q*s_q*(2r + d_R)/(r + d_R) FLOP/B -- the
  latent is read once and reused by every query row (section 4 "MQA-absorb
  path": ~242 at s_q = 1, ~484 at s_q = 2).
* Intensity of the GQA path: h_q*s_q*(2*d_h + d_R)/(2*g*d_h + d_R) FLOP/B
  (section 4 "GQA path": ~38.8 at (g, s_q) = (8, 2), ~37.6 at (4, 1)).
* Roofline bound: time = max(bytes / BW, FLOPs / peak) (section 4 "Roofline
  motivation": throughput bound min(I * BW, FLOPs_max)).

Per-launch algorithmic bytes add, to the cache bytes, the query (q_nope and
q_rope, bf16), the output (bf16) and -- on the absorb path -- the two weight
tensors, each moved once.  Split partials are not algorithmic traffic.
"""
from __future__ import annotations

from dataclasses import dataclass

BF16 = 2

# MI355X published peaks (dense; no sparsity).
MI355X_HBM_GBPS = 8000.0            # GB/s
MI355X_BF16_TFLOPS = 2500.0         # dense bf16 MFMA, TFLOP/s
MI355X_FP32_TFLOPS = 157.3

# Hardware the pages' predictions are quoted for (context only).  The H20
# figures are printed on the pages (pwwt.cn section 2: ~148 TFLOPS, ~4.0
# TB/s); the H100 figures are the public dense-bf16 / HBM3 numbers that give
# the pages' ridge of ~295 FLOP/B.
H100 = dict(tflops=989.0, tbps=3.35)
H20 = dict(tflops=148.0, tbps=4.0)


def latent_elems_per_token(r: int, d_R: int) -> int:
    return r + d_R


def expanded_elems_per_token(g: int, d_h: int, d_R: int) -> int:
    return 2 * g * d_h + d_R


def intensity_absorb(h_q: int, s_q: int, r: int, d_R: int) -> float:
    return h_q * s_q * (2 * r + d_R) / (r + d_R)


def intensity_gqa(h_q: int, s_q: int, g: int, d_h: int, d_R: int) -> float:
    return h_q * s_q * (2 * d_h + d_R) / (2 * g * d_h + d_R)


def flops_per_token_absorb(h_q: int, s_q: int, r: int, d_R: int) -> int:
    """QK over r + d_R plus PV over r, per cache token, all h_q*s_q rows."""
    return 2 * h_q * s_q * (2 * r + d_R)


def flops_per_token_gqa(h_q: int, s_q: int, d_h: int, d_R: int) -> int:
    return 2 * h_q * s_q * (2 * d_h + d_R)


def model_step_us(bytes_: float, flops: float, tbps: float, tflops: float) -> float:
    """The pages' roofline step time: max(memory time, compute time), in microseconds."""
    return max(bytes_ / (tbps * 1e12), flops / (tflops * 1e12)) * 1e6


@dataclass
class Work:
    bytes: int
    flops: int
    cache_bytes: int

    def hbm_us(self, gbps=MI355X_HBM_GBPS) -> float:
        return self.bytes / (gbps * 1e9) * 1e6

    def mfma_us(self, tflops=MI355X_BF16_TFLOPS) -> float:
        return self.flops / (tflops * 1e12) * 1e6

    def roofline_us(self) -> float:
        return max(self.hbm_us(), self.mfma_us())

    def bound(self) -> str:
        return "hbm" if self.hbm_us() >= self.mfma_us() else "mfma"


def _visible(L: int, s_q: int):
    return [L - s_q + i + 1 for i in range(s_q)]


def work_absorb(seqlens, h_q, g, r, d_R, d_nope, d_v, s_q) -> Work:
    """Algorithmic work of one gqla_decode_mqa_absorb call over the batch."""
    B = len(seqlens)
    cache = sum(int(L) for L in seqlens) * latent_elems_per_token(r, d_R) * BF16
    q = B * s_q * h_q * (d_nope + d_R) * BF16
    w = g * r * (d_nope + d_v) * BF16
    out = B * s_q * h_q * d_v * BF16
    attn = sum(n for L in seqlens for n in _visible(int(L), s_q)) * h_q * 2 * (2 * r + d_R)
    proj = 2 * B * s_q * h_q * r * (d_nope + d_v)
    return Work(bytes=cache + q + w + out, flops=attn + proj, cache_bytes=cache)


def work_gqa(seqlens, h_q, g, d_R, d_nope, d_v, s_q) -> Work:
    """Algorithmic work of one gqla_decode_gqa call over the batch."""
    B = len(seqlens)
    per_tok = (g * (d_nope + d_v) + d_R) * BF16
    cache = sum(int(L) for L in seqlens) * per_tok
    q = B * s_q * h_q * (d_nope + d_R) * BF16
    out = B * s_q * h_q * d_v * BF16
    attn = sum(n for L in seqlens for n in _visible(int(L), s_q)) * h_q * 2 * (d_nope + d_R + d_v)
    return Work(bytes=cache + q + out, flops=attn, cache_bytes=cache)


def work_gqa_sparse(indices, seqlens, h_q, g, d_R, d_nope, d_v, s_q) -> Work:
    """Algorithmic work of one gqla_decode_gqa_sparse call: every valid entry of group G moves
    its K, V and rope rows once (each group gathers its own rows, rope included), plus the
    queries, the index lists and the output; FLOPs count each (row, visible entry) pair."""
    B = len(seqlens)
    hpg = h_q // g
    entries = 0
    pairs = 0
    n_idx = 0
    for b in range(B):
        L = int(seqlens[b])
        for G in range(g):
            ts = [int(t) for t in indices[b][G]]
            n_idx += len(ts)
            valid = [t for t in ts if 0 <= t < L]
            entries += len(valid)
            pairs += sum(1 for i in range(s_q) for t in valid if t <= L - s_q + i)
    cache = entries * (d_nope + d_v + d_R) * BF16
    q = B * s_q * h_q * (d_nope + d_R) * BF16
    out = B * s_q * h_q * d_v * BF16
    return Work(bytes=cache + q + out + n_idx * 4, flops=pairs * hpg * 2 * (d_nope + d_R + d_v),
                cache_bytes=cache)


def work_expand(num_pages, bs, g, r, d_R, d_nope, d_v) -> Work:
    tokens = num_pages * bs
    read = tokens * (r + d_R) * BF16 + g * r * (d_nope + d_v) * BF16
    write = tokens * (g * (d_nope + d_v) + d_R) * BF16
    return Work(bytes=read + write, flops=2 * tokens * r * g * (d_nope + d_v),
                cache_bytes=tokens * (r + d_R) * BF16)


def work_combine(total_splits, batch, s_q, h_q, d_v) -> Work:
    read = total_splits * s_q * h_q * (d_v + 1) * 4
    write = batch * s_q * h_q * (d_v * BF16 + 4)
    return Work(bytes=read + write, flops=0, cache_bytes=0)
