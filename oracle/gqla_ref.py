"""fp64 numpy oracle of GQLA decode attention (test infrastructure only).

Everything here is written from the definition, in float64, with no blocking,
fusion or reordering beyond what the definition states.  Inputs are numpy
arrays (any float dtype; they are converted to float64 exactly).

Notation (GQLA pages, paperlayer.ai section 3 "Architecture"; gist.science
section 2 "Methodik"):

  h_q      query heads              g        KV groups (one W_UK/W_UV each)
  r        latent dim of c^KV_t     d_R      shared decoupled-RoPE key dim
  d_nope   per-head K-NoPE dim      d_v      per-head V dim
  s_q      query tokens per sequence per decode step (1 + MTP heads)
  bs       tokens per cache page

Readings where the pages are silent (each is listed in the design doc):

* head h belongs to group G = h // (h_q // g)  (contiguous GQA grouping);
* W_UK[G] is (r x d_nope) and the key of token t for group G is the row
  vector c_t @ W_UK[G]; likewise V = c_t @ W_UV[G] with W_UV[G] (r x d_v);
* logit scale is 1/sqrt(d_nope + d_R);
* q_rope and k_rope arrive already rotated;
* cache_seqlens[b] counts the s_q new tokens; query row i of sequence b sits
  at position L_b - s_q + i and sees tokens t <= L_b - s_q + i;
* lse is the natural log of sum(exp(scaled logits)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Dims:
    h_q: int
    g: int
    r: int
    d_R: int
    d_nope: int
    d_v: int
    s_q: int
    bs: int = 64

    @property
    def heads_per_group(self) -> int:
        return self.h_q // self.g

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_nope + self.d_R)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even), from the format definition:
# 1 sign bit, 8 exponent bits (same range as fp32), 7 stored mantissa bits.
# ---------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Works directly from float64 (no intermediate float32, so no double
    rounding).  Normal bf16 numbers carry 8 significant bits; below 2**-126
    the spacing is fixed at 2**-133 (subnormals).  Values whose rounded
    magnitude reaches 2**128 become +-inf.  NaN stays NaN.
    """
    x = _f64(x)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    xf = x[finite]
    _, e2 = np.frexp(xf)                 # |x| in [2**(e2-1), 2**e2)
    e = np.maximum(e2 - 1, -126)         # unbiased exponent, clamped at subnormal range
    ulp = np.ldexp(1.0, e - 7)           # spacing of bf16 values at that exponent
    q = np.round(xf / ulp) * ulp         # np.round is round-half-to-even; scaling is exact
    q = np.where(np.abs(q) >= 2.0 ** 128, np.copysign(np.inf, xf), q)
    out[finite] = q
    return out


# ---------------------------------------------------------------------------
# Paged latent cache: token t of sequence b is slot t % bs of page
# block_table[b][t // bs].  A latent page row holds [c_t (r) | k_rope_t (d_R)].
# ---------------------------------------------------------------------------
def gather_latent(pages, block_table_row, L: int, d: Dims) -> tuple[np.ndarray, np.ndarray]:
    """Return (C, KR): the L latent rows (L x r) and rope keys (L x d_R) of one sequence."""
    pages = _f64(pages)
    rows = np.empty((L, d.r + d.d_R), dtype=np.float64)
    for t in range(L):
        page = int(block_table_row[t // d.bs])
        rows[t] = pages[page, t % d.bs]
    return rows[:, : d.r], rows[:, d.r:]


def visible_tokens(L: int, i: int, s_q: int) -> int:
    """Number of cache tokens query row i of an s_q-row step can attend to (causal MTP mask)."""
    return L - s_q + i + 1


def _softmax_attend(scores: np.ndarray, values: np.ndarray) -> tuple[np.ndarray, float]:
    """softmax(scores) @ values and the natural-log sum-exp of scores."""
    m = float(np.max(scores))
    e = np.exp(scores - m)
    z = float(np.sum(e))
    return (e @ values) / z, m + math.log(z)


def decode_literal(q_nope, q_rope, pages, block_table, seqlens, w_uk, w_uv, d: Dims,
                   seqs=None):
    """GQA form, written literally: expand the latent per group, then attend.

    out[b,i,h] = softmax_t((q_nope[b,i,h] . (c_t W_UK[G]) + q_rope[b,i,h] . k_rope_t) * scale)
                 @ (c_t W_UV[G]),   t < L_b - s_q + i + 1,  G = h // (h_q/g).

    Returns (out [B', s_q, h_q, d_v], lse [B', s_q, h_q]) for the sequences in
    ``seqs`` (default: all), in that order.
    Pinned by: brute force (``brute.decode``), torch SDPA in fp64, special
    cases (L=1, q=0, one dominant logit, selection W_UV), the absorb form.
    """
    q_nope, q_rope, w_uk, w_uv = map(_f64, (q_nope, q_rope, w_uk, w_uv))
    seqs = range(q_nope.shape[0]) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), d.s_q, d.h_q, d.d_v))
    lse = np.zeros((len(seqs), d.s_q, d.h_q))
    for bi, b in enumerate(seqs):
        L = int(seqlens[b])
        C, KR = gather_latent(pages, block_table[b], L, d)
        for G in range(d.g):
            K = C @ w_uk[G]                      # L x d_nope
            V = C @ w_uv[G]                      # L x d_v
            for h in range(G * d.heads_per_group, (G + 1) * d.heads_per_group):
                for i in range(d.s_q):
                    n = visible_tokens(L, i, d.s_q)
                    s = (K[:n] @ q_nope[b, i, h] + KR[:n] @ q_rope[b, i, h]) * d.scale
                    out[bi, i, h], lse[bi, i, h] = _softmax_attend(s, V[:n])
    return out, lse


def decode_absorb_form(q_nope, q_rope, pages, block_table, seqlens, w_uk, w_uv, d: Dims,
                       seqs=None):
    """MQA-absorb form: fold W_UK[G] into the query, attend over the latent, up-project by W_UV[G].

    q_abs = W_UK[G] @ q_nope[b,i,h]   (r),
    s_t   = (q_abs . c_t + q_rope . k_rope_t) * scale,
    o_lat = softmax(s) @ C            (r),
    out   = o_lat @ W_UV[G]           (d_v).

    Algebraically equal to ``decode_literal`` (the pages' "two algebraically
    equivalent decoding paths").  Pinned by agreement with decode_literal to
    ~1e-12 relative in fp64.
    """
    q_nope, q_rope, w_uk, w_uv = map(_f64, (q_nope, q_rope, w_uk, w_uv))
    seqs = range(q_nope.shape[0]) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), d.s_q, d.h_q, d.d_v))
    lse = np.zeros((len(seqs), d.s_q, d.h_q))
    for bi, b in enumerate(seqs):
        L = int(seqlens[b])
        C, KR = gather_latent(pages, block_table[b], L, d)
        for h in range(d.h_q):
            G = h // d.heads_per_group
            for i in range(d.s_q):
                n = visible_tokens(L, i, d.s_q)
                q_abs = w_uk[G] @ q_nope[b, i, h]
                s = (C[:n] @ q_abs + KR[:n] @ q_rope[b, i, h]) * d.scale
                o_lat, lse[bi, i, h] = _softmax_attend(s, C[:n])
                out[bi, i, h] = o_lat @ w_uv[G]
    return out, lse


# ---------------------------------------------------------------------------
# Expanded (per-group) cache.  The pages fix only its size, 2*g*d_h + d_R
# elements per token (paperlayer.ai section 5, "Conversion setup").  Our page
# layout, for one page of bs slots:
#   for G in 0..g-1:  K block  [bs slots][d_nope]   (token-major)
#                     V block  [bs slots][d_v]      (token-major)
#   then              rope     [bs slots][d_R]
# (every per-token row is contiguous, so a decode over a per-group token
# subset gathers whole rows)
# so a page holds bs*(g*(d_nope+d_v) + d_R) elements.
# ---------------------------------------------------------------------------
def expanded_page_elems(d: Dims) -> int:
    return d.bs * (d.g * (d.d_nope + d.d_v) + d.d_R)


def expanded_offset_k(d: Dims, G: int, slot: int, j: int) -> int:
    return G * d.bs * (d.d_nope + d.d_v) + slot * d.d_nope + j


def expanded_offset_v(d: Dims, G: int, slot: int, j: int) -> int:
    return G * d.bs * (d.d_nope + d.d_v) + d.bs * d.d_nope + slot * d.d_v + j


def expanded_offset_rope(d: Dims, slot: int, j: int) -> int:
    return d.g * d.bs * (d.d_nope + d.d_v) + slot * d.d_R + j


def expand_pages(pages, w_uk, w_uv, d: Dims, page_ids=None) -> np.ndarray:
    """One-shot latent -> per-group expansion of whole pages (every slot).

    K[t,G] = RNE_bf16(c_t @ W_UK[G]),  V[t,G] = RNE_bf16(c_t @ W_UV[G]) computed
    exactly in fp64 before the single rounding; k_rope copied unchanged.
    Output: [n_pages', expanded_page_elems] float64 holding bf16 values, in the
    layout described above.  Pinned by: selection-matrix weights (pure
    gather), bf16 rounding pins, and decode over the expanded cache equal to
    the literal decode.
    """
    pages, w_uk, w_uv = map(_f64, (pages, w_uk, w_uv))
    page_ids = range(pages.shape[0]) if page_ids is None else list(page_ids)
    out = np.zeros((len(page_ids), expanded_page_elems(d)))
    for pi, p in enumerate(page_ids):
        C = pages[p, :, : d.r]
        KR = pages[p, :, d.r:]
        for G in range(d.g):
            k_view, v_view = _expanded_group_views(out[pi], d, G)
            k_view[...] = bf16_round(C @ w_uk[G])        # [slot][j]
            v_view[...] = bf16_round(C @ w_uv[G])        # [slot][j]
        _expanded_rope_view(out[pi], d)[...] = KR
    return out


def _expanded_group_views(page: np.ndarray, d: Dims, G: int):
    """Views of one page's group-G blocks: K as [slot][j], V as [slot][j]."""
    base = G * d.bs * (d.d_nope + d.d_v)
    k_view = page[base: base + d.bs * d.d_nope].reshape(d.bs, d.d_nope)
    v_view = page[base + d.bs * d.d_nope: base + d.bs * (d.d_nope + d.d_v)].reshape(d.bs, d.d_v)
    return k_view, v_view


def _expanded_rope_view(page: np.ndarray, d: Dims):
    base = d.g * d.bs * (d.d_nope + d.d_v)
    return page[base: base + d.bs * d.d_R].reshape(d.bs, d.d_R)


def decode_gqa_expanded(q_nope, q_rope, expanded_pages, block_table, seqlens, d: Dims,
                        seqs=None):
    """GQA decode over a stored expanded cache (layout above); no weights involved.

    Separates kernel error from expansion rounding: feeding it the expanded
    cache the GPU produced gives the exact answer for that cache.
    """
    q_nope, q_rope, E = map(_f64, (q_nope, q_rope, expanded_pages))
    seqs = range(q_nope.shape[0]) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), d.s_q, d.h_q, d.d_v))
    lse = np.zeros((len(seqs), d.s_q, d.h_q))
    for bi, b in enumerate(seqs):
        L = int(seqlens[b])
        for G in range(d.g):
            K = np.empty((L, d.d_nope))
            V = np.empty((L, d.d_v))
            KR = np.empty((L, d.d_R))
            for t in range(L):
                page = E[int(block_table[b][t // d.bs])]
                slot = t % d.bs
                k_view, v_view = _expanded_group_views(page, d, G)
                K[t] = k_view[slot]
                V[t] = v_view[slot]
                KR[t] = _expanded_rope_view(page, d)[slot]
            for h in range(G * d.heads_per_group, (G + 1) * d.heads_per_group):
                for i in range(d.s_q):
                    n = visible_tokens(L, i, d.s_q)
                    s = (K[:n] @ q_nope[b, i, h] + KR[:n] @ q_rope[b, i, h]) * d.scale
                    out[bi, i, h], lse[bi, i, h] = _softmax_attend(s, V[:n])
    return out, lse


# ---------------------------------------------------------------------------
# Sparse GQLA on the GQA path (gist.science section 2, subsection "Sparse
# GQLA"; pwwt.cn section 5 on the sparse extension; ai-feeds.com "Methods",
# the optional sparse extension).  Each KV group attends to its own subset of
# the cached tokens, and the subset is shared by every query head of the
# group, which is what keeps a group's h_q/g heads a dense matrix tile.  The
# pages leave open how the subset is chosen (an indexer such as DSA or HISA
# picks it); here it is an input: indices[b][G] lists token positions of
# sequence b.  Readings (each listed in the design notes):
# * the list is shared by the s_q query rows of the step as well; row i still
#   sees only positions t <= L - s_q + i (the causal MTP mask);
# * entries outside [0, L) (e.g. -1 padding) are ignored;
# * every remaining entry is one attention term, in list order, so an entry
#   listed twice counts twice;
# * a row that sees no entry gets out = 0 and lse = -inf.
# ---------------------------------------------------------------------------
def decode_gqa_sparse(q_nope, q_rope, expanded_pages, block_table, seqlens, indices, d: Dims,
                      seqs=None):
    """Sparse GQA decode over a stored expanded cache: softmax over the listed tokens only."""
    q_nope, q_rope, E = map(_f64, (q_nope, q_rope, expanded_pages))
    indices = np.asarray(indices)
    seqs = range(q_nope.shape[0]) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), d.s_q, d.h_q, d.d_v))
    lse = np.full((len(seqs), d.s_q, d.h_q), -np.inf)
    for bi, b in enumerate(seqs):
        L = int(seqlens[b])
        for G in range(d.g):
            sel = [int(t) for t in indices[b][G] if 0 <= int(t) < L]
            n = len(sel)
            K = np.empty((n, d.d_nope))
            V = np.empty((n, d.d_v))
            KR = np.empty((n, d.d_R))
            for e, t in enumerate(sel):
                page = E[int(block_table[b][t // d.bs])]
                slot = t % d.bs
                k_view, v_view = _expanded_group_views(page, d, G)
                K[e] = k_view[slot]
                V[e] = v_view[slot]
                KR[e] = _expanded_rope_view(page, d)[slot]
            for i in range(d.s_q):
                vis = np.array([t < visible_tokens(L, i, d.s_q) for t in sel], dtype=bool)
                if not vis.any():
                    continue                      # out stays 0, lse -inf
                for h in range(G * d.heads_per_group, (G + 1) * d.heads_per_group):
                    s = (K[vis] @ q_nope[b, i, h] + KR[vis] @ q_rope[b, i, h]) * d.scale
                    out[bi, i, h], lse[bi, i, h] = _softmax_attend(s, V[vis])
    return out, lse


# ---------------------------------------------------------------------------
# Split-KV partials and their log-sum-exp merge (the pages are silent on
# split-KV; this is the standard exact decomposition of a softmax over a
# union of disjoint token ranges).
# ---------------------------------------------------------------------------
def split_ranges(L: int, split_tokens: int) -> list[tuple[int, int]]:
    """Disjoint token ranges [lo, hi) of length split_tokens covering [0, L)."""
    return [(lo, min(lo + split_tokens, L)) for lo in range(0, L, split_tokens)]


def decode_partials(q_nope, q_rope, pages, block_table, seqlens, w_uk, w_uv, d: Dims,
                    split_tokens: int):
    """Per-split normalized outputs and lse, literal form.

    For split [lo, hi) of sequence b and row (i, h): the attention restricted
    to visible tokens in [lo, hi).  A split with no visible token has
    out = 0 and lse = -inf.  Splits are numbered sequence by sequence.
    Returns (part_out [S, s_q, h_q, d_v], part_lse [S, s_q, h_q], offsets [B+1]).
    """
    q_nope, q_rope, w_uk, w_uv = map(_f64, (q_nope, q_rope, w_uk, w_uv))
    B = q_nope.shape[0]
    parts_o, parts_l, offsets = [], [], [0]
    for b in range(B):
        L = int(seqlens[b])
        C, KR = gather_latent(pages, block_table[b], L, d)
        ranges = split_ranges(L, split_tokens)
        offsets.append(offsets[-1] + len(ranges))
        for lo, hi in ranges:
            po = np.zeros((d.s_q, d.h_q, d.d_v))
            pl = np.full((d.s_q, d.h_q), -np.inf)
            for G in range(d.g):
                K = C @ w_uk[G]
                V = C @ w_uv[G]
                for h in range(G * d.heads_per_group, (G + 1) * d.heads_per_group):
                    for i in range(d.s_q):
                        n_hi = min(hi, visible_tokens(L, i, d.s_q))
                        if n_hi <= lo:
                            continue
                        s = (K[lo:n_hi] @ q_nope[b, i, h] + KR[lo:n_hi] @ q_rope[b, i, h]) * d.scale
                        po[i, h], pl[i, h] = _softmax_attend(s, V[lo:n_hi])
            parts_o.append(po)
            parts_l.append(pl)
    return np.stack(parts_o), np.stack(parts_l), np.array(offsets)


def decode_partials_latent(q_nope, q_rope, pages, block_table, seqlens, w_uk, d: Dims,
                           split_tokens: int):
    """Per-split normalized latent outputs and lse, absorb form.

    For split [lo, hi) of sequence b and row (i, h) of group G:
    q_abs = W_UK[G] q_nope[b,i,h], s_t = (q_abs . c_t + q_rope . k_rope_t) * scale
    over the visible tokens t in [lo, hi), o_lat = softmax(s) C (d_latent wide).
    These are the split partials of the MQA-absorb path taken before the
    up-projection by W_UV[G] (paperlayer.ai section 4, "MQA-absorb path":
    attention runs over the latent, W_UV maps its output back); o_lat W_UV[G]
    is the ``decode_partials`` output of the same split, by linearity.
    A split with no visible token has o_lat = 0 and lse = -inf.
    Returns (part_lat [S, s_q, h_q, d_latent], part_lse [S, s_q, h_q], offsets [B+1]).
    """
    q_nope, q_rope, w_uk = map(_f64, (q_nope, q_rope, w_uk))
    B = q_nope.shape[0]
    parts_o, parts_l, offsets = [], [], [0]
    for b in range(B):
        L = int(seqlens[b])
        C, KR = gather_latent(pages, block_table[b], L, d)
        ranges = split_ranges(L, split_tokens)
        offsets.append(offsets[-1] + len(ranges))
        for lo, hi in ranges:
            po = np.zeros((d.s_q, d.h_q, d.r))
            pl = np.full((d.s_q, d.h_q), -np.inf)
            for h in range(d.h_q):
                G = h // d.heads_per_group
                for i in range(d.s_q):
                    n_hi = min(hi, visible_tokens(L, i, d.s_q))
                    if n_hi <= lo:
                        continue
                    q_abs = w_uk[G] @ q_nope[b, i, h]
                    s = (C[lo:n_hi] @ q_abs + KR[lo:n_hi] @ q_rope[b, i, h]) * d.scale
                    po[i, h], pl[i, h] = _softmax_attend(s, C[lo:n_hi])
            parts_o.append(po)
            parts_l.append(pl)
    return np.stack(parts_o), np.stack(parts_l), np.array(offsets)


def combine(part_out, part_lse, split_offsets):
    """Merge normalized split partials by log-sum-exp.

    For each output row: m = max_s lse_s, w_s = exp(lse_s - m),
    out = sum_s w_s o_s / sum_s w_s, lse = m + log(sum_s w_s).
    Splits with lse = -inf carry weight 0.  If every split of a row is empty
    the row is out = 0, lse = -inf.
    Returns (out [B, ...], lse [B, ...]).
    """
    part_out, part_lse = _f64(part_out), _f64(part_lse)
    B = len(split_offsets) - 1
    out = np.zeros((B,) + part_out.shape[1:])
    lse = np.full((B,) + part_lse.shape[1:], -np.inf)
    for b in range(B):
        lo, hi = int(split_offsets[b]), int(split_offsets[b + 1])
        for idx in np.ndindex(*part_lse.shape[1:]):
            ls = [part_lse[(s,) + idx] for s in range(lo, hi)]
            if not ls or all(v == -np.inf for v in ls):
                continue
            m = max(ls)
            w = [0.0 if v == -np.inf else math.exp(v - m) for v in ls]
            z = sum(w)
            acc = np.zeros(part_out.shape[-1])
            for s, ws in zip(range(lo, hi), w):
                if ws != 0.0:
                    acc += ws * part_out[(s,) + idx]
            out[(b,) + idx] = acc / z
            lse[(b,) + idx] = m + math.log(z)
    return out, lse


# ---------------------------------------------------------------------------
# Acceptance metric used by the parity tests.
# ---------------------------------------------------------------------------
def _ratio(num: float, den: float) -> float:
    """num / den for the acceptance ratios; a zero reference scale admits only a zero error."""
    if den > 0:
        return num / den
    return 0.0 if num == 0 else math.inf


def error_stats(got, ref) -> dict:
    """The acceptance metric of the parity tests, for got against ref (float64):

      max_rel = max_i |got_i - ref_i| / max_i |ref_i|      (both maxima over all elements)
      rel_l2  = ||got - ref||_2 / ||ref||_2                 (Euclidean norms, not squared)

    so the bar max|err| <= tol * max|ref| reads max_rel <= tol.  With ref all zero the bar
    admits only got == ref: the ratio is then 0 for a zero error and inf otherwise.  `finite`
    is False when got holds a NaN or an infinity (max_rel and rel_l2 are then NaN or inf)."""
    got, ref = _f64(got), _f64(ref)
    if got.shape != ref.shape:
        raise ValueError(f"shape mismatch: {got.shape} vs {ref.shape}")
    err = got - ref
    max_err = float(np.max(np.abs(err))) if err.size else 0.0
    max_ref = float(np.max(np.abs(ref))) if ref.size else 0.0
    l2_err = float(np.linalg.norm(err.ravel()))
    l2_ref = float(np.linalg.norm(ref.ravel()))
    return {
        "max_err": max_err,
        "max_ref": max_ref,
        "max_rel": _ratio(max_err, max_ref),
        "rel_l2": _ratio(l2_err, l2_ref),
        "finite": bool(np.all(np.isfinite(got))),
    }
