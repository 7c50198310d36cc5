"""GQLA decode attention on MI355X (gfx950): Python binding of libgqla.

The functions below carry the C-ABI names (include/gqla.h) and only marshal
arguments: they check tensor devices, dtypes and shapes, pass raw device
pointers and the current HIP stream to the library, and raise on a negative
status.  Every step of the computation runs in the library's HIP kernels;
there is no CPU fallback -- if libgqla.so is missing or no GPU is visible the
calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "GqlaError", "Dims", "lib", "gqla_expand_cache", "gqla_decode_mqa_absorb", "gqla_decode_gqa",
    "gqla_splitkv_combine", "gqla_decode_gqa_sparse", "gqla_sparse_workspace_bytes",
    "sparse_workspace", "gqla_sparse_workspace_offsets", "gqla_status_string", "make_split_plan", "latent_page_elems",
    "expanded_page_elems", "decode_mqa_absorb", "decode_gqa", "expand_cache",
    "gqla_mqa_absorb_workspace_bytes", "gqla_mqa_absorb_workspace_offsets", "absorb_workspace",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqla.so")

GQLA_OK = 0
STATUS_NAMES = {0: "GQLA_OK", -1: "GQLA_ERR_INVALID_ARG", -2: "GQLA_ERR_UNSUPPORTED_SHAPE",
                -3: "GQLA_ERR_MISALIGNED", -4: "GQLA_ERR_BAD_SPLIT_PLAN", -5: "GQLA_ERR_HIP",
                -6: "GQLA_ERR_SCRATCH_LIMIT"}
NOALLOC_SCRATCH_BYTES = 32 << 20       # GQLA_NOALLOC_SCRATCH_BYTES


class GqlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gqla_status_string(status)}")


class Dims(ctypes.Structure):
    """gqla_dims: h_q, g, latent r, rope d_R, d_nope, d_v, s_q, page size, softmax scale."""
    _fields_ = [("num_heads", ctypes.c_int32), ("num_groups", ctypes.c_int32),
                ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("s_q", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]

    @classmethod
    def make(cls, h_q, g, r, d_R, d_nope, d_v, s_q, bs=64, scale=0.0) -> "Dims":
        return cls(h_q, g, r, d_R, d_nope, d_v, s_q, bs, scale)

    @classmethod
    def of(cls, case) -> "Dims":
        """Dims of an ``inputs.Case``."""
        return cls.make(case.h_q, case.g, case.r, case.d_R, case.d_nope, case.d_v, case.s_q, case.bs)


class Hw(ctypes.Structure):
    """gqla_hw: sustained HBM GB/s and bf16 matrix TFLOP/s, the fraction of the roofline each
    path reaches, and the byte-counting convention (cache_only = the pages' step-time model)."""
    _fields_ = [("hbm_gbps", ctypes.c_double), ("mfma_tflops", ctypes.c_double),
                ("frac_absorb", ctypes.c_double), ("frac_gqa", ctypes.c_double),
                ("cache_only", ctypes.c_int32)]


class PathEstimate(ctypes.Structure):
    """gqla_path_estimate: roofline estimate of one decode call of one path."""
    _fields_ = [("bytes", ctypes.c_double), ("flops", ctypes.c_double),
                ("t_hbm_us", ctypes.c_double), ("t_mfma_us", ctypes.c_double),
                ("t_roofline_us", ctypes.c_double), ("t_expected_us", ctypes.c_double),
                ("tokens_per_s", ctypes.c_double), ("bound", ctypes.c_int32)]

    def as_dict(self) -> dict:
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["bound"] = "mfma" if self.bound else "hbm"
        return d


PATH_ABSORB, PATH_GQA = 0, 1

_vp, _i32p, _f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
_SIGS = {
    "gqla_abi_version": ([], ctypes.c_int),
    "gqla_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "gqla_latent_page_elems": ([ctypes.POINTER(Dims)], ctypes.c_int64),
    "gqla_expanded_page_elems": ([ctypes.POINTER(Dims)], ctypes.c_int64),
    "gqla_expand_cache": ([ctypes.POINTER(Dims), _vp, _vp, _vp, ctypes.c_int64, _i32p,
                           ctypes.c_int64, _vp, _vp], ctypes.c_int),
    "gqla_decode_mqa_absorb": ([ctypes.POINTER(Dims), ctypes.c_int32, _vp, _vp, _vp, _i32p,
                                ctypes.c_int32, _i32p, _vp, _vp, _i32p, ctypes.c_int32,
                                ctypes.c_int32, _vp, _f32p, _vp, ctypes.c_uint64, _vp],
                               ctypes.c_int),
    "gqla_mqa_absorb_workspace_bytes": ([ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32],
                                        ctypes.c_uint64),
    "gqla_mqa_absorb_workspace_offsets": ([ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
    "gqla_decode_mqa_absorb_noalloc": ([ctypes.POINTER(Dims), ctypes.c_int32, _vp, _vp, _vp, _i32p,
                                        ctypes.c_int32, _i32p, _vp, _vp, _i32p, ctypes.c_int32,
                                        ctypes.c_int32, _vp, _f32p, _vp], ctypes.c_int),
    "gqla_mqa_absorb_merge": ([ctypes.POINTER(Dims), ctypes.c_int32, _vp, _f32p, _i32p, ctypes.c_int32, _vp,
                               _vp, _f32p, _vp, ctypes.c_uint64, _vp], ctypes.c_int),
    "gqla_mqa_absorb_merge_workspace_bytes": ([ctypes.POINTER(Dims)], ctypes.c_uint64),
    "gqla_decode_gqa": ([ctypes.POINTER(Dims), ctypes.c_int32, _vp, _vp, _vp, _i32p,
                         ctypes.c_int32, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32, _vp,
                         _f32p, _f32p, _f32p, _vp], ctypes.c_int),
    "gqla_splitkv_combine": ([ctypes.POINTER(Dims), ctypes.c_int32, _i32p, ctypes.c_int32,
                              _f32p, _f32p, _vp, _f32p, _vp], ctypes.c_int),
    "gqla_decode_gqa_sparse": ([ctypes.POINTER(Dims), ctypes.c_int32, _vp, _vp, _vp, ctypes.c_int64,
                                _i32p, ctypes.c_int32, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                _vp, _f32p, _vp, ctypes.c_uint64, _vp], ctypes.c_int),
    "gqla_sparse_workspace_bytes": ([ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32], ctypes.c_uint64),
    "gqla_sparse_workspace_offsets": ([ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
    "gqla_append_tokens": ([ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32, _vp, _vp,
                            ctypes.c_int64, _i32p, ctypes.c_int32, _i32p, _vp, _vp, _vp, _vp],
                           ctypes.c_int),
    "gqla_select_path": ([ctypes.POINTER(Dims), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                          ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(Hw),
                          ctypes.POINTER(PathEstimate), ctypes.POINTER(PathEstimate)], ctypes.c_int),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libgqla.so (built in-tree by ``decode_attention_gqla_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m decode_attention_gqla_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def gqla_status_string(status: int) -> str:
    try:
        return lib().gqla_status_string(int(status)).decode()
    except ImportError:
        return STATUS_NAMES.get(status, f"status {status}")


def latent_page_elems(d: Dims) -> int:
    return int(lib().gqla_latent_page_elems(ctypes.byref(d)))


def expanded_page_elems(d: Dims) -> int:
    return int(lib().gqla_expanded_page_elems(ctypes.byref(d)))


# --- marshalling helpers ------------------------------------------------------
def _ptr(t, dtype, name, shape=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != GQLA_OK:
        raise GqlaError(status, where)


# --- raw entry points (same names and arguments as the C ABI) -------------------
def gqla_expand_cache(d: Dims, latent_pages, w_uk, w_uv, expanded_pages, page_ids=None,
                      stream=None) -> None:
    n_pages = latent_pages.shape[0]
    bs = d.block_size
    _ptr(latent_pages, torch.bfloat16, "latent_pages", (n_pages, bs, d.d_latent + d.d_rope))
    n_exp = page_ids.numel() if page_ids is not None else n_pages
    st = lib().gqla_expand_cache(
        ctypes.byref(d), _ptr(latent_pages, torch.bfloat16, "latent_pages"),
        _ptr(w_uk, torch.bfloat16, "w_uk", (d.num_groups, d.d_latent, d.d_nope)),
        _ptr(w_uv, torch.bfloat16, "w_uv", (d.num_groups, d.d_latent, d.d_v)),
        n_pages, _ptr(page_ids, torch.int32, "page_ids", allow_none=True), n_exp,
        _ptr(expanded_pages, torch.bfloat16, "expanded_pages",
             (n_pages, bs * (d.num_groups * (d.d_nope + d.d_v) + d.d_rope))),
        _stream(stream))
    _check(st, "gqla_expand_cache")


def _decode_common(d, q_nope, q_rope, block_table, cache_seqlens, split_offsets, total_splits,
                   out, lse, part_out, part_lse):
    B = q_nope.shape[0]
    args = dict(
        q_nope=_ptr(q_nope, torch.bfloat16, "q_nope", (B, d.s_q, d.num_heads, d.d_nope)),
        q_rope=_ptr(q_rope, torch.bfloat16, "q_rope", (B, d.s_q, d.num_heads, d.d_rope)),
        block_table=_ptr(block_table, torch.int32, "block_table"),
        seqlens=_ptr(cache_seqlens, torch.int32, "cache_seqlens", (B,)),
        split_offsets=_ptr(split_offsets, torch.int32, "split_offsets", (B + 1,), allow_none=True),
        out=_ptr(out, torch.bfloat16, "out", (B, d.s_q, d.num_heads, d.d_v), allow_none=True),
        lse=_ptr(lse, torch.float32, "lse", (B, d.s_q, d.num_heads), allow_none=True),
        part_out=_ptr(part_out, torch.float32, "part_out", (total_splits, d.s_q, d.num_heads, d.d_v),
                      allow_none=True),
        part_lse=_ptr(part_lse, torch.float32, "part_lse", (total_splits, d.s_q, d.num_heads),
                      allow_none=True),
    )
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [batch, max_blocks]")
    return B, block_table.shape[1], args


def gqla_mqa_absorb_workspace_bytes(d: Dims, batch: int, total_splits: int = 0) -> int:
    return int(lib().gqla_mqa_absorb_workspace_bytes(ctypes.byref(d), int(batch),
                                                      int(total_splits)))


def gqla_mqa_absorb_workspace_offsets(d: Dims, batch: int, total_splits: int = 0) -> list[int]:
    """Byte offsets of the absorb workspace regions: q_abs rows, W_UV^T, split o_lat, split lse."""
    off = (ctypes.c_uint64 * 4)()
    _check(lib().gqla_mqa_absorb_workspace_offsets(ctypes.byref(d), int(batch), int(total_splits),
                                                   off), "gqla_mqa_absorb_workspace_offsets")
    return [int(x) for x in off]


def gqla_decode_mqa_absorb_noalloc(d: Dims, q_nope, q_rope, latent_pages, block_table, cache_seqlens,
                                   w_uk, w_uv, out=None, lse=None, split_offsets=None, split_tokens=0,
                                   total_splits=0, stream=None) -> None:
    """gqla_decode_mqa_absorb with the library's fixed scratch array as its workspace."""
    B, mb, a = _decode_common(d, q_nope, q_rope, block_table, cache_seqlens, split_offsets,
                              total_splits, out, lse, None, None)
    st = lib().gqla_decode_mqa_absorb_noalloc(
        ctypes.byref(d), B, a["q_nope"], a["q_rope"],
        _ptr(latent_pages, torch.bfloat16, "latent_pages"), a["block_table"], mb, a["seqlens"],
        _ptr(w_uk, torch.bfloat16, "w_uk", (d.num_groups, d.d_latent, d.d_nope)),
        _ptr(w_uv, torch.bfloat16, "w_uv", (d.num_groups, d.d_latent, d.d_v)),
        a["split_offsets"], int(split_tokens), int(total_splits), a["out"], a["lse"], _stream(stream))
    _check(st, "gqla_decode_mqa_absorb_noalloc")


def gqla_mqa_absorb_merge_workspace_bytes(d: Dims) -> int:
    return int(lib().gqla_mqa_absorb_merge_workspace_bytes(ctypes.byref(d)))


def gqla_mqa_absorb_merge(d: Dims, part_lat, part_lse, w_uv, out, lse=None, split_offsets=None,
                          total_splits=0, workspace=None, stream=None) -> None:
    """Latent-space merge of absorb split partials and the up-projection by W_UV[G]."""
    B = out.shape[0]
    units = total_splits if split_offsets is not None else B
    rows = (d.s_q, d.num_heads)
    pl = _ptr(part_lat, torch.bfloat16, "part_lat", (units,) + rows + (d.d_latent,))
    pe = _ptr(part_lse, torch.float32, "part_lse", (units,) + rows)
    so = _ptr(split_offsets, torch.int32, "split_offsets", (B + 1,), allow_none=True)
    wv = _ptr(w_uv, torch.bfloat16, "w_uv", (d.num_groups, d.d_latent, d.d_v))
    o = _ptr(out, torch.bfloat16, "out", (B,) + rows + (d.d_v,))
    ls = _ptr(lse, torch.float32, "lse", (B,) + rows, allow_none=True)
    if workspace is None:
        workspace = torch.empty(max(gqla_mqa_absorb_merge_workspace_bytes(d), 16), dtype=torch.uint8,
                                device=out.device)
    ws = _ptr(workspace, torch.uint8, "workspace")
    st = lib().gqla_mqa_absorb_merge(ctypes.byref(d), B, pl, pe, so, int(total_splits), wv, o, ls, ws,
                                     int(workspace.numel()), _stream(stream))
    _check(st, "gqla_mqa_absorb_merge")


def gqla_decode_mqa_absorb(d: Dims, q_nope, q_rope, latent_pages, block_table, cache_seqlens,
                           w_uk, w_uv, out=None, lse=None, split_offsets=None, split_tokens=0,
                           total_splits=0, workspace=None, stream=None) -> None:
    B, mb, a = _decode_common(d, q_nope, q_rope, block_table, cache_seqlens, split_offsets,
                              total_splits, out, lse, None, None)
    if workspace is None:
        raise ValueError("workspace is required (see gqla_mqa_absorb_workspace_bytes)")
    ws = _ptr(workspace, torch.uint8, "workspace")
    st = lib().gqla_decode_mqa_absorb(
        ctypes.byref(d), B, a["q_nope"], a["q_rope"],
        _ptr(latent_pages, torch.bfloat16, "latent_pages"), a["block_table"], mb, a["seqlens"],
        _ptr(w_uk, torch.bfloat16, "w_uk", (d.num_groups, d.d_latent, d.d_nope)),
        _ptr(w_uv, torch.bfloat16, "w_uv", (d.num_groups, d.d_latent, d.d_v)),
        a["split_offsets"], int(split_tokens), int(total_splits), a["out"], a["lse"],
        ws, int(workspace.numel()), _stream(stream))
    _check(st, "gqla_decode_mqa_absorb")


def gqla_decode_gqa(d: Dims, q_nope, q_rope, expanded_pages, block_table, cache_seqlens,
                    out=None, lse=None, split_offsets=None, split_tokens=0, total_splits=0,
                    part_out=None, part_lse=None, stream=None) -> None:
    B, mb, a = _decode_common(d, q_nope, q_rope, block_table, cache_seqlens, split_offsets,
                              total_splits, out, lse, part_out, part_lse)
    st = lib().gqla_decode_gqa(
        ctypes.byref(d), B, a["q_nope"], a["q_rope"],
        _ptr(expanded_pages, torch.bfloat16, "expanded_pages"), a["block_table"], mb,
        a["seqlens"], a["split_offsets"], int(split_tokens), int(total_splits), a["out"],
        a["lse"], a["part_out"], a["part_lse"], _stream(stream))
    _check(st, "gqla_decode_gqa")


def gqla_sparse_workspace_bytes(d: Dims, batch: int, topk: int, split_entries: int = 0) -> int:
    return int(lib().gqla_sparse_workspace_bytes(ctypes.byref(d), int(batch), int(topk),
                                                 int(split_entries)))


def gqla_sparse_workspace_offsets(d: Dims, batch: int, topk: int, split_entries: int = 0) -> list[int]:
    """Byte offsets of the sparse workspace regions: row codes, split plan, partials, partial
    lse, end."""
    off = (ctypes.c_uint64 * 5)()
    _check(lib().gqla_sparse_workspace_offsets(ctypes.byref(d), int(batch), int(topk),
                                               int(split_entries), off),
           "gqla_sparse_workspace_offsets")
    return [int(x) for x in off]


def sparse_workspace(d: Dims, batch: int, topk: int, split_entries: int = 0, device="cuda"):
    """A workspace tensor of the size gqla_decode_gqa_sparse needs."""
    return torch.empty(max(gqla_sparse_workspace_bytes(d, batch, topk, split_entries), 16),
                       dtype=torch.uint8, device=device)


def gqla_decode_gqa_sparse(d: Dims, q_nope, q_rope, expanded_pages, block_table, cache_seqlens,
                           indices, out, lse=None, workspace=None, split_entries=0,
                           stream=None) -> None:
    """Sparse GQA decode: group G of sequence b attends to the positions indices[b, G, :]
    (optionally split into ranges of ``split_entries`` entries, merged by log-sum-exp)."""
    B, mb, a = _decode_common(d, q_nope, q_rope, block_table, cache_seqlens, None, 0, out, lse,
                              None, None)
    if indices.dim() != 3 or indices.shape[0] != B or indices.shape[1] != d.num_groups:
        raise ValueError("indices must be int32 [batch, num_groups, topk]")
    topk = int(indices.shape[2])
    if workspace is None:
        raise ValueError("workspace is required (see gqla_sparse_workspace_bytes)")
    st = lib().gqla_decode_gqa_sparse(
        ctypes.byref(d), B, a["q_nope"], a["q_rope"],
        _ptr(expanded_pages, torch.bfloat16, "expanded_pages"), int(expanded_pages.shape[0]),
        a["block_table"], mb, a["seqlens"], _ptr(indices, torch.int32, "indices"), topk,
        int(split_entries), a["out"], a["lse"], _ptr(workspace, torch.uint8, "workspace"),
        int(workspace.numel()), _stream(stream))
    _check(st, "gqla_decode_gqa_sparse")


def gqla_splitkv_combine(d: Dims, split_offsets, part_out, part_lse, out, lse=None,
                         stream=None) -> None:
    B = split_offsets.numel() - 1
    S = part_out.shape[0]
    st = lib().gqla_splitkv_combine(
        ctypes.byref(d), B, _ptr(split_offsets, torch.int32, "split_offsets", (B + 1,)), S,
        _ptr(part_out, torch.float32, "part_out", (S, d.s_q, d.num_heads, d.d_v)),
        _ptr(part_lse, torch.float32, "part_lse", (S, d.s_q, d.num_heads)),
        _ptr(out, torch.bfloat16, "out", (B, d.s_q, d.num_heads, d.d_v)),
        _ptr(lse, torch.float32, "lse", (B, d.s_q, d.num_heads), allow_none=True),
        _stream(stream))
    _check(st, "gqla_splitkv_combine")


# --- host-side split planning and allocating conveniences ------------------------
def make_split_plan(seqlens_host, split_tokens: int, device="cuda"):
    """Split plan for split-KV decode: ceil(L_b / split_tokens) splits per sequence.

    Returns (split_offsets int32 [B+1] on ``device``, total_splits)."""
    counts = [max(1, math.ceil(int(L) / split_tokens)) for L in seqlens_host]
    offs = [0]
    for n in counts:
        offs.append(offs[-1] + n)
    return torch.tensor(offs, dtype=torch.int32, device=device), offs[-1]


def _outputs(d, B, device, with_lse):
    out = torch.empty(B, d.s_q, d.num_heads, d.d_v, dtype=torch.bfloat16, device=device)
    lse = torch.empty(B, d.s_q, d.num_heads, dtype=torch.float32, device=device) if with_lse else None
    return out, lse


def _partials(d, total, device):
    return (torch.empty(total, d.s_q, d.num_heads, d.d_v, dtype=torch.float32, device=device),
            torch.empty(total, d.s_q, d.num_heads, dtype=torch.float32, device=device))


def absorb_workspace(d: Dims, batch: int, device="cuda", total_splits: int = 0):
    """A workspace tensor (uint8) large enough for gqla_decode_mqa_absorb."""
    n = gqla_mqa_absorb_workspace_bytes(d, batch, total_splits)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def decode_mqa_absorb(d: Dims, q_nope, q_rope, latent_pages, block_table, cache_seqlens, w_uk,
                      w_uv, split=None, with_lse=True, workspace=None, stream=None):
    """Allocate outputs and run the absorb path; ``split`` = (split_offsets, total, split_tokens)."""
    B = q_nope.shape[0]
    out, lse = _outputs(d, B, q_nope.device, with_lse)
    total = split[1] if split is not None else 0
    ws = workspace if workspace is not None else absorb_workspace(d, B, q_nope.device, total)
    if split is None:
        gqla_decode_mqa_absorb(d, q_nope, q_rope, latent_pages, block_table, cache_seqlens, w_uk,
                               w_uv, out=out, lse=lse, workspace=ws, stream=stream)
    else:
        offs, total, tokens = split
        gqla_decode_mqa_absorb(d, q_nope, q_rope, latent_pages, block_table, cache_seqlens, w_uk,
                               w_uv, out=out, lse=lse, split_offsets=offs, split_tokens=tokens,
                               total_splits=total, workspace=ws, stream=stream)
    return out, lse


def decode_gqa(d: Dims, q_nope, q_rope, expanded_pages, block_table, cache_seqlens, split=None,
               with_lse=True, stream=None):
    """Allocate outputs and run the GQA path; ``split`` = (split_offsets, total, split_tokens)."""
    out, lse = _outputs(d, q_nope.shape[0], q_nope.device, with_lse)
    if split is None:
        gqla_decode_gqa(d, q_nope, q_rope, expanded_pages, block_table, cache_seqlens, out=out,
                        lse=lse, stream=stream)
    else:
        offs, total, tokens = split
        po, pl = _partials(d, total, q_nope.device)
        gqla_decode_gqa(d, q_nope, q_rope, expanded_pages, block_table, cache_seqlens, out=out,
                        lse=lse, split_offsets=offs, split_tokens=tokens, total_splits=total,
                        part_out=po, part_lse=pl, stream=stream)
    return out, lse


def expand_cache(d: Dims, latent_pages, w_uk, w_uv, page_ids=None, stream=None):
    """Allocate the expanded pool (same page count as the latent pool) and expand into it."""
    n = latent_pages.shape[0]
    E = torch.empty(n, d.block_size * (d.num_groups * (d.d_nope + d.d_v) + d.d_rope),
                    dtype=torch.bfloat16, device=latent_pages.device)
    gqla_expand_cache(d, latent_pages, w_uk, w_uv, E, page_ids=page_ids, stream=stream)
    return E


def gqla_select_path(d: Dims, seqlens_host, s_q_absorb: int, s_q_gqa: int, hw: Hw):
    """Roofline advisor: (chosen path, absorb estimate, GQA estimate) for one decode call of
    each path over sequences of the given (host) lengths."""
    lens = (ctypes.c_int32 * len(seqlens_host))(*[int(x) for x in seqlens_host])
    ea, eg = PathEstimate(), PathEstimate()
    st = lib().gqla_select_path(ctypes.byref(d), len(seqlens_host), lens, int(s_q_absorb),
                                int(s_q_gqa), ctypes.byref(hw), ctypes.byref(ea), ctypes.byref(eg))
    if st < 0:
        raise GqlaError(st, "gqla_select_path")
    return st, ea, eg


def gqla_append_tokens(d: Dims, new_rows, latent_pages, block_table, cache_seqlens, w_uk=None,
                       w_uv=None, expanded_pages=None, stream=None) -> None:
    """Write the new tokens' latent rows (bf16 [batch, n_new, r + d_R]) into their paged slots;
    with expanded_pages, also their K, V and rope slots of the expanded cache."""
    B, n_new = int(new_rows.shape[0]), int(new_rows.shape[1])
    row = d.d_latent + d.d_rope
    st = lib().gqla_append_tokens(
        ctypes.byref(d), B, n_new, _ptr(new_rows, torch.bfloat16, "new_rows", (B, n_new, row)),
        _ptr(latent_pages, torch.bfloat16, "latent_pages"), int(latent_pages.shape[0]),
        _ptr(block_table, torch.int32, "block_table"), int(block_table.shape[1]),
        _ptr(cache_seqlens, torch.int32, "cache_seqlens", (B,)),
        _ptr(w_uk, torch.bfloat16, "w_uk", allow_none=True),
        _ptr(w_uv, torch.bfloat16, "w_uv", allow_none=True),
        _ptr(expanded_pages, torch.bfloat16, "expanded_pages", allow_none=True), _stream(stream))
    _check(st, "gqla_append_tokens")
