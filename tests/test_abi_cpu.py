"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call (so these
calls are safe with fake device pointers)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest
import torch

import decode_attention_gqla_amd as G
from decode_attention_gqla_amd import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqla.h")
OK, INVALID, UNSUPPORTED, MISALIGNED, BADSPLIT = 0, -1, -2, -3, -4
A = ctypes.c_void_p(0x10000)     # fake, 16-byte aligned "device" pointers: never dereferenced
B_ = ctypes.c_void_p(0x20000)
ODD = ctypes.c_void_p(0x10002)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(G.LIB_PATH):
        from decode_attention_gqla_amd import build
        build.build()
    return G.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gqla_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) >= {"gqla_expand_cache", "gqla_decode_mqa_absorb", "gqla_decode_gqa",
                          "gqla_splitkv_combine", "gqla_status_string"}
    nm = subprocess.run(["nm", "-D", "--defined-only", G.LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (gqla_\w+)", nm.stdout))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def dsv3(s_q=1, **kw):
    d = Dims.make(128, 8, 512, 64, 128, 128, s_q)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def absorb(lib, d, batch=1, q=A, split=None, split_tokens=0, total=0, out=A, part=(None, None),
           ws=A, ws_bytes=1 << 40):
    # the absorb path has no partial buffers (it merges its splits itself)
    return lib.gqla_decode_mqa_absorb(ctypes.byref(d) if d is not None else None, batch, q, A, A,
                                      A, 4, A, A, A, split, split_tokens, total, out, None,
                                      ws, ws_bytes, None)


def gqa(lib, d, batch=1, q=A, split=None, split_tokens=0, total=0, out=A, part=(None, None)):
    return lib.gqla_decode_gqa(ctypes.byref(d) if d is not None else None, batch, q, A, A, A, 4,
                               A, split, split_tokens, total, out, None, part[0], part[1], None)


def test_version_and_status_strings(lib):
    assert lib.gqla_abi_version() >= 100
    for st in (OK, INVALID, UNSUPPORTED, MISALIGNED, BADSPLIT, -5, 7):
        assert isinstance(G.gqla_status_string(st), str)
    assert "MISALIGNED" in G.gqla_status_string(MISALIGNED)


def test_page_sizes(lib):
    d = dsv3()
    assert lib.gqla_latent_page_elems(ctypes.byref(d)) == 64 * 576
    assert lib.gqla_expanded_page_elems(ctypes.byref(d)) == 64 * 2112
    d4 = Dims.make(128, 4, 512, 64, 128, 128, 1)
    assert lib.gqla_expanded_page_elems(ctypes.byref(d4)) == 64 * 1088


@pytest.mark.parametrize("call", [absorb, gqa])
def test_decode_argument_errors_return_before_any_launch(lib, call):
    assert call(lib, None) == INVALID
    assert call(lib, dsv3(num_heads=127)) == INVALID                 # h_q % g != 0
    assert call(lib, dsv3(num_heads=96)) == UNSUPPORTED               # 12 heads per group
    assert call(lib, dsv3(block_size=32)) == UNSUPPORTED
    assert call(lib, dsv3(s_q=3)) == UNSUPPORTED
    assert call(lib, dsv3(d_rope=32)) == UNSUPPORTED
    assert call(lib, dsv3(softmax_scale=float("nan"))) == INVALID
    assert call(lib, dsv3(), batch=-1) == INVALID
    assert call(lib, dsv3(), q=None) == INVALID
    assert call(lib, dsv3(), q=ODD) == MISALIGNED
    assert call(lib, dsv3(), out=None) == INVALID                     # unsplit needs out
    assert call(lib, dsv3(), out=ODD) == MISALIGNED
    # split plans
    assert call(lib, dsv3(), split=A, split_tokens=100, total=4, part=(A, B_)) == BADSPLIT
    assert call(lib, dsv3(), split=A, split_tokens=0, total=4, part=(A, B_)) == BADSPLIT
    assert call(lib, dsv3(), batch=4, split=A, split_tokens=1024, total=2, part=(A, B_)) == BADSPLIT
    if call is gqa:   # the GQA split plan writes caller partials
        assert call(lib, dsv3(), split=A, split_tokens=1024, total=4, part=(None, B_)) == INVALID
        assert call(lib, dsv3(), split=A, split_tokens=1024, total=4, part=(ODD, B_)) == MISALIGNED
    else:             # the absorb path always writes out
        assert call(lib, dsv3(), split=A, split_tokens=1024, total=4, out=None) == INVALID
    # an empty batch is a valid no-op
    assert call(lib, dsv3(), batch=0) == OK
    assert call(lib, dsv3(), batch=0, split=A, split_tokens=1024, total=0, part=(A, B_)) == OK


def test_absorb_needs_weights_and_workspace(lib):
    d = dsv3()
    st = lib.gqla_decode_mqa_absorb(ctypes.byref(d), 1, A, A, A, A, 4, A, None, A, None, 0, 0, A,
                                    None, A, 1 << 40, None)
    assert st == INVALID
    up = lambda n: (n + 255) // 256 * 256
    rows = 1 * 128
    # q_abs rows, W_UV^T, split o_lat (bf16) and split lse (fp32); units = batch unsplit
    need = lib.gqla_mqa_absorb_workspace_bytes(ctypes.byref(d), 3, 0)
    assert need == up(3 * rows * 576 * 2) + up(8 * 128 * 512 * 2) + up(3 * rows * 512 * 2) + up(3 * rows * 4)
    need7 = lib.gqla_mqa_absorb_workspace_bytes(ctypes.byref(d), 3, 7)
    assert need7 == up(3 * rows * 576 * 2) + up(8 * 128 * 512 * 2) + up(7 * rows * 512 * 2) + up(7 * rows * 4)
    off = (ctypes.c_uint64 * 4)()
    assert lib.gqla_mqa_absorb_workspace_offsets(ctypes.byref(d), 3, 7, off) == OK
    assert list(off) == [0, up(3 * rows * 576 * 2), up(3 * rows * 576 * 2) + up(8 * 128 * 512 * 2),
                         up(3 * rows * 576 * 2) + up(8 * 128 * 512 * 2) + up(7 * rows * 512 * 2)]
    assert lib.gqla_mqa_absorb_workspace_offsets(ctypes.byref(d), 0, 7, off) == INVALID
    assert absorb(lib, d, batch=3, ws_bytes=need - 1) == INVALID
    assert absorb(lib, d, batch=3, ws=None, ws_bytes=need) == INVALID
    assert absorb(lib, d, batch=3, ws=ODD, ws_bytes=need) == MISALIGNED
    # a split plan needs room for its partials
    assert absorb(lib, d, batch=3, split=A, split_tokens=1024, total=7, ws_bytes=need7 - 1) == INVALID
    assert lib.gqla_mqa_absorb_workspace_bytes(None, 3, 0) == 0
    assert lib.gqla_mqa_absorb_workspace_bytes(ctypes.byref(d), 3, -1) == 0


def test_expand_and_combine_argument_errors(lib):
    d = dsv3()
    assert lib.gqla_expand_cache(ctypes.byref(d), A, A, A, 10, None, 0, A, None) == OK   # nothing to do
    assert lib.gqla_expand_cache(ctypes.byref(d), A, A, A, 10, None, 11, A, None) == INVALID
    assert lib.gqla_expand_cache(ctypes.byref(d), ODD, A, A, 10, None, 10, A, None) == MISALIGNED
    assert lib.gqla_expand_cache(ctypes.byref(d), None, A, A, 10, None, 10, A, None) == INVALID
    assert lib.gqla_expand_cache(None, A, A, A, 10, None, 10, A, None) == INVALID
    assert lib.gqla_splitkv_combine(ctypes.byref(d), 2, None, 4, A, A, A, None, None) == INVALID
    assert lib.gqla_splitkv_combine(ctypes.byref(d), 2, A, 4, ODD, A, A, None, None) == MISALIGNED
    assert lib.gqla_splitkv_combine(ctypes.byref(d), 0, A, 0, A, A, A, None, None) == OK
    assert lib.gqla_splitkv_combine(ctypes.byref(d), -1, A, 0, A, A, A, None, None) == INVALID


def test_append_argument_errors(lib):
    d = Dims.make(128, 8, 512, 64, 128, 128, 1)
    fn = lib.gqla_append_tokens
    # d, batch, n_new, rows, latent, num_pages, table, max_blocks, lens, w_uk, w_uv, expanded, stream
    # every call below fails its argument checks on the host, before any launch
    assert fn(ctypes.byref(d), 0, 1, A, A, 8, A, 4, A, None, None, None, None) == INVALID
    assert fn(ctypes.byref(d), 2, 0, A, A, 8, A, 4, A, None, None, None, None) == INVALID
    assert fn(ctypes.byref(d), 2, 65, A, A, 8, A, 4, A, None, None, None, None) == INVALID
    assert fn(ctypes.byref(d), 2, 1, A, A, 0, A, 4, A, None, None, None, None) == INVALID
    assert fn(ctypes.byref(d), 2, 1, None, A, 8, A, 4, A, None, None, None, None) == INVALID
    assert fn(ctypes.byref(d), 2, 1, A, A, 8, A, 4, A, None, None, A, None) == INVALID   # weights needed
    assert fn(ctypes.byref(d), 2, 1, A, A, 8, A, 4, A, A, ODD, A, None) == MISALIGNED
    assert fn(ctypes.byref(d), 2, 1, ODD, A, 8, A, 4, A, None, None, None, None) == MISALIGNED
    assert fn(None, 2, 1, A, A, 8, A, 4, A, None, None, None, None) == INVALID
    assert fn(ctypes.byref(Dims.make(96, 8, 512, 64, 128, 128, 1)), 2, 1, A, A, 8, A, 4, A,
              None, None, None, None) == UNSUPPORTED


def test_sparse_argument_errors(lib):
    d = Dims.make(128, 8, 512, 64, 128, 128, 2)
    fn = lib.gqla_decode_gqa_sparse
    need = 2 * 8 * 64 * 4                  # batch 2, 8 groups, 40 entries padded to 64, 4 bytes
    assert lib.gqla_sparse_workspace_bytes(ctypes.byref(d), 2, 40, 0) == need
    assert lib.gqla_sparse_workspace_bytes(ctypes.byref(d), 0, 40, 0) == 0
    assert lib.gqla_sparse_workspace_bytes(ctypes.byref(d), 2, 0, 0) == 0
    assert lib.gqla_sparse_workspace_bytes(ctypes.byref(d), 2, 40, -32) == 0
    assert lib.gqla_sparse_workspace_bytes(None, 2, 40, 0) == 0
    # with a split of 32 entries: 2 ranges per list; plan, partials and their lse follow the codes
    off = G.gqla_sparse_workspace_offsets(d, 2, 40, 32)
    units, rows = 2 * 2, 2 * 2 * 2 * 128
    assert off[0] == 0 and off[1] == need and off[1] % 256 == 0
    assert off[2] == off[1] + 256 and off[3] == off[2] + rows * 128 * 4
    assert off[4] == off[3] + rows * 4 and rows == units * 2 * 128
    assert lib.gqla_sparse_workspace_bytes(ctypes.byref(d), 2, 40, 32) == off[4]

    def call(dd=d, batch=2, qn=A, pages=A, num_pages=8, idx=A, topk=40, split=0, out=A, ws=A,
             ws_bytes=need):
        # d, batch, q_nope, q_rope, expanded, num_pages, table, max_blocks, lens, indices, topk,
        # split_entries, out, lse, workspace, workspace_bytes, stream
        return fn(dd, batch, qn, A, pages, num_pages, A, 4, A, idx, topk, split, out, None, ws,
                  ws_bytes, None)
    # every call below fails its argument checks on the host, before any launch
    assert call(topk=0) == INVALID
    assert call(idx=None) == INVALID
    assert call(num_pages=0) == INVALID
    assert call(num_pages=(1 << 28) // 64 + 1) == INVALID        # rows must fit 28 bits
    assert call(ws=None) == INVALID
    assert call(ws_bytes=need - 1) == INVALID
    assert call(split=32, ws_bytes=need) == INVALID              # a split needs the larger workspace
    assert call(split=33) == BADSPLIT
    assert call(split=-32) == BADSPLIT
    assert call(out=None) == INVALID
    assert call(qn=None) == INVALID
    assert call(dd=None) == INVALID
    assert call(idx=ODD) == MISALIGNED
    assert call(ws=ODD) == MISALIGNED
    assert call(pages=ODD) == MISALIGNED
    assert call(dd=ctypes.byref(Dims.make(96, 8, 512, 64, 128, 128, 2))) == UNSUPPORTED
    assert call(batch=-1) == INVALID
    assert call(batch=0) == OK                                   # nothing to do, nothing enqueued


def test_binding_rejects_cpu_tensors_and_wrong_dtypes(lib):
    d = Dims.make(16, 2, 64, 16, 32, 32, 1)
    q = torch.zeros(1, 1, 16, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        G.gqla_decode_gqa(d, q, q, q, torch.zeros(1, 1, dtype=torch.int32),
                          torch.zeros(1, dtype=torch.int32), out=q)


def test_split_plan_counts_ceil_per_sequence():
    offs, total = G.make_split_plan([1, 1024, 1025, 4096], 1024, device="cpu")
    assert offs.tolist() == [0, 1, 2, 4, 8] and total == 8


def merge(lib, d, batch=1, part=A, plse=A, split=None, total=0, wuv=A, out=A, lse=None, ws=A, ws_bytes=1 << 40):
    return lib.gqla_mqa_absorb_merge(ctypes.byref(d) if d is not None else None, batch, part, plse, split, total,
                                     wuv, out, lse, ws, ws_bytes, None)


def test_absorb_merge_rejects_bad_arguments_on_the_host(lib):
    d = dsv3()
    need = lib.gqla_mqa_absorb_merge_workspace_bytes(ctypes.byref(d))
    assert need == 8 * 128 * 512 * 2                  # W_UV transposed, bf16
    assert lib.gqla_mqa_absorb_merge_workspace_bytes(None) == 0
    assert merge(lib, None) == INVALID
    assert merge(lib, d, batch=-1) == INVALID
    for kw in (dict(part=None), dict(plse=None), dict(wuv=None), dict(out=None), dict(ws=None)):
        assert merge(lib, d, **kw) == INVALID, kw
    for kw in (dict(part=ODD), dict(wuv=ODD), dict(out=ODD), dict(ws=ODD),
               dict(plse=ctypes.c_void_p(0x10002)), dict(lse=ctypes.c_void_p(0x10002)),
               dict(split=ctypes.c_void_p(0x10002), total=4)):
        assert merge(lib, d, **kw) == MISALIGNED, kw
    assert merge(lib, d, batch=3, split=A, total=2) == BADSPLIT
    assert merge(lib, d, ws_bytes=need - 1) == INVALID
    bad = dsv3(d_v=96)
    assert merge(lib, bad) == UNSUPPORTED
    assert merge(lib, d, batch=0) == OK               # nothing to do, nothing enqueued


def test_noalloc_absorb_checks_arguments_and_its_scratch_limit_on_the_host(lib):
    d = dsv3()
    call = lambda **kw: lib.gqla_decode_mqa_absorb_noalloc(
        ctypes.byref(d), kw.get("batch", 1), kw.get("q", A), A, A, A, 4, A, kw.get("wuk", A), A,
        kw.get("split", None), kw.get("split_tokens", 0), kw.get("total", 0), kw.get("out", A), None, None)
    assert call(q=None) == INVALID
    assert call(wuk=None) == INVALID
    assert call(q=ODD) == MISALIGNED
    assert call(split=A, split_tokens=1000, total=4) == BADSPLIT
    assert call(batch=0) == OK
    # 64 x 4096 tokens in 64-token splits: the workspace exceeds the fixed 32 MiB scratch,
    # rejected before any HIP call
    assert call(batch=64, split=A, split_tokens=64, total=64 * 64) == -6
    assert b"SCRATCH_LIMIT" in lib.gqla_status_string(-6)
