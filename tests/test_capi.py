"""The C-ABI library: it loads without a GPU, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call.
CPU only -- no compute call is made."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import q4_swiglu_mlp_amd as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000          # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10004        # misaligned by 4


def _declared():
    text = open(os.path.join(ROOT, "include", "zinc_mlp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zinc_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(Z.EXPORTS)
    for n in names:
        assert hasattr(Z.lib, n), n
    # and they are real dynamic symbols of the shared object
    so = ctypes.CDLL(Z.LIB_PATH)
    for n in names:
        assert ctypes.cast(getattr(so, n), ctypes.c_void_p).value


def test_strerror_covers_every_status():
    for st in range(-7, 1):
        assert Z.strerror(st) and "unknown" not in Z.strerror(st)
    assert "unknown" in Z.strerror(-99)


def prefill(**kw):
    args = dict(wg=A, wu=A, wd=A, hidden=4096, inter=11008, x=A, y=A, M=256, a=0, b=0, ws=A, wsb=1 << 30)
    args.update(kw)
    return Z.lib.zinc_mlp_q4k_prefill(args["wg"], args["wu"], args["wd"], args["hidden"], args["inter"], args["x"],
                                      args["y"], args["M"], args["a"], args["b"], args["ws"], args["wsb"], None)


def decode(**kw):
    args = dict(wg=A, wu=A, wd=A, hidden=4096, inter=11008, x=A, y=A, M=4, a=0, b=0, ws=A, wsb=1 << 30)
    args.update(kw)
    return Z.lib.zinc_mlp_q4k_decode(args["wg"], args["wu"], args["wd"], args["hidden"], args["inter"], args["x"],
                                     args["y"], args["M"], args["a"], args["b"], args["ws"], args["wsb"], None)


def prefill_staged(**kw):
    args = dict(wg=A, wu=A, wd=A, hidden=4096, inter=11008, x=A, y=A, M=256, a=0, b=0, ws=A, wsb=1 << 31)
    args.update(kw)
    return Z.lib.zinc_mlp_q4k_prefill_staged(args["wg"], args["wu"], args["wd"], args["hidden"], args["inter"],
                                             args["x"], args["y"], args["M"], args["a"], args["b"], args["ws"],
                                             args["wsb"], None)


@pytest.mark.parametrize("fn", [prefill, prefill_staged, decode])
def test_dense_argument_errors(fn):
    assert fn(wg=None) == -1 and fn(wd=None) == -1 and fn(x=None) == -1 and fn(y=None) == -1
    assert fn(hidden=0) == -2 and fn(hidden=300) == -2 and fn(inter=-256) == -2 and fn(inter=1000) == -2
    assert fn(hidden=16384 + 256) == -2
    assert fn(wg=MIS) == -3 and fn(x=MIS) == -3 and fn(y=MIS) == -3
    assert fn(M=-1) == -5
    assert fn(a=-1) == -5 and fn(a=31) == -5 and fn(b=31) == -5
    assert fn(ws=None) == -1
    assert fn(ws=MIS) == -3
    assert fn(wsb=16) == -4
    # M == 0: a no-op that succeeds without touching the GPU or the workspace
    assert fn(M=0, ws=None, wsb=0) == 0


def test_prefill_addressing_limits():
    # the staged activation, (M+1) x hidden/256 x 544 B, is addressed with
    # 32-bit offsets: at hidden 16384 M = 123360 fits, M = 123361 does not
    assert (123360 + 1) * 64 * 544 <= 0xFFFFFFFF < (123361 + 1) * 64 * 544
    assert prefill(hidden=16384, M=123361) == -5
    assert Z.prefill_workspace_size(123361, 16384, 11008) == 0
    assert Z.prefill_workspace_size(123360, 16384, 256) > 0
    assert prefill(M=(1 << 20) + 1) == -5
    assert Z.prefill_workspace_size((1 << 20) + 1, 256, 256) == 0


def test_decode_token_limit():
    assert decode(M=9) == -5
    assert Z.decode_workspace_size(9, 4096, 11008) == 0


def test_workspace_sizes():
    assert Z.prefill_workspace_size(256, 4096, 11008) >= 256 * 4096 * 4
    assert Z.prefill_workspace_size(257, 4096, 11008) >= Z.prefill_workspace_size(256, 4096, 11008)
    assert Z.prefill_workspace_size(256, 4000, 11008) == 0
    # the staged baseline adds G, U and the intermediate, M x inter fp16 each
    assert (Z.prefill_staged_workspace_size(256, 4096, 11008)
            >= Z.prefill_workspace_size(256, 4096, 11008) + 3 * 256 * 11008 * 2)
    assert Z.prefill_staged_workspace_size(256, 4000, 11008) == 0


@pytest.mark.parametrize("size", ["prefill_workspace_size", "prefill_staged_workspace_size"])
def test_prefill_workspace_size_monotone(size):
    # a workspace sized for M serves every smaller M, although the chunk count
    # of the plan drops as token tiles are added (e.g. 256 -> 257 tokens)
    f = getattr(Z, size)
    ms = sorted(set(list(range(1, 1200, 13)) + [64 * t + d for t in range(1, 40) for d in (-1, 0, 1)] + [2048, 4096]))
    sizes = [f(m, 4096, 11008) for m in ms]
    assert all(s > 0 for s in sizes)
    assert all(b >= a for a, b in zip(sizes, sizes[1:]))
    assert Z.decode_workspace_size(4, 4096, 11008) >= 4 * 11008 * 2
    assert Z.moe_workspace_size(512, 8, 64, 2048, 768) >= 512 * 2048 * 4 + 512 * 8 * 4
    assert Z.moe_workspace_size(512, 65, 64, 2048, 768) == 0


def moe(**kw):
    args = dict(wg=A, wu=A, wd=A, E=64, hidden=2048, inter=768, x=A, M=512, ids=A, p=A, k=8, y=A, a=0, b=0, ws=A,
                wsb=1 << 30, err=None)
    args.update(kw)
    return Z.lib.zinc_moe_q4k_experts(args["wg"], args["wu"], args["wd"], args["E"], args["hidden"], args["inter"],
                                      args["x"], args["M"], args["ids"], args["p"], args["k"], args["y"], args["a"],
                                      args["b"], args["ws"], args["wsb"], args["err"], None)


def test_moe_argument_errors():
    assert moe(ids=None) == -1 and moe(p=None) == -1 and moe(wu=None) == -1
    assert moe(hidden=100) == -2
    assert moe(ids=A + 2) == -3 and moe(err=A + 1) == -3 and moe(x=MIS) == -3
    assert moe(k=0) == -5 and moe(k=65) == -5 and moe(E=0) == -5 and moe(E=1025, k=8) == -5
    assert moe(M=-3) == -5 and moe(M=(1 << 24) // 8 + 1) == -5
    # a chunk's partial rows, (M*k + 1) x hidden fp16, use 32-bit offsets
    assert moe(M=65536, k=2, hidden=16384) == -5
    assert Z.moe_workspace_size(65536, 2, 64, 16384, 768) == 0
    assert moe(ws=None) == -1 and moe(wsb=100) == -4
    assert moe(M=0, ws=None, wsb=0) == 0


def test_dequant_argument_errors():
    f = Z.lib.zinc_q4k_dequant_f32
    assert f(None, 4, 256, A, None) == -1
    assert f(A, 4, 255, A, None) == -2
    assert f(A, -1, 256, A, None) == -5
    assert f(MIS, 4, 256, A, None) == -3
    assert f(A, 1 << 20, 1 << 12, A, None) == -2     # rows*cols beyond int32
    assert f(A, 0, 256, A, None) == 0


def route(**kw):
    args = dict(logits=A, M=16, E=64, k=8, ids=A, p=A)
    args.update(kw)
    return Z.lib.zinc_moe_route_topk(args["logits"], args["M"], args["E"], args["k"], args["ids"], args["p"], None)


def test_router_argument_errors():
    assert route(logits=None) == -1 and route(ids=None) == -1 and route(p=None) == -1
    assert route(logits=A + 2) == -3 and route(ids=A + 1) == -3 and route(p=A + 3) == -3
    assert route(k=0) == -5 and route(k=65) == -5 and route(E=8, k=9) == -5
    assert route(E=0, k=1) == -5 and route(E=1025, k=8) == -5
    assert route(M=-1) == -5 and route(M=(1 << 24) // 8 + 1) == -5
    # no tokens: nothing is read, so empty (NULL) buffers are accepted
    assert route(M=0) == 0 and route(M=0, logits=None, ids=None, p=None) == 0
    assert route(M=0, k=0) == -5


def block(fn_name, **kw):
    args = dict(wg=A, wu=A, wd=A, hidden=4096, inter=11008, x=A, g=A, eps=1e-5, s=1.0, y=A, M=4, a=0, b=0, ws=A,
                wsb=1 << 31)
    args.update(kw)
    return getattr(Z.lib, fn_name)(args["wg"], args["wu"], args["wd"], args["hidden"], args["inter"], args["x"],
                                   args["g"], args["eps"], args["s"], args["y"], args["M"], args["a"], args["b"],
                                   args["ws"], args["wsb"], None)


@pytest.mark.parametrize("fn_name", ["zinc_mlp_q4k_prefill_block", "zinc_mlp_q4k_decode_block"])
def test_block_argument_errors(fn_name):
    f = lambda **kw: block(fn_name, **kw)
    assert f(g=None) == -1 and f(x=None) == -1 and f(wd=None) == -1
    assert f(g=A + 2) == -3 and f(x=MIS) == -3
    assert f(eps=-1e-6) == -5 and f(eps=float("nan")) == -5 and f(eps=float("inf")) == -5
    assert f(s=float("nan")) == -5 and f(s=float("inf")) == -5
    assert f(hidden=300) == -2 and f(M=-1) == -5
    assert f(ws=None) == -1 and f(wsb=16) == -4
    assert f(M=0, ws=None, wsb=0) == 0
    assert f(eps=0.0, M=0) == 0 and f(s=0.0, M=0) == 0


def test_block_workspace_sizes():
    for M in (1, 4):
        assert Z.lib.zinc_mlp_q4k_decode_block_workspace_size(M, 4096, 11008) >= \
            Z.decode_workspace_size(M, 4096, 11008) + M * 4096 * 2
    assert Z.lib.zinc_mlp_q4k_prefill_block_workspace_size(256, 4096, 11008) >= \
        Z.prefill_workspace_size(256, 4096, 11008) + 256 * 4096 * 2
    assert Z.lib.zinc_mlp_q4k_decode_block_workspace_size(9, 4096, 11008) == 0
    assert Z.lib.zinc_mlp_q4k_prefill_block_workspace_size(256, 4000, 11008) == 0
    assert block("zinc_mlp_q4k_decode_block", M=9) == -5


def test_moe_down_format_errors():
    f = Z.lib.zinc_moe_experts_fmt
    call = lambda fmt, **kw: f(A, A, A, fmt, 64, 2048, 768, A, kw.get("M", 512), A, A, 8, A, 0, 0, A, 1 << 30, None,
                               None)
    assert call(3) == -5 and call(-1) == -5
    assert call(1, M=0) == 0 and call(2, M=0) == 0
    g = Z.lib.zinc_q5_1_dequant_f32
    assert g(A, 4, 48, A, None) == -2          # Q5_1 rows are whole 32-weight blocks
    assert g(None, 4, 64, A, None) == -1 and g(A, -1, 64, A, None) == -5 and g(A, 0, 64, A, None) == 0
    assert Z.lib.zinc_q5k_dequant_f32(A, 4, 288, A, None) == -2
