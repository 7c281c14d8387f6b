"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function ``include/diffattn.h`` declares,
and reject bad arguments before anything is launched.  The calls below pass
fake, never-dereferenced device addresses and always fail validation, so no
kernel is launched and no device is touched.
"""
import ctypes
import math
import os
import re

import pytest

import oracle
from differential_softmax_attention_diffattn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "diffattn.h")

E_INVALID, E_UNSUPPORTED, E_ALIGN, E_WORKSPACE = -1, -2, -3, -4
F32, BF16 = 0, 1
P = 0x10000  # a 16-byte aligned fake address; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail(f"{_lib.LIB_PATH} not built (run python -m differential_softmax_attention_diffattn_amd.build)")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"DIFFATTN_API\s+[\w\s\*]+?\b(diffattn_\w+)\s*\(", text)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"diffattn_v1_fwd", "diffattn_v2_fwd", "diffattn_v2_decode"} <= names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks a signature for {name}"


def test_version_and_lambda_init(lib):
    assert lib.diffattn_version() >= 100
    for layer in (1, 2, 3, 10, 28):
        assert abs(lib.diffattn_lambda_init(layer) - oracle.lambda_init(layer)) < 2e-7
    assert math.isnan(lib.diffattn_lambda_init(0))
    assert b"layer" in lib.diffattn_last_error()


def v1(lib, **kw):
    a = dict(q1=P, k1=P, q2=P, k2=P, v=P, w=None, out=P, B=1, T=16, H=1, d=128, dv=256, lam=0.2,
             li=0.2, eps=1e-12, causal=1, dt=BF16, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.diffattn_v1_fwd(a["q1"], a["k1"], a["q2"], a["k2"], a["v"], a["w"], a["out"], a["B"],
                               a["T"], a["H"], a["d"], a["dv"], a["lam"], a["li"], a["eps"],
                               a["causal"], a["dt"], a["ws"], a["wsb"], a["stream"])


def test_v1_rejects_bad_arguments(lib):
    assert v1(lib, q1=None) == E_INVALID
    assert v1(lib, T=-1) == E_INVALID
    assert v1(lib, d=0) == E_INVALID
    assert v1(lib, causal=2) == E_INVALID
    assert v1(lib, lam=float("nan")) == E_INVALID
    assert v1(lib, eps=-1.0) == E_INVALID
    assert v1(lib, dt=7) == E_INVALID
    assert v1(lib, d=96, dv=192) == E_UNSUPPORTED  # bf16 fast path needs (128,256) or (64,128)
    assert v1(lib, dt=F32, d=136, dv=272) == E_UNSUPPORTED
    assert v1(lib, q1=P + 8) == E_ALIGN
    assert v1(lib, w=P + 2) == E_ALIGN
    assert v1(lib, ws=None) == E_WORKSPACE
    assert v1(lib, wsb=16) == E_WORKSPACE
    assert b"workspace" in lib.diffattn_last_error()


def test_v1_empty_problem_is_a_no_op(lib):
    assert v1(lib, T=0, ws=None, wsb=0) == 0
    assert v1(lib, B=0, ws=None, wsb=0) == 0


def test_v1_workspace_query(lib):
    assert lib.diffattn_v1_workspace_bytes(4, 4096, 12, 128, 256, F32) == 0
    need = lib.diffattn_v1_workspace_bytes(4, 4096, 12, 128, 256, BF16)
    # one fp16 block [256 rows][64 keys] per (batch, head, 64-key tile)
    assert need == 4 * 12 * 64 * 256 * 64 * 2
    assert lib.diffattn_v1_workspace_bytes(4, 4096, 12, 96, 192, BF16) == 0


def v2(lib, **kw):
    a = dict(q=P, k=P, v=P, lg=P, out=P, cu=None, nseq=0, maxlen=0, B=2, T=64, Hq=16, Hkv=2, d=128,
             scale=0.0, causal=1, dt=BF16, stream=None)
    a.update(kw)
    return lib.diffattn_v2_fwd(a["q"], a["k"], a["v"], a["lg"], a["out"], a["cu"], a["nseq"],
                               a["maxlen"], a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["scale"],
                               a["causal"], a["dt"], a["stream"])


def test_v2_rejects_bad_arguments(lib):
    assert v2(lib, out=None) == E_INVALID
    assert v2(lib, Hq=15, Hkv=3) == E_INVALID       # odd number of query heads
    assert v2(lib, Hq=16, Hkv=3) == E_INVALID       # not a multiple
    assert v2(lib, Hq=6, Hkv=2) == E_INVALID        # group of 3: a pair would straddle groups
    assert b"pair" in lib.diffattn_last_error()
    assert v2(lib, d=96) == E_UNSUPPORTED
    assert v2(lib, dt=F32) == E_UNSUPPORTED
    assert v2(lib, scale=float("inf")) == E_INVALID
    assert v2(lib, B=-1) == E_INVALID
    assert v2(lib, cu=P, nseq=-1, maxlen=5) == E_INVALID
    assert v2(lib, k=P + 4) == E_ALIGN
    assert v2(lib, cu=P + 2, nseq=2, maxlen=8) == E_ALIGN


def test_v2_empty_problem_is_a_no_op(lib):
    assert v2(lib, B=0) == 0
    assert v2(lib, T=0) == 0
    assert v2(lib, cu=P, nseq=0, maxlen=0) == 0


def dec(lib, **kw):
    a = dict(q=P, k=P, v=P, lens=None, lg=P, out=P, ws=P, wsb=1 << 30, B=4, S=1024, Hq=16, Hkv=2,
             d=128, scale=0.0, dt=BF16, stream=None)
    a.update(kw)
    return lib.diffattn_v2_decode(a["q"], a["k"], a["v"], a["lens"], a["lg"], a["out"], a["ws"],
                                  a["wsb"], a["B"], a["S"], a["Hq"], a["Hkv"], a["d"], a["scale"],
                                  a["dt"], a["stream"])


def test_decode_rejects_bad_arguments(lib):
    assert dec(lib, q=None) == E_INVALID
    assert dec(lib, Hq=6, Hkv=2) == E_INVALID
    assert dec(lib, Hq=64, Hkv=2) == E_UNSUPPORTED  # 32 query heads per KV head
    assert dec(lib, d=80) == E_UNSUPPORTED
    assert dec(lib, ws=None) == E_WORKSPACE
    assert dec(lib, wsb=8) == E_WORKSPACE
    assert dec(lib, lens=P + 1) == E_ALIGN
    assert dec(lib, B=0) == 0


def test_decode_workspace_query(lib):
    n = lib.diffattn_v2_decode_workspace_bytes(64, 32768, 64, 8, 128)
    # fp32 partial records of d + 4 floats per (batch, query head, part)
    assert n > 0 and n % (4 * 132 * 64 * 64) == 0
    nparts = n // (4 * 132 * 64 * 64)
    assert 1 <= nparts <= 512
    assert lib.diffattn_v2_decode_workspace_bytes(64, 32768, 64, 3, 128) == 0


def v2t(lib, **kw):
    a = dict(q=P, k=P, v=P, lg=P, out=P, oh=P, lse=P, B=2, T=64, Hq=16, Hkv=2, d=128, scale=0.0,
             causal=1, dt=BF16, stream=None)
    a.update(kw)
    return lib.diffattn_v2_fwd_train(a["q"], a["k"], a["v"], a["lg"], a["out"], a["oh"], a["lse"],
                                     a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["scale"],
                                     a["causal"], a["dt"], a["stream"])


def test_v2_train_forward_rejects_bad_arguments(lib):
    assert v2t(lib, oh=None) == E_INVALID
    assert v2t(lib, lse=None) == E_INVALID
    assert v2t(lib, Hq=6, Hkv=2) == E_INVALID
    assert v2t(lib, d=96) == E_UNSUPPORTED
    assert v2t(lib, T=-3) == E_INVALID
    assert v2t(lib, oh=P + 8) == E_ALIGN
    assert v2t(lib, lse=P + 2) == E_ALIGN
    assert v2t(lib, B=0) == 0


def bwd(lib, **kw):
    a = dict(q=P, k=P, v=P, lg=P, oh=P, lse=P, dout=P, dq=P, dk=P, dv=P, dlg=P, ws=P, wsb=1 << 30,
             B=2, T=64, Hq=16, Hkv=2, d=128, scale=0.0, causal=1, dt=BF16, stream=None)
    a.update(kw)
    return lib.diffattn_v2_bwd(a["q"], a["k"], a["v"], a["lg"], a["oh"], a["lse"], a["dout"],
                               a["dq"], a["dk"], a["dv"], a["dlg"], a["ws"], a["wsb"], a["B"],
                               a["T"], a["Hq"], a["Hkv"], a["d"], a["scale"], a["causal"],
                               a["dt"], a["stream"])


def test_v2_backward_rejects_bad_arguments(lib):
    assert bwd(lib, dout=None) == E_INVALID
    assert bwd(lib, dlg=None) == E_INVALID
    assert bwd(lib, Hq=16, Hkv=3) == E_INVALID
    assert bwd(lib, Hq=6, Hkv=2) == E_INVALID
    assert bwd(lib, causal=3) == E_INVALID
    assert bwd(lib, d=80) == E_UNSUPPORTED
    assert bwd(lib, dt=F32) == E_UNSUPPORTED
    assert bwd(lib, dq=P + 4) == E_ALIGN
    assert bwd(lib, dlg=P + 1) == E_ALIGN
    assert bwd(lib, ws=None) == E_WORKSPACE
    assert bwd(lib, wsb=64) == E_WORKSPACE
    assert b"workspace" in lib.diffattn_last_error()
    assert bwd(lib, T=0, ws=None, wsb=0) == 0


def test_v2_backward_workspace_query(lib):
    # fp32 delta and log2-lse values [B][Hq][T rounded up to 64]
    assert lib.diffattn_v2_bwd_workspace_bytes(2, 8192, 64, 8, 128) == 4 * 2 * 8192 * 64 * 2
    assert lib.diffattn_v2_bwd_workspace_bytes(1, 65, 16, 2, 128) == 4 * 128 * 16 * 2
    assert lib.diffattn_v2_bwd_workspace_bytes(1, 64, 6, 2, 128) == 0
    assert lib.diffattn_v2_bwd_workspace_bytes(1, 64, 16, 2, 96) == 0


def v1t(lib, **kw):
    a = dict(q1=P, k1=P, q2=P, k2=P, v=P, w=None, out=P, o1=P, o2=P, lse=P, B=1, T=16, H=1, d=128,
             dv=256, lam=0.2, li=0.2, eps=1e-12, causal=1, dt=BF16, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.diffattn_v1_fwd_train(a["q1"], a["k1"], a["q2"], a["k2"], a["v"], a["w"], a["out"],
                                     a["o1"], a["o2"], a["lse"], a["B"], a["T"], a["H"], a["d"],
                                     a["dv"], a["lam"], a["li"], a["eps"], a["causal"], a["dt"],
                                     a["ws"], a["wsb"], a["stream"])


def test_v1_train_forward_rejects_bad_arguments(lib):
    assert v1t(lib, o1=None) == E_INVALID
    assert v1t(lib, lse=None) == E_INVALID
    assert v1t(lib, dt=F32) == E_UNSUPPORTED
    assert v1t(lib, d=96, dv=192) == E_UNSUPPORTED
    assert v1t(lib, o2=P + 8) == E_ALIGN
    assert v1t(lib, ws=None) == E_WORKSPACE
    assert v1t(lib, T=0, ws=None, wsb=0) == 0


def v1b(lib, **kw):
    a = dict(q1=P, k1=P, q2=P, k2=P, v=P, w=None, o1=P, o2=P, lse=P, dy=P, dq1=P, dk1=P, dq2=P,
             dk2=P, dv=P, dlam=P, dw=P, B=1, T=16, H=1, d=128, dvd=256, lam=0.2, li=0.2,
             eps=1e-12, causal=1, dt=BF16, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.diffattn_v1_bwd(a["q1"], a["k1"], a["q2"], a["k2"], a["v"], a["w"], a["o1"],
                               a["o2"], a["lse"], a["dy"], a["dq1"], a["dk1"], a["dq2"], a["dk2"],
                               a["dv"], a["dlam"], a["dw"], a["B"], a["T"], a["H"], a["d"],
                               a["dvd"], a["lam"], a["li"], a["eps"], a["causal"], a["dt"],
                               a["ws"], a["wsb"], a["stream"])


def test_v1_backward_rejects_bad_arguments(lib):
    assert v1b(lib, dy=None) == E_INVALID
    assert v1b(lib, dk2=None) == E_INVALID
    assert v1b(lib, lse=None) == E_INVALID
    assert v1b(lib, dlam=None, T=0) == E_INVALID  # dlambda is written even with no rows
    assert v1b(lib, dw=None) == E_INVALID
    assert v1b(lib, causal=2) == E_INVALID
    assert v1b(lib, lam=float("inf")) == E_INVALID
    assert v1b(lib, eps=-1.0) == E_INVALID
    assert v1b(lib, dt=F32) == E_UNSUPPORTED
    assert v1b(lib, d=96, dvd=192) == E_UNSUPPORTED
    assert v1b(lib, dq1=P + 4) == E_ALIGN
    assert v1b(lib, dlam=P + 1) == E_ALIGN
    assert v1b(lib, w=P + 2) == E_ALIGN
    assert v1b(lib, ws=None) == E_WORKSPACE
    assert v1b(lib, wsb=64) == E_WORKSPACE
    assert b"workspace" in lib.diffattn_last_error()


def test_v1_backward_workspace_query(lib):
    # bf16 dz [B,T,H,dv], fp32 stats [B][H][4][T rounded up to 64], then the
    # preprocessing grid's partial sums (at most 1024 blocks of dv + 4 floats)
    assert lib.diffattn_v1_bwd_workspace_bytes(4, 4096, 12, 128, 256) == (
        4 * 4096 * 12 * 256 * 2 + 4 * 12 * 4 * 4096 * 4 + 1024 * 260 * 4)
    assert lib.diffattn_v1_bwd_workspace_bytes(1, 1, 1, 64, 128) == (
        256 + 4 * 64 * 4 + 4 * 132 * 4)  # 16 rows per workgroup: 4 for the 64 padded rows
    assert lib.diffattn_v1_bwd_workspace_bytes(1, 64, 1, 96, 192) == 0
    assert lib.diffattn_v1_bwd_workspace_bytes(0, 64, 1, 128, 256) == 0


def test_lambda_proj_rejects_bad_arguments(lib):
    f = lambda x=P, w=P, o=P, N=64, dm=4096, h=32, dt=BF16: lib.diffattn_v2_lambda_proj(
        x, w, o, N, dm, h, dt, None)
    assert f(N=-1) == E_INVALID
    assert f(h=0) == E_INVALID
    assert f(dt=F32) == E_UNSUPPORTED
    assert f(dt=5) == E_INVALID
    assert f(h=24) == E_UNSUPPORTED
    assert f(h=80) == E_UNSUPPORTED
    assert f(dm=4000) == E_UNSUPPORTED
    assert f(x=None) == E_INVALID
    assert f(w=P + 8) == E_ALIGN
    assert f(o=P + 2) == E_ALIGN
    assert f(N=0, x=None, w=None, o=None) == 0


def test_out_proj_rejects_bad_arguments(lib):
    f = lambda a=P, w=P, y=P, M=64, K=4096, N=4096, dt=BF16: lib.diffattn_out_proj(
        a, w, y, M, K, N, dt, None)
    assert f(M=-1) == E_INVALID
    assert f(K=0) == E_INVALID
    assert f(dt=F32) == E_UNSUPPORTED
    assert f(K=100) == E_UNSUPPORTED
    assert f(N=6) == E_UNSUPPORTED
    assert f(K=1 << 25) == E_INVALID
    assert f(y=None) == E_INVALID
    assert f(a=P + 8) == E_ALIGN
    assert f(M=0, a=None, w=None, y=None) == 0


def vbwd(lib, **kw):
    a = dict(q=P, k=P, v=P, lg=P, cu=P, nseq=2, oh=P, lse=P, dout=P, dq=P, dk=P, dv=P, dlg=P, ws=P,
             wsb=1 << 30, N=100, Hq=16, Hkv=2, d=128, scale=0.0, causal=1, dt=BF16, stream=None)
    a.update(kw)
    return lib.diffattn_v2_varlen_bwd(a["q"], a["k"], a["v"], a["lg"], a["cu"], a["nseq"], a["oh"],
                                      a["lse"], a["dout"], a["dq"], a["dk"], a["dv"], a["dlg"],
                                      a["ws"], a["wsb"], a["N"], a["Hq"], a["Hkv"], a["d"],
                                      a["scale"], a["causal"], a["dt"], a["stream"])


def test_v2_varlen_backward_rejects_bad_arguments(lib):
    assert vbwd(lib, cu=None) == E_INVALID
    assert vbwd(lib, dq=None) == E_INVALID
    assert vbwd(lib, N=-1) == E_INVALID
    assert vbwd(lib, Hq=6, Hkv=2) == E_INVALID
    assert vbwd(lib, d=96) == E_UNSUPPORTED
    assert vbwd(lib, cu=P + 2) == E_ALIGN
    assert vbwd(lib, dk=P + 4) == E_ALIGN
    assert vbwd(lib, ws=None) == E_WORKSPACE
    assert vbwd(lib, wsb=128) == E_WORKSPACE
    assert vbwd(lib, N=0) == 0
    assert vbwd(lib, nseq=0) == 0


def test_v2_varlen_backward_workspace_query(lib):
    # per-row values of every sequence padded to 64 rows: rows <= N rounded up + 64 per sequence
    Np = (65536 + 63) // 64 * 64 + 64 * 8
    assert lib.diffattn_v2_varlen_bwd_workspace_bytes(65536, 8, 64, 8, 128) == 4 * Np * 64 * 2
    assert lib.diffattn_v2_varlen_bwd_workspace_bytes(100, 3, 16, 2, 128) == 4 * (128 + 192) * 16 * 2
    assert lib.diffattn_v2_varlen_bwd_workspace_bytes(100, 3, 16, 2, 96) == 0
    assert lib.diffattn_v2_varlen_bwd_workspace_bytes(0, 3, 16, 2, 128) == 0


def test_v2_varlen_train_forward_rejects_bad_arguments(lib):
    f = lambda **kw: lib.diffattn_v2_varlen_fwd_train(*[{**dict(q=P, k=P, v=P, lg=P, cu=P, nseq=2, ms=64, N=100, out=P, oh=P, lse=P, Hq=16, Hkv=2, d=128, scale=0.0, causal=1, dt=BF16, st=None), **kw}[n] for n in ("q", "k", "v", "lg", "cu", "nseq", "ms", "N", "out", "oh", "lse", "Hq", "Hkv", "d", "scale", "causal", "dt", "st")])
    assert f(cu=None) == E_INVALID
    assert f(oh=None) == E_INVALID
    assert f(nseq=-1) == E_INVALID
    assert f(Hq=6) == E_INVALID
    assert f(oh=P + 8) == E_ALIGN
    assert f(nseq=0) == 0


def test_v2_decode_noalloc_rejects_bad_and_oversize_arguments(lib):
    # the checks run before the library's array is looked up or anything launches
    f = lambda **kw: lib.diffattn_v2_decode_noalloc(*[{**dict(
        q=P, k=P, v=P, cl=None, lg=P, out=P, B=4, S=4096, Hq=64, Hkv=8, d=128, scale=0.0, dt=BF16,
        st=None), **kw}[n] for n in ("q", "k", "v", "cl", "lg", "out", "B", "S", "Hq", "Hkv", "d",
                                     "scale", "dt", "st")])
    assert f(q=None) == E_INVALID
    assert f(Hq=6, Hkv=2) == E_INVALID
    assert f(d=96) == E_UNSUPPORTED
    assert f(out=P + 8) == E_ALIGN
    assert f(B=0) == 0
    # partials beyond the library's 32 MiB array: rejected with a message
    assert lib.diffattn_v2_decode_workspace_bytes(2048, 4096, 64, 8, 128) > 32 << 20
    assert f(B=2048) == E_UNSUPPORTED
    assert b"diffattn_v2_decode with a workspace" in lib.diffattn_last_error()


def gda(lib, **kw):
    a = dict(q=P, k=P, v=P, lg=P, out=P, cu=None, nseq=0, maxlen=0, B=2, T=64, Hq=16, Hkv=2,
             d=128, ratio=3, scale=0.0, causal=1, dt=BF16, stream=None)
    a.update(kw)
    return lib.diffattn_gda_fwd(a["q"], a["k"], a["v"], a["lg"], a["out"], a["cu"], a["nseq"],
                                a["maxlen"], a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["ratio"],
                                a["scale"], a["causal"], a["dt"], a["stream"])


def test_gda_forward_rejects_bad_arguments(lib):
    assert gda(lib, ratio=0) == E_INVALID
    assert gda(lib, ratio=16) == E_INVALID
    # groups of 8 query heads: blocks of 4 (ratio 3) fit, blocks of 5 (ratio 4) do not
    assert gda(lib, ratio=4) == E_INVALID
    assert b"ratio + 1" in lib.diffattn_last_error()
    assert gda(lib, Hq=15, Hkv=5, ratio=4) == E_INVALID     # groups of 3 cannot hold 5
    assert gda(lib, Hq=15, Hkv=3, ratio=4, B=0) == 0          # odd Hq: one block per group
    assert gda(lib, Hq=10, Hkv=2, ratio=4, B=0) == 0
    assert gda(lib, Hq=10, Hkv=2, ratio=4, T=0) == 0
    assert gda(lib, d=96) == E_UNSUPPORTED
    assert gda(lib, dt=F32) == E_UNSUPPORTED
    assert gda(lib, out=P + 2) == E_ALIGN
    assert gda(lib, cu=P, nseq=-1, maxlen=5) == E_INVALID
    assert gda(lib, cu=P, nseq=0, maxlen=0) == 0


def gdec(lib, **kw):
    a = dict(q=P, k=P, v=P, lens=None, lg=P, out=P, ws=P, wsb=1 << 30, B=4, S=1024, Hq=16, Hkv=2,
             d=128, ratio=3, scale=0.0, dt=BF16, stream=None)
    a.update(kw)
    return lib.diffattn_gda_decode(a["q"], a["k"], a["v"], a["lens"], a["lg"], a["out"], a["ws"],
                                   a["wsb"], a["B"], a["S"], a["Hq"], a["Hkv"], a["d"], a["ratio"],
                                   a["scale"], a["dt"], a["stream"])


def test_gda_decode_rejects_bad_arguments_and_sizes_its_workspace(lib):
    assert gdec(lib, ratio=4) == E_INVALID
    assert gdec(lib, Hq=64, Hkv=2, ratio=3) == E_UNSUPPORTED   # 32 query heads per KV head
    assert gdec(lib, ws=None) == E_WORKSPACE
    assert gdec(lib, wsb=8) == E_WORKSPACE
    assert gdec(lib, B=0) == 0
    # partials are kept per query head, whatever the blocks: the V2 size
    for B, S in ((1, 32768), (64, 4096)):
        assert (lib.diffattn_gda_decode_workspace_bytes(B, S, 16, 2, 128, 3)
                == lib.diffattn_gda_decode_workspace_bytes(B, S, 16, 2, 128, 1)
                == lib.diffattn_v2_decode_workspace_bytes(B, S, 16, 2, 128) > 0)
    assert lib.diffattn_gda_decode_workspace_bytes(4, 1024, 16, 2, 128, 4) == 0
    assert lib.diffattn_gda_decode_workspace_bytes(4, 1024, 10, 2, 128, 4) > 0
