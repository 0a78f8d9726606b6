"""Host-side checks of the C ABI that need no GPU: the library loads, it
exports every function the header declares, and argument validation
returns the documented status codes before anything is enqueued (these
calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

import bit_group_quantized_amd as ql

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlinear.h")

OK, INVALID, SHAPE, MISALIGNED, WORKSPACE = 0, 1, 2, 3, 4
A16 = 0x10000  # fake, 16-byte aligned addresses: validation never dereferences them


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    return ql.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 10
    assert set(names) == set(ql.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_layout_version_and_status_strings(L):
    assert L.ql_layout_version() == 1
    for s in range(6):
        assert L.ql_status_string(s)
    assert L.ql_status_string(99) == b"unknown status"


def _w(K=2048, N=64, gs=64, qw=A16, sc=A16, bi=A16):
    return ql.ql_w4(qw, sc, bi, K, N, gs)


def test_gemv_validation(L):
    f = L.qlinear_gemv
    assert f(None, A16, A16, None) == INVALID
    assert f(ctypes.byref(_w(K=100)), A16, A16, None) == SHAPE
    assert f(ctypes.byref(_w(K=0)), A16, A16, None) == SHAPE
    assert f(ctypes.byref(_w(K=65536)), A16, A16, None) == SHAPE
    assert f(ctypes.byref(_w(gs=32)), A16, A16, None) == SHAPE
    assert f(ctypes.byref(_w(N=-1)), A16, A16, None) == INVALID
    assert f(ctypes.byref(_w(qw=A16 + 4)), A16, A16, None) == MISALIGNED
    assert f(ctypes.byref(_w(sc=A16 + 1)), A16, A16, None) == MISALIGNED
    assert f(ctypes.byref(_w()), A16 + 8, A16, None) == MISALIGNED
    assert f(ctypes.byref(_w()), None, A16, None) == INVALID
    assert f(ctypes.byref(_w(qw=0)), A16, A16, None) == INVALID
    assert f(ctypes.byref(_w(N=0, qw=0, sc=0, bi=0)), None, None, None) == OK  # empty: nothing enqueued


def test_gemv_multi_validation(L):
    f = L.qlinear_gemv_multi

    def call(ws, x=A16, ys=None, count=None):
        arr = (ql.ql_w4 * len(ws))(*ws)
        yp = (ctypes.c_void_p * len(ws))(*([A16] * len(ws) if ys is None else ys))
        return f(arr, len(ws) if count is None else count, x, yp, None)

    assert call([_w()], count=0) == INVALID
    assert call([_w()] * 9) == INVALID                       # more than QL_GEMV_MULTI_MAX
    assert f(None, 1, A16, None, None) == INVALID
    assert call([_w(), _w(K=1024)]) == INVALID               # K differs
    assert call([_w(K=192), _w(K=192)]) == SHAPE             # K not a chunked-kernel K
    assert call([_w(K=100)]) == SHAPE
    assert call([_w(), _w(qw=A16 + 4)]) == MISALIGNED
    assert call([_w()], x=A16 + 8) == MISALIGNED
    assert call([_w()], x=None) == INVALID
    assert call([_w(), _w()], ys=[A16, None]) == INVALID
    assert call([_w(), _w()], ys=[A16, A16 + 1]) == MISALIGNED
    assert call([_w(N=0, qw=0, sc=0, bi=0)] * 2, x=None, ys=[None, None]) == OK  # nothing to do


def test_gemm_validation(L):
    f = L.qlinear_gemm
    assert f(ctypes.byref(_w()), A16, -1, A16, None) == INVALID
    assert f(ctypes.byref(_w()), A16, 0, A16, None) == OK  # empty
    assert f(ctypes.byref(_w(K=96)), A16, 4, A16, None) == SHAPE
    assert f(ctypes.byref(_w()), A16 + 2, 4, A16, None) == MISALIGNED
    assert f(ctypes.byref(_w()), None, 4, A16, None) == INVALID


def test_gemm_few_rows_validation(L):
    f = L.qlinear_gemm_few_rows
    assert f(ctypes.byref(_w(K=2048)), A16, -1, A16, None) == INVALID
    assert f(ctypes.byref(_w(K=2048)), A16, 0, A16, None) == OK  # empty
    assert f(ctypes.byref(_w(K=4096)), A16, 4, A16, None) == SHAPE  # K outside {512, 1024, 2048}
    assert f(ctypes.byref(_w(K=192)), A16, 4, A16, None) == SHAPE
    assert f(ctypes.byref(_w(K=2048)), A16 + 2, 4, A16, None) == MISALIGNED
    assert f(ctypes.byref(_w(K=2048)), None, 4, A16, None) == INVALID


def test_gemm_ksplit_validation(L):
    f = L.qlinear_gemm_ksplit
    assert f(ctypes.byref(_w(K=2048)), A16, -1, A16, None) == INVALID
    assert f(ctypes.byref(_w(K=2048)), A16, 0, A16, None) == OK  # empty
    assert f(ctypes.byref(_w(K=192)), A16, 4, A16, None) == SHAPE  # K not a multiple of 128
    assert f(ctypes.byref(_w(K=64)), A16, 4, A16, None) == SHAPE
    assert f(ctypes.byref(_w(K=2048)), A16 + 2, 4, A16, None) == MISALIGNED
    assert f(ctypes.byref(_w(K=2048)), None, 4, A16, None) == INVALID


def test_pack_validation(L):
    f = L.qlinear_pack
    assert f(A16, 4, 12, A16, None) == SHAPE
    assert f(A16, -1, 16, A16, None) == INVALID
    assert f(A16 + 1, 4, 16, A16, None) == MISALIGNED
    assert f(None, 4, 16, A16, None) == INVALID
    assert f(None, 0, 16, None, None) == OK


def test_workspace_bytes(L):
    f = L.moe_workspace_bytes
    assert f(4096, 256, 8) > 0
    assert f(1, 256, 8) > 0
    assert f(0, 256, 8) > 0
    assert f(4096, 256, 8) >= f(1024, 256, 8) >= f(1, 256, 8)
    assert f(4, 256, 300) == 0      # topk > E
    assert f(4, 2048, 8) == 0       # E > QL_MAX_EXPERTS
    assert f(4, 256, 0) == 0
    assert f(-1, 256, 8) == 0
    # the logits live inside the workspace, after the tile map
    off = L.ql_moe_logits_offset(4096, 256, 8)
    assert off >= 16 + 16 * (4096 * 8 // 128 + 256)
    assert off + 4096 * 256 * 4 <= f(4096, 256, 8)


def _route(L, T=8, D=2048, E=256, topk=8, ws=None, wsb=None, H=A16):
    wsb = L.moe_workspace_bytes(max(T, 0), E, min(topk, E)) if wsb is None else wsb
    return L.moe_route(H, A16, None, T, D, E, topk, A16, A16, A16, A16, A16, A16,
                       A16 if ws is None else ws, wsb, None)


def test_route_validation(L):
    assert _route(L, topk=300) == INVALID
    assert _route(L, T=-1) == INVALID
    assert _route(L, E=2048, topk=8, wsb=1 << 30) == SHAPE
    assert _route(L, topk=33, wsb=1 << 30) == SHAPE
    assert _route(L, D=100) == SHAPE
    assert _route(L, D=0) == INVALID
    assert _route(L, wsb=16) == WORKSPACE
    assert _route(L, ws=0) == WORKSPACE
    assert _route(L, ws=A16 + 16) == MISALIGNED
    assert _route(L, H=None) == INVALID
    assert _route(L, H=A16 + 2) == MISALIGNED


def test_dispatch_validation(L):
    f = L.moe_dispatch
    wsb = L.moe_workspace_bytes(8, 256, 8)
    assert f(None, 8, 256, 8, A16, A16, A16, A16, A16, wsb, None) == INVALID
    assert f(A16, 8, 256, 8, A16, A16, A16, A16, A16, 0, None) == WORKSPACE
    assert f(A16 + 1, 8, 256, 8, A16, A16, A16, A16, A16, wsb, None) == MISALIGNED
    assert f(A16, 8, 4, 8, A16, A16, A16, A16, A16, wsb, None) == INVALID


def test_grouped_gemm_validation(L):
    W = ql.ql_w4_experts(A16, A16, A16, 2048, 1024, 64, 256)
    S = ql.ql_w4(A16, A16, A16, 2048, 1024, 64)
    wsb = L.moe_workspace_bytes(64, 256, 8)
    f = L.moe_grouped_gemm

    def call(op=1, T=64, topk=8, w=W, s=S, wsb=wsb, X=A16):
        return f(ctypes.byref(w), ctypes.byref(s) if s is not None else None, X, T, topk, op,
                 A16, A16, A16, A16, A16, wsb, A16, None)

    assert call(op=7) == INVALID
    assert call(op=3) == SHAPE                 # DOWN_COMBINE is a decode path (T <= 4)
    assert call(topk=300) == INVALID
    assert call(wsb=0) == WORKSPACE
    assert call(X=A16 + 2) == MISALIGNED
    assert call(X=None) == INVALID
    assert call(w=ql.ql_w4_experts(A16, A16, A16, 2048, 1023, 64, 256), s=None) == SHAPE  # odd gate_up width
    assert call(s=ql.ql_w4(A16, A16, A16, 2048, 512, 64)) == INVALID           # shared shape differs
    assert call(T=0) == OK
    # the shared expert alone: needs the shared matrix, not DOWN_COMBINE
    assert call(op=1 | 0x100, s=None) == INVALID
    assert call(op=3 | 0x100) == INVALID
    assert call(op=1 | 0x100, X=A16 + 2) == MISALIGNED
    assert call(op=1 | 0x100, T=0) == OK
    assert call(op=2 | 0x100, T=0, wsb=0) == OK   # no workspace needed


def test_combine_validation(L):
    f = L.moe_combine
    assert f(A16, A16, A16, 4, 33, 2048, 1, A16, None) == SHAPE
    assert f(A16, A16, A16, -1, 8, 2048, 1, A16, None) == INVALID
    assert f(A16 + 2, A16, A16, 4, 8, 2048, 1, A16, None) == MISALIGNED
    assert f(A16, A16, A16, 0, 8, 2048, 1, A16, None) == OK


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "bit_group_quantized_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                assert not re.search(r"\bimport\s+oracle|\bfrom\s+oracle\b|oracle\.", text), fn


def test_gemv_rmsnorm_validation(L):
    f = L.qlinear_gemv_rmsnorm
    assert f(None, A16, A16, 1e-6, A16, None) == INVALID
    assert f(ctypes.byref(_w(K=192)), A16, A16, 1e-6, A16, None) == SHAPE   # not a power of two
    assert f(ctypes.byref(_w(K=128)), A16, A16, 1e-6, A16, None) == SHAPE   # below 256
    assert f(ctypes.byref(_w()), A16, A16, -1.0, A16, None) == INVALID
    assert f(ctypes.byref(_w()), A16, A16, float("nan"), A16, None) == INVALID
    assert f(ctypes.byref(_w()), A16, A16, float("inf"), A16, None) == INVALID
    assert f(ctypes.byref(_w()), A16, None, 1e-6, A16, None) == INVALID
    assert f(ctypes.byref(_w()), A16, A16 + 2, 1e-6, A16, None) == MISALIGNED
    assert f(ctypes.byref(_w()), A16 + 8, A16, 1e-6, A16, None) == MISALIGNED
    assert f(ctypes.byref(_w(N=0, qw=0, sc=0, bi=0)), None, None, 1e-6, None, None) == OK


def test_gemv_argmax_validation(L):
    f = L.qlinear_gemv_argmax
    wsb = L.qlinear_gemv_argmax_workspace_bytes
    assert wsb(151552) == 151552 and wsb(9) == 16 and wsb(1) == 8 and wsb(0) == 0 and wsb(-3) == 0
    ok = wsb(64)
    assert f(None, A16, None, A16, A16, ok, None) == INVALID
    assert f(ctypes.byref(_w(N=0, qw=0, sc=0, bi=0)), A16, None, A16, A16, ok, None) == INVALID  # N < 1
    assert f(ctypes.byref(_w(K=192)), A16, None, A16, A16, ok, None) == SHAPE
    assert f(ctypes.byref(_w()), None, None, A16, A16, ok, None) == INVALID
    assert f(ctypes.byref(_w()), A16, None, None, A16, ok, None) == INVALID
    assert f(ctypes.byref(_w()), A16, None, A16 + 2, A16, ok, None) == MISALIGNED
    assert f(ctypes.byref(_w()), A16, A16 + 1, A16, A16, ok, None) == MISALIGNED
    assert f(ctypes.byref(_w()), A16, None, A16, A16, ok - 8, None) == WORKSPACE
    assert f(ctypes.byref(_w()), A16, None, A16, None, ok, None) == WORKSPACE
    assert f(ctypes.byref(_w()), A16, None, A16, A16 + 4, ok, None) == MISALIGNED


def test_embed_token_validation(L):
    f = L.qlinear_embed_token
    assert f(None, A16, A16, None) == INVALID
    assert f(ctypes.byref(_w(N=0, qw=0, sc=0, bi=0)), A16, A16, None) == INVALID
    assert f(ctypes.byref(_w(K=100)), A16, A16, None) == SHAPE
    assert f(ctypes.byref(_w()), None, A16, None) == INVALID
    assert f(ctypes.byref(_w()), A16, None, None) == INVALID
    assert f(ctypes.byref(_w()), A16 + 2, A16, None) == MISALIGNED
    assert f(ctypes.byref(_w()), A16, A16 + 8, None) == MISALIGNED


def test_bf16_validation(L):
    f = L.qlinear_gemv_bf16
    assert f(None, A16, A16, None) == INVALID
    assert f(ctypes.byref(_w(K=192)), A16, A16, None) == SHAPE      # not a power of two
    assert f(ctypes.byref(_w(K=65536)), A16, A16, None) == SHAPE
    assert f(ctypes.byref(_w()), A16 + 8, A16, None) == MISALIGNED
    assert f(ctypes.byref(_w()), None, A16, None) == INVALID
    assert f(ctypes.byref(_w(N=0, qw=0, sc=0, bi=0)), None, None, None) == OK
    g = L.qlinear_gemm_bf16
    assert g(ctypes.byref(_w()), A16, -1, A16, None) == INVALID
    assert g(ctypes.byref(_w()), A16, 0, A16, None) == OK
    assert g(ctypes.byref(_w(K=96)), A16, 4, A16, None) == SHAPE
    assert g(ctypes.byref(_w()), A16 + 2, 4, A16, None) == MISALIGNED
    assert g(ctypes.byref(_w()), None, 4, A16, None) == INVALID


def test_codec_validation(L):
    f8 = L.qlinear_gemv_fp8
    W8 = lambda K=2048, N=64, c=A16, s=A16: ql.ql_fp8(c, s, K, N)
    assert f8(None, A16, A16, None) == INVALID
    assert f8(ctypes.byref(W8(K=16384)), A16, A16, None) == SHAPE     # FP8 stops at 8192
    assert f8(ctypes.byref(W8(K=192)), A16, A16, None) == SHAPE
    assert f8(ctypes.byref(W8(N=-1)), A16, A16, None) == INVALID
    assert f8(ctypes.byref(W8(c=A16 + 8)), A16, A16, None) == MISALIGNED
    assert f8(ctypes.byref(W8(s=A16 + 1)), A16, A16, None) == MISALIGNED
    assert f8(ctypes.byref(W8()), A16 + 2, A16, None) == MISALIGNED
    assert f8(ctypes.byref(W8(c=0)), A16, A16, None) == INVALID
    assert f8(ctypes.byref(W8(N=0, c=0, s=0)), None, None, None) == OK
    f4 = L.qlinear_gemv_nvfp4
    W4 = lambda K=2048, N=64, q=A16, b=A16: ql.ql_nvfp4(q, b, 0.01, K, N)
    assert f4(None, A16, A16, None) == INVALID
    assert f4(ctypes.byref(W4(K=128)), A16, A16, None) == SHAPE
    assert f4(ctypes.byref(W4(q=A16 + 4)), A16, A16, None) == MISALIGNED
    assert f4(ctypes.byref(W4(b=A16 + 1)), A16, A16, None) == MISALIGNED
    assert f4(ctypes.byref(W4()), None, A16, None) == INVALID
    assert f4(ctypes.byref(W4(N=0, q=0, b=0)), None, None, None) == OK


def test_moe_decode_validation(L):
    GU = ql.ql_w4_experts(A16, A16, A16, 2048, 1024, 64, 256)
    DN = ql.ql_w4_experts(A16, A16, A16, 512, 2048, 64, 256)
    SG = ql.ql_w4(A16, A16, A16, 2048, 1024, 64)
    SD = ql.ql_w4(A16, A16, A16, 512, 2048, 64)
    wsb = L.moe_decode_workspace_bytes(1, 256, 8, 512)
    assert wsb > 0
    assert L.moe_decode_workspace_bytes(5, 256, 8, 512) == 0   # T > QL_DECODE_MAX_T
    assert L.moe_decode_workspace_bytes(1, 256, 300, 512) == 0
    assert L.moe_decode_logits_offset(1, 256, 8) >= 8 * 256 * 4   # after the 8 router partials of 256 fp32
    f = L.moe_decode

    def call(T=1, D=2048, E=256, topk=8, gu=GU, dn=DN, sg=SG, sd=SD, H=A16, ws=A16, wsb=wsb, out=A16):
        r = lambda x: ctypes.byref(x) if x is not None else None
        return f(H, A16, None, T, D, E, topk, r(gu), r(dn), r(sg), r(sd), A16, A16, ws, wsb, out, None)

    assert call(T=5) == SHAPE
    assert call(T=-1) == INVALID
    assert call(topk=300) == INVALID
    assert call(topk=33) == SHAPE
    assert call(E=128) == INVALID                    # experts in W != E
    assert call(D=1024) == INVALID                   # gate_up K != D
    assert call(sd=None) == INVALID                  # shared halves must come together
    assert call(gu=None) == INVALID
    assert call(dn=ql.ql_w4_experts(A16, A16, A16, 256, 2048, 64, 256)) == INVALID  # gate_up N != 2 I
    assert call(gu=ql.ql_w4_experts(A16, A16, A16, 1536, 1024, 64, 256), D=1536,
                dn=ql.ql_w4_experts(A16, A16, A16, 512, 1536, 64, 256),
                sg=None, sd=None) == SHAPE           # D not a power of two
    assert call(H=A16 + 2) == MISALIGNED
    assert call(H=None) == INVALID
    assert call(wsb=16) == WORKSPACE
    assert call(ws=A16 + 16) == MISALIGNED
    assert call(T=0) == OK


def test_moe_decode_codec_validation(L):
    """Host validation of moe_decode_fp8 / moe_decode_nvfp4: the decode
    limits of moe_decode plus each format's own rules."""
    wsb = L.moe_decode_workspace_bytes(1, 256, 8, 512)
    r = lambda x: ctypes.byref(x) if x is not None else None
    f8 = L.moe_decode_fp8
    GU8 = ql.ql_fp8_experts(A16, A16, 2048, 1024, 256)
    DN8 = ql.ql_fp8_experts(A16, A16, 512, 2048, 256)
    SG8, SD8 = ql.ql_fp8(A16, A16, 2048, 1024), ql.ql_fp8(A16, A16, 512, 2048)

    def c8(T=1, D=2048, E=256, topk=8, gu=GU8, dn=DN8, sg=SG8, sd=SD8, H=A16, wsb=wsb):
        return f8(H, A16, None, T, D, E, topk, r(gu), r(dn), r(sg), r(sd), A16, A16, A16, wsb, A16, None)

    assert c8(T=5) == SHAPE
    assert c8(E=128) == INVALID
    assert c8(sd=None) == INVALID
    assert c8(gu=ql.ql_fp8_experts(A16 + 8, A16, 2048, 1024, 256)) == MISALIGNED  # codes 16-byte aligned
    assert c8(sg=ql.ql_fp8(A16, A16, 2048, 512)) == INVALID                       # shared shape differs
    assert c8(H=A16 + 2) == MISALIGNED
    assert c8(wsb=16) == WORKSPACE
    assert c8(T=0) == OK
    f4 = L.moe_decode_nvfp4
    GU4 = ql.ql_nvfp4_experts(A16, A16, A16, 2048, 1024, 256)
    DN4 = ql.ql_nvfp4_experts(A16, A16, A16, 512, 2048, 256)
    SG4, SD4 = ql.ql_nvfp4(A16, A16, 1.0, 2048, 1024), ql.ql_nvfp4(A16, A16, 1.0, 512, 2048)

    def c4(T=1, D=2048, E=256, topk=8, gu=GU4, dn=DN4, sg=SG4, sd=SD4, H=A16, wsb=wsb):
        return f4(H, A16, None, T, D, E, topk, r(gu), r(dn), r(sg), r(sd), A16, A16, A16, wsb, A16, None)

    assert c4(T=5) == SHAPE
    assert c4(topk=33) == SHAPE
    assert c4(gu=ql.ql_nvfp4_experts(A16, A16, None, 2048, 1024, 256)) == INVALID  # global scales needed
    assert c4(sg=ql.ql_nvfp4(A16, A16, float("nan"), 2048, 1024)) == INVALID
    assert c4(dn=ql.ql_nvfp4_experts(A16, A16 + 2, A16, 512, 2048, 256)) == MISALIGNED
    assert c4(D=1024) == INVALID
    assert c4(T=0) == OK


def test_moe_decode_noalloc_validation(L):
    """Host validation of the no-workspace decode entry: every error is
    returned before the scratch array is looked up."""
    GU = ql.ql_w4_experts(A16, A16, A16, 2048, 1024, 64, 256)
    DN = ql.ql_w4_experts(A16, A16, A16, 512, 2048, 64, 256)
    SG = ql.ql_w4(A16, A16, A16, 2048, 1024, 64)
    SD = ql.ql_w4(A16, A16, A16, 512, 2048, 64)
    f = L.moe_decode_noalloc

    def call(T=1, D=2048, E=256, topk=8, gu=GU, dn=DN, sg=SG, sd=SD, H=A16, out=A16):
        r = lambda x: ctypes.byref(x) if x is not None else None
        return f(H, A16, None, T, D, E, topk, r(gu), r(dn), r(sg), r(sd), A16, A16, out, None)

    assert call(T=5) == SHAPE
    assert call(T=-1) == INVALID
    assert call(topk=33) == SHAPE
    assert call(E=128) == INVALID
    assert call(sd=None) == INVALID
    assert call(H=A16 + 2) == MISALIGNED
    assert call(out=None) == INVALID
    assert call(T=0) == OK
    assert ql.QL_DECODE_SCRATCH_BYTES == 1 << 20
    # every shape inside moe_decode's own limits fits the scratch
    assert L.moe_decode_workspace_bytes(4, 1024, 32, 1024) <= ql.QL_DECODE_SCRATCH_BYTES


def test_gemm_fp8_validation(L):
    f = L.qlinear_gemm_fp8

    def call(K=2048, N=64, M=8, codes=A16, X=A16):
        w = ql.ql_fp8(codes, A16, K, N)
        return f(ctypes.byref(w), X, M, A16, None)

    assert call(K=100) == SHAPE
    assert call(K=65536) == SHAPE
    assert call(M=-1) == INVALID
    assert call(codes=None) == INVALID
    assert call(codes=A16 + 8) == MISALIGNED
    assert call(X=A16 + 2) == MISALIGNED
    assert call(M=0) == OK
    assert call(N=0) == OK
    assert f(None, A16, 8, A16, None) == INVALID


def test_gemm_nvfp4_validation(L):
    f = L.qlinear_gemm_nvfp4

    def call(K=2048, N=64, M=8, qw=A16, bs=A16, g=1.0, X=A16):
        w = ql.ql_nvfp4(qw, bs, g, K, N)
        return f(ctypes.byref(w), X, M, A16, None)

    assert call(K=96) == SHAPE
    assert call(M=-1) == INVALID
    assert call(g=float("inf")) == INVALID
    assert call(qw=None) == INVALID
    assert call(bs=A16 + 2) == MISALIGNED
    assert call(qw=A16 + 4) == MISALIGNED
    assert call(M=0) == OK


def test_grouped_gemm_fp8_validation(L):
    f = L.moe_grouped_gemm_fp8
    wsb = L.moe_workspace_bytes(64, 256, 8)

    def call(op=1, T=64, topk=8, K=2048, N=1024, E=256, codes=A16, s=True, sN=1024, wsb=wsb, X=A16):
        w = ql.ql_fp8_experts(codes, A16, K, N, E)
        sh = ql.ql_fp8(A16, A16, K, sN)
        return f(ctypes.byref(w), ctypes.byref(sh) if s else None, X, T, topk, op, A16, A16, gp, gp,
                 A16, wsb, A16, None)

    gp = A16
    assert f(None, None, A16, 64, 8, 1, A16, A16, A16, A16, A16, wsb, A16, None) == INVALID
    assert call(op=7) == INVALID
    assert call(op=3) == SHAPE                 # DOWN_COMBINE is a decode path (T <= 4)
    gp = None
    assert call(op=3, T=2) == INVALID          # ... and needs the gates and positions
    gp = A16
    assert call(K=100) == SHAPE
    assert call(K=65536) == SHAPE
    assert call(codes=None) == INVALID
    assert call(codes=A16 + 8) == MISALIGNED
    assert call(sN=512) == INVALID             # shared shape differs
    assert call(N=1023, s=False) == SHAPE      # odd gate_up width
    assert call(topk=300) == INVALID
    assert call(E=0) == INVALID
    assert call(wsb=0) == WORKSPACE
    assert call(X=A16 + 2) == MISALIGNED
    assert call(X=None) == INVALID
    assert call(T=0) == OK


def test_grouped_gemm_nvfp4_validation(L):
    f = L.moe_grouped_gemm_nvfp4
    wsb = L.moe_workspace_bytes(64, 256, 8)

    def call(op=1, T=64, topk=8, K=2048, N=1024, E=256, qw=A16, bs=A16, gs=A16, s=True, sN=1024,
             sg=1.0, wsb=wsb, X=A16):
        w = ql.ql_nvfp4_experts(qw, bs, gs, K, N, E)
        sh = ql.ql_nvfp4(A16, A16, sg, K, sN)
        return f(ctypes.byref(w), ctypes.byref(sh) if s else None, X, T, topk, op, A16, A16, A16, A16,
                 A16, wsb, A16, None)

    assert f(None, None, A16, 64, 8, 1, A16, A16, A16, A16, A16, wsb, A16, None) == INVALID
    assert call(op=7) == INVALID
    assert call(op=3) == SHAPE                 # DOWN_COMBINE is a decode path (T <= 4)
    assert call(K=96) == SHAPE
    assert call(qw=None) == INVALID
    assert call(gs=None) == INVALID
    assert call(qw=A16 + 8) == MISALIGNED
    assert call(bs=A16 + 2) == MISALIGNED
    assert call(gs=A16 + 2) == MISALIGNED
    assert call(sN=512) == INVALID
    assert call(sg=float("nan")) == INVALID
    assert call(sg=float("inf")) == INVALID
    assert call(N=1023, s=False) == SHAPE
    assert call(topk=300) == INVALID
    assert call(wsb=0) == WORKSPACE
    assert call(X=A16 + 2) == MISALIGNED
    assert call(T=0) == OK
