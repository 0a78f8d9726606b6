"""Python binding of libqlinear (group-affine 4-bit linear layers and
routed-expert MoE on MI355X / gfx950).

Argument marshalling only: every function here checks nothing beyond what
is needed to build the C call, passes device pointers from torch tensors
and the current HIP stream, and raises QLError on a nonzero status.  All
arithmetic runs in the HIP kernels of the library.  There is no fallback:
if the library is not built, importing the functions works but every call
raises.

Weights are passed as dicts of torch tensors with keys ``qweight`` (int32
or uint32-as-int32, [N, K/8] or [E, N, K/8]), ``scales`` and ``biases``
(float16, [N, K/64] or [E, N, K/64]) and ints ``K`` and ``N``.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqlinear.so")

QL_OK = 0
QL_OP_GATE_UP_SILU = 1
QL_OP_DOWN = 2
QL_OP_DOWN_COMBINE = 3
QL_OP_SHARED_ONLY = 0x100  # or'ed into op: the shared expert's rows only
QL_MOE_TILE_ROWS = 128
QL_DECODE_MAX_T = 4
GROUP = 64


class QLError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class ql_w4(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("K", ctypes.c_int32), ("N", ctypes.c_int32),
                ("group_size", ctypes.c_int32)]


class ql_w4_experts(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("K", ctypes.c_int32), ("N", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("num_experts", ctypes.c_int32)]


class ql_fp8(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("K", ctypes.c_int32),
                ("N", ctypes.c_int32)]


class ql_fp8_experts(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("K", ctypes.c_int32),
                ("N", ctypes.c_int32), ("num_experts", ctypes.c_int32)]


class ql_nvfp4(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("block_scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_float), ("K", ctypes.c_int32), ("N", ctypes.c_int32)]


class ql_nvfp4_experts(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("block_scales", ctypes.c_void_p),
                ("global_scales", ctypes.c_void_p), ("K", ctypes.c_int32), ("N", ctypes.c_int32),
                ("num_experts", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "ql_layout_version": (ctypes.c_int, []),
    "ql_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlinear_pack": (ctypes.c_int, [_P, _I32, _I32, _P, _P]),
    "qlinear_gemv": (ctypes.c_int, [ctypes.POINTER(ql_w4), _P, _P, _P]),
    "qlinear_gemm": (ctypes.c_int, [ctypes.POINTER(ql_w4), _P, ctypes.c_int64, _P, _P]),
    "qlinear_gemm_few_rows": (ctypes.c_int, [ctypes.POINTER(ql_w4), _P, ctypes.c_int64, _P, _P]),
    "qlinear_gemm_ksplit": (ctypes.c_int, [ctypes.POINTER(ql_w4), _P, ctypes.c_int64, _P, _P]),
    "qlinear_gemv_fp8": (ctypes.c_int, [ctypes.POINTER(ql_fp8), _P, _P, _P]),
    "qlinear_gemv_nvfp4": (ctypes.c_int, [ctypes.POINTER(ql_nvfp4), _P, _P, _P]),
    "qlinear_gemm_fp8": (ctypes.c_int, [ctypes.POINTER(ql_fp8), _P, ctypes.c_int64, _P, _P]),
    "qlinear_gemm_nvfp4": (ctypes.c_int, [ctypes.POINTER(ql_nvfp4), _P, ctypes.c_int64, _P, _P]),
    "qlinear_gemv_bf16": (ctypes.c_int, [ctypes.POINTER(ql_w4), _P, _P, _P]),
    "qlinear_gemm_bf16": (ctypes.c_int, [ctypes.POINTER(ql_w4), _P, ctypes.c_int64, _P, _P]),
    "qlinear_gemv_rmsnorm": (ctypes.c_int, [ctypes.POINTER(ql_w4), _P, _P, ctypes.c_float, _P, _P]),
    "qlinear_gemv_argmax_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64]),
    "qlinear_gemv_argmax": (ctypes.c_int, [ctypes.POINTER(ql_w4), _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "qlinear_embed_token": (ctypes.c_int, [ctypes.POINTER(ql_w4), _P, _P, _P]),
    "moe_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32]),
    "ql_moe_logits_offset": (ctypes.c_size_t, [_I32, _I32, _I32]),
    "moe_route": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                 _P, ctypes.c_size_t, _P]),
    "qlinear_gemv_multi": (ctypes.c_int, [ctypes.POINTER(ql_w4), _I32, _P, ctypes.POINTER(ctypes.c_void_p), _P]),
    "moe_dispatch": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_grouped_gemm": (ctypes.c_int, [ctypes.POINTER(ql_w4_experts), ctypes.POINTER(ql_w4), _P,
                                        _I32, _I32, _I32, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                        _P, _P]),
    "moe_combine": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P]),
    "moe_route_bf16": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                      _P, ctypes.c_size_t, _P]),
    "moe_grouped_gemm_bf16": (ctypes.c_int, [ctypes.POINTER(ql_w4_experts), ctypes.POINTER(ql_w4), _P,
                                             _I32, _I32, _I32, _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "moe_combine_bf16": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P]),
    "moe_grouped_gemm_fp8": (ctypes.c_int, [ctypes.POINTER(ql_fp8_experts), ctypes.POINTER(ql_fp8), _P,
                                            _I32, _I32, _I32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "moe_grouped_gemm_nvfp4": (ctypes.c_int, [ctypes.POINTER(ql_nvfp4_experts), ctypes.POINTER(ql_nvfp4),
                                              _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P,
                                              _P]),
    "moe_decode_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32]),
    "moe_decode_logits_offset": (ctypes.c_size_t, [_I32, _I32, _I32]),
    "moe_decode": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32,
                                  ctypes.POINTER(ql_w4_experts), ctypes.POINTER(ql_w4_experts),
                                  ctypes.POINTER(ql_w4), ctypes.POINTER(ql_w4), _P, _P, _P,
                                  ctypes.c_size_t, _P, _P]),
    "moe_decode_bf16": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32,
                                       ctypes.POINTER(ql_w4_experts), ctypes.POINTER(ql_w4_experts),
                                       ctypes.POINTER(ql_w4), ctypes.POINTER(ql_w4), _P, _P, _P,
                                       ctypes.c_size_t, _P, _P]),
    "moe_decode_fp8": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32,
                                      ctypes.POINTER(ql_fp8_experts), ctypes.POINTER(ql_fp8_experts),
                                      ctypes.POINTER(ql_fp8), ctypes.POINTER(ql_fp8), _P, _P, _P,
                                      ctypes.c_size_t, _P, _P]),
    "moe_decode_nvfp4": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32,
                                        ctypes.POINTER(ql_nvfp4_experts), ctypes.POINTER(ql_nvfp4_experts),
                                        ctypes.POINTER(ql_nvfp4), ctypes.POINTER(ql_nvfp4), _P, _P, _P,
                                        ctypes.c_size_t, _P, _P]),
    "moe_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32,
                                          ctypes.POINTER(ql_w4_experts), ctypes.POINTER(ql_w4_experts),
                                          ctypes.POINTER(ql_w4), ctypes.POINTER(ql_w4), _P, _P, _P, _P]),
}
EXPORTS = tuple(_SIGS)

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m bit_group_quantized_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != QL_OK:
        raise QLError(fn, status, lib().ql_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_w4(W: dict) -> ql_w4:
    return ql_w4(W["qweight"].data_ptr(), W["scales"].data_ptr(), W["biases"].data_ptr(),
                 int(W["K"]), int(W["N"]), GROUP)


def make_w4_experts(W: dict) -> ql_w4_experts:
    return ql_w4_experts(W["qweight"].data_ptr(), W["scales"].data_ptr(), W["biases"].data_ptr(),
                         int(W["K"]), int(W["N"]), GROUP, int(W["qweight"].shape[0]))


def ql_layout_version() -> int:
    return lib().ql_layout_version()


def qlinear_pack(codes, qweight=None, stream=None):
    """codes uint8 [N, K] (values 0..15) -> packed int32 [N, K/8] on the device."""
    import torch
    N, K = codes.shape
    if qweight is None:
        qweight = torch.empty((N, K // 8), dtype=torch.int32, device=codes.device)
    _check("qlinear_pack", lib().qlinear_pack(_ptr(codes), N, K, _ptr(qweight), _stream(stream)))
    return qweight


def qlinear_gemv(W: dict, x, y=None, stream=None):
    """y [N] fp16 = x [K] fp16 . dequant(W)."""
    import torch
    if y is None:
        y = torch.empty((int(W["N"]),), dtype=torch.float16, device=x.device)
    w = make_w4(W)
    _check("qlinear_gemv", lib().qlinear_gemv(ctypes.byref(w), _ptr(x), _ptr(y), _stream(stream)))
    return y


def qlinear_gemv_fp8(W: dict, x, y=None, stream=None):
    """y [N] fp16 = x [K] fp16 . W, W = {"codes": uint8 [N, K] E4M3,
    "scales": fp16 [N, K/64], "K", "N"}."""
    import torch
    if y is None:
        y = torch.empty((int(W["N"]),), dtype=torch.float16, device=x.device)
    w = ql_fp8(W["codes"].data_ptr(), W["scales"].data_ptr(), int(W["K"]), int(W["N"]))
    _check("qlinear_gemv_fp8", lib().qlinear_gemv_fp8(ctypes.byref(w), _ptr(x), _ptr(y), _stream(stream)))
    return y


def qlinear_gemm_fp8(W: dict, X, Y=None, stream=None):
    """Y [M, N] fp16 = X [M, K] fp16 . W for FP8-E4M3 weights (as
    qlinear_gemv_fp8's W)."""
    import torch
    M = int(X.shape[0])
    if Y is None:
        Y = torch.empty((M, int(W["N"])), dtype=torch.float16, device=X.device)
    w = ql_fp8(W["codes"].data_ptr(), W["scales"].data_ptr(), int(W["K"]), int(W["N"]))
    _check("qlinear_gemm_fp8", lib().qlinear_gemm_fp8(ctypes.byref(w), _ptr(X), M, _ptr(Y), _stream(stream)))
    return Y


def qlinear_gemm_nvfp4(W: dict, X, Y=None, stream=None):
    """Y [M, N] fp16 = X [M, K] fp16 . W for NVFP4 weights (as
    qlinear_gemv_nvfp4's W)."""
    import torch
    M = int(X.shape[0])
    if Y is None:
        Y = torch.empty((M, int(W["N"])), dtype=torch.float16, device=X.device)
    w = ql_nvfp4(W["qweight"].data_ptr(), W["block_scales"].data_ptr(), float(W["global_scale"]),
                 int(W["K"]), int(W["N"]))
    _check("qlinear_gemm_nvfp4", lib().qlinear_gemm_nvfp4(ctypes.byref(w), _ptr(X), M, _ptr(Y), _stream(stream)))
    return Y


def qlinear_gemv_nvfp4(W: dict, x, y=None, stream=None):
    """y [N] fp16 = x [K] fp16 . W, W = {"qweight": int32 [N, K/8] E2M1,
    "block_scales": uint8 [N, K/16] E4M3, "global_scale": float, "K", "N"}."""
    import torch
    if y is None:
        y = torch.empty((int(W["N"]),), dtype=torch.float16, device=x.device)
    w = ql_nvfp4(W["qweight"].data_ptr(), W["block_scales"].data_ptr(), float(W["global_scale"]),
                 int(W["K"]), int(W["N"]))
    _check("qlinear_gemv_nvfp4", lib().qlinear_gemv_nvfp4(ctypes.byref(w), _ptr(x), _ptr(y), _stream(stream)))
    return y


def qlinear_gemv_bf16(W: dict, x, y=None, stream=None):
    """y [N] bf16 = x [K] bf16 . dequant(W), W's scales and biases bf16."""
    import torch
    if y is None:
        y = torch.empty((int(W["N"]),), dtype=torch.bfloat16, device=x.device)
    w = make_w4(W)
    _check("qlinear_gemv_bf16", lib().qlinear_gemv_bf16(ctypes.byref(w), _ptr(x), _ptr(y), _stream(stream)))
    return y


def qlinear_gemm_bf16(W: dict, X, Y=None, stream=None):
    """Y [M, N] bf16 = X [M, K] bf16 . dequant(W), W's scales and biases bf16."""
    import torch
    M = int(X.shape[0])
    if Y is None:
        Y = torch.empty((M, int(W["N"])), dtype=torch.bfloat16, device=X.device)
    w = make_w4(W)
    _check("qlinear_gemm_bf16", lib().qlinear_gemm_bf16(ctypes.byref(w), _ptr(X), M, _ptr(Y), _stream(stream)))
    return Y


def qlinear_gemv_rmsnorm(W: dict, x, gamma, eps: float, y=None, stream=None):
    """y [N] fp16 = fp16(rmsnorm(x [K], gamma [K], eps)) . dequant(W)."""
    import torch
    if y is None:
        y = torch.empty((int(W["N"]),), dtype=torch.float16, device=x.device)
    w = make_w4(W)
    _check("qlinear_gemv_rmsnorm", lib().qlinear_gemv_rmsnorm(
        ctypes.byref(w), _ptr(x), _ptr(gamma), float(eps), _ptr(y), _stream(stream)))
    return y


def gemv_argmax_workspace(N: int, device):
    """Workspace tensor for qlinear_gemv_argmax with N outputs."""
    import torch
    nbytes = lib().qlinear_gemv_argmax_workspace_bytes(int(N))
    return torch.empty((max(nbytes, 8) // 8,), dtype=torch.int64, device=device)


def qlinear_gemv_argmax(W: dict, x, token=None, logits=None, workspace=None, stream=None):
    """token int32 [1] (device) = index of the largest logit of x . dequant(W);
    logits fp16 [N] are written too when given."""
    import torch
    if token is None:
        token = torch.empty((1,), dtype=torch.int32, device=x.device)
    if workspace is None:
        workspace = gemv_argmax_workspace(int(W["N"]), x.device)
    w = make_w4(W)
    _check("qlinear_gemv_argmax", lib().qlinear_gemv_argmax(
        ctypes.byref(w), _ptr(x), _ptr(logits), _ptr(token), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return token


def qlinear_embed_token(E: dict, token, x=None, stream=None):
    """x [K] fp16 = row token[0] (device int32) of the w4 table E."""
    import torch
    if x is None:
        x = torch.empty((int(E["K"]),), dtype=torch.float16, device=token.device)
    w = make_w4(E)
    _check("qlinear_embed_token", lib().qlinear_embed_token(
        ctypes.byref(w), _ptr(token), _ptr(x), _stream(stream)))
    return x


def qlinear_gemm(W: dict, X, Y=None, stream=None):
    """Y [M, N] fp16 = X [M, K] fp16 . dequant(W)."""
    import torch
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, int(W["N"])), dtype=torch.float16, device=X.device)
    w = make_w4(W)
    _check("qlinear_gemm", lib().qlinear_gemm(ctypes.byref(w), _ptr(X), M, _ptr(Y), _stream(stream)))
    return Y


def qlinear_gemm_few_rows(W: dict, X, Y=None, stream=None):
    """Y [M, N] fp16 = X [M, K] fp16 . dequant(W), weight-stationary kernel
    for few rows (K in 512, 1024, 2048)."""
    import torch
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, int(W["N"])), dtype=torch.float16, device=X.device)
    w = make_w4(W)
    _check("qlinear_gemm_few_rows",
           lib().qlinear_gemm_few_rows(ctypes.byref(w), _ptr(X), M, _ptr(Y), _stream(stream)))
    return Y


def qlinear_gemm_ksplit(W: dict, X, Y=None, stream=None):
    """Y [M, N] fp16 = X [M, K] fp16 . dequant(W), each workgroup's K in two
    halves side by side (a few hundred rows; K a multiple of 128)."""
    import torch
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, int(W["N"])), dtype=torch.float16, device=X.device)
    w = make_w4(W)
    _check("qlinear_gemm_ksplit",
           lib().qlinear_gemm_ksplit(ctypes.byref(w), _ptr(X), M, _ptr(Y), _stream(stream)))
    return Y


def moe_workspace_bytes(T: int, E: int, topk: int) -> int:
    return int(lib().moe_workspace_bytes(T, E, topk))


def ql_moe_logits_offset(T: int, E: int, topk: int) -> int:
    return int(lib().ql_moe_logits_offset(T, E, topk))


def alloc_route_outputs(T: int, E: int, topk: int, device):
    """Device buffers for moe_route / moe_dispatch outputs."""
    import torch
    i32 = dict(dtype=torch.int32, device=device)
    ws_bytes = moe_workspace_bytes(T, E, topk)
    return {
        "ids": torch.empty((T, topk), **i32),
        "gates": torch.empty((T, topk), dtype=torch.float32, device=device),
        "counts": torch.empty((E,), **i32),
        "offsets": torch.empty((E + 1,), **i32),
        "sorted_assign": torch.empty((T * topk,), **i32),
        "pos": torch.empty((T * topk,), **i32),
        "workspace": torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device=device),
    }


def moe_route(H, Wr, logit_bias, topk: int, out: dict | None = None, stream=None) -> dict:
    T, D = H.shape
    E = Wr.shape[1]
    if out is None:
        out = alloc_route_outputs(T, E, topk, H.device)
    ws = out["workspace"]
    _check("moe_route", lib().moe_route(
        _ptr(H), _ptr(Wr), _ptr(logit_bias), T, D, E, topk, _ptr(out["ids"]), _ptr(out["gates"]),
        _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["sorted_assign"]), _ptr(out["pos"]),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_dispatch(ids, E: int, out: dict | None = None, stream=None) -> dict:
    T, topk = ids.shape
    if out is None:
        out = alloc_route_outputs(T, E, topk, ids.device)
    out["ids"] = ids
    ws = out["workspace"]
    _check("moe_dispatch", lib().moe_dispatch(
        _ptr(ids), T, E, topk, _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["sorted_assign"]), _ptr(out["pos"]), _ptr(ws), ws.numel(), _stream(stream)))
    return out


QL_GEMV_MULTI_MAX = 8


def qlinear_gemv_multi(Ws: list, x, ys: list | None = None, stream=None) -> list:
    """y_i = x . dequant(W_i) for matrices sharing x (same K), one launch."""
    import torch
    n = len(Ws)
    arr = (ql_w4 * n)(*[make_w4(W) for W in Ws])
    if ys is None:
        ys = [torch.empty(int(W["N"]), dtype=torch.float16, device=x.device) for W in Ws]
    yp = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    _check("qlinear_gemv_multi", lib().qlinear_gemv_multi(arr, n, _ptr(x), yp, _stream(stream)))
    return ys


def _route_args(route):
    """Routing pointers of a grouped-GEMM call; route may be None for the
    QL_OP_SHARED_ONLY calls, which read none of them."""
    if route is None:
        return None, None, None, None, None, 0
    ws = route["workspace"]
    return (_ptr(route["offsets"]), _ptr(route["sorted_assign"]), _ptr(route.get("gates")),
            _ptr(route.get("pos")), _ptr(ws), ws.numel())


def moe_grouped_gemm(W: dict, shared: dict | None, X, T: int, topk: int, op: int, route: dict,
                     Y=None, stream=None):
    """Expert projections over the routed rows described by ``route`` (the
    dict returned by moe_route / moe_dispatch)."""
    import torch
    w = make_w4_experts(W)
    s = make_w4(shared) if shared is not None else None
    rows = T * topk + (T if shared is not None else 0)
    base = op & ~QL_OP_SHARED_ONLY
    if Y is None:
        if base == QL_OP_GATE_UP_SILU:
            shape = (rows, int(W["N"]) // 2)
        elif base == QL_OP_DOWN:
            shape = (rows, int(W["N"]))
        else:
            shape = (T, int(W["N"]))
        Y = torch.empty(shape, dtype=torch.float16, device=X.device)
    off, sa, gates, pos, ws, nws = _route_args(route)
    _check("moe_grouped_gemm", lib().moe_grouped_gemm(
        ctypes.byref(w), ctypes.byref(s) if s is not None else None, _ptr(X), T, topk, op,
        off, sa, gates, pos, ws, nws, _ptr(Y), _stream(stream)))
    return Y


def moe_route_bf16(H, Wr, logit_bias, topk: int, out: dict | None = None, stream=None) -> dict:
    """moe_route with bf16 H and Wr (tensors of bf16 patterns, any 16-bit dtype)."""
    T, D = H.shape
    E = Wr.shape[1]
    if out is None:
        out = alloc_route_outputs(T, E, topk, H.device)
    ws = out["workspace"]
    _check("moe_route_bf16", lib().moe_route_bf16(
        _ptr(H), _ptr(Wr), _ptr(logit_bias), T, D, E, topk, _ptr(out["ids"]), _ptr(out["gates"]),
        _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["sorted_assign"]), _ptr(out["pos"]),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_grouped_gemm_bf16(W: dict, shared: dict | None, X, T: int, topk: int, op: int, route: dict,
                          Y=None, stream=None):
    """moe_grouped_gemm with bf16 X, scales, biases and Y (QL_OP_GATE_UP_SILU or QL_OP_DOWN)."""
    import torch
    w = make_w4_experts(W)
    s = make_w4(shared) if shared is not None else None
    rows = T * topk + (T if shared is not None else 0)
    if Y is None:
        shape = ((rows, int(W["N"]) // 2) if (op & ~QL_OP_SHARED_ONLY) == QL_OP_GATE_UP_SILU
                 else (rows, int(W["N"])))
        Y = torch.empty(shape, dtype=torch.bfloat16, device=X.device)
    off, sa, _, _, ws, nws = _route_args(route)
    _check("moe_grouped_gemm_bf16", lib().moe_grouped_gemm_bf16(
        ctypes.byref(w), ctypes.byref(s) if s is not None else None, _ptr(X), T, topk, op,
        off, sa, ws, nws, _ptr(Y), _stream(stream)))
    return Y


def moe_grouped_gemm_fp8(W: dict, shared: dict | None, X, T: int, topk: int, op: int, route: dict,
                         Y=None, stream=None):
    """moe_grouped_gemm with FP8 experts: W holds codes uint8 [E][N][K] and
    fp16 scales [E][N][K/64] (device tensors), shared one such matrix or None
    (QL_OP_GATE_UP_SILU or QL_OP_DOWN)."""
    import torch
    w, s = _fp8_structs(W, shared)
    rows = T * topk + (T if shared is not None else 0)
    Y = _grouped_out(Y, W, T, rows, op, X.device)
    off, sa, gates, pos, ws, nws = _route_args(route)
    _check("moe_grouped_gemm_fp8", lib().moe_grouped_gemm_fp8(
        ctypes.byref(w), ctypes.byref(s) if s is not None else None, _ptr(X), T, topk, op,
        off, sa, gates, pos, ws, nws, _ptr(Y), _stream(stream)))
    return Y


def _grouped_out(Y, W, T, rows, op, device):
    import torch
    if Y is not None:
        return Y
    base = op & ~QL_OP_SHARED_ONLY
    if base == QL_OP_GATE_UP_SILU:
        shape = (rows, int(W["N"]) // 2)
    elif base == QL_OP_DOWN:
        shape = (rows, int(W["N"]))
    else:
        shape = (T, int(W["N"]))
    return torch.empty(shape, dtype=torch.float16, device=device)


def _fp8_structs(W, shared):
    import torch
    codes = W["codes"]
    if codes.dtype != torch.uint8 or codes.dim() != 3 or W["scales"].dtype != torch.float16:
        raise ValueError("FP8 experts: codes uint8 [E][N][K], scales float16 [E][N][K/64]")
    w = ql_fp8_experts(codes.data_ptr(), W["scales"].data_ptr(), int(W["K"]), int(W["N"]),
                       int(codes.shape[0]))
    s = (ql_fp8(shared["codes"].data_ptr(), shared["scales"].data_ptr(), int(shared["K"]),
                int(shared["N"])) if shared is not None else None)
    return w, s


def _nvfp4_structs(W, shared):
    import torch
    qw = W["qweight"]
    g = W["global_scale"]
    if (qw.dim() != 3 or W["block_scales"].dtype != torch.uint8 or not torch.is_tensor(g)
            or g.dtype != torch.float32 or g.numel() != qw.shape[0] or not g.is_cuda):
        raise ValueError("NVFP4 experts: qweight [E][N][K/8], block_scales uint8 [E][N][K/16], "
                         "global_scale a float32 device tensor [E]")
    w = ql_nvfp4_experts(qw.data_ptr(), W["block_scales"].data_ptr(), W["global_scale"].data_ptr(),
                         int(W["K"]), int(W["N"]), int(qw.shape[0]))
    s = (ql_nvfp4(shared["qweight"].data_ptr(), shared["block_scales"].data_ptr(),
                  float(shared["global_scale"]), int(shared["K"]), int(shared["N"]))
         if shared is not None else None)
    return w, s


def moe_grouped_gemm_nvfp4(W: dict, shared: dict | None, X, T: int, topk: int, op: int, route: dict,
                           Y=None, stream=None):
    """moe_grouped_gemm with NVFP4 experts: W holds qweight [E][N][K/8],
    block_scales uint8 [E][N][K/16] and global_scale fp32 [E] (device
    tensors), shared one NVFP4 matrix (global_scale a float) or None."""
    w, s = _nvfp4_structs(W, shared)
    rows = T * topk + (T if shared is not None else 0)
    Y = _grouped_out(Y, W, T, rows, op, X.device)
    off, sa, gates, pos, ws, nws = _route_args(route)
    _check("moe_grouped_gemm_nvfp4", lib().moe_grouped_gemm_nvfp4(
        ctypes.byref(w), ctypes.byref(s) if s is not None else None, _ptr(X), T, topk, op,
        off, sa, gates, pos, ws, nws, _ptr(Y), _stream(stream)))
    return Y


def moe_combine_bf16(Ydown, gates, pos, T: int, topk: int, has_shared: bool, out=None, stream=None):
    """moe_combine over bf16 rows; out holds bf16 patterns."""
    import torch
    N = Ydown.shape[1]
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=Ydown.device)
    _check("moe_combine_bf16", lib().moe_combine_bf16(_ptr(Ydown), _ptr(gates), _ptr(pos), T, topk, N,
                                                      int(has_shared), _ptr(out), _stream(stream)))
    return out


def moe_decode_workspace_bytes(T: int, E: int, topk: int, I: int) -> int:
    return int(lib().moe_decode_workspace_bytes(T, E, topk, I))


def moe_decode_logits_offset(T: int, E: int, topk: int) -> int:
    return int(lib().moe_decode_logits_offset(T, E, topk))


def alloc_decode_outputs(T: int, E: int, topk: int, D: int, I: int, device) -> dict:
    """Device buffers for moe_decode."""
    import torch
    ws_bytes = moe_decode_workspace_bytes(T, E, topk, I)
    return {
        "ids": torch.empty((T, topk), dtype=torch.int32, device=device),
        "gates": torch.empty((T, topk), dtype=torch.float32, device=device),
        "out": torch.empty((T, D), dtype=torch.float16, device=device),
        "workspace": torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device=device),
    }


def moe_decode(H, Wr, logit_bias, topk: int, gate_up: dict, down: dict, shared_gate_up=None,
               shared_down=None, out: dict | None = None, stream=None, bf16: bool = False) -> dict:
    """The routed-expert layer of T <= QL_DECODE_MAX_T tokens in three
    launches; returns the dict of ids, gates, out and workspace.  bf16=True
    calls moe_decode_bf16 (every 16-bit array bf16; out is then bfloat16)."""
    import torch
    T, D = H.shape
    E = Wr.shape[1]
    I = int(down["K"])
    if out is None:
        out = alloc_decode_outputs(T, E, topk, D, I, H.device)
        if bf16:
            out["out"] = torch.empty((T, D), dtype=torch.bfloat16, device=H.device)
    gu, dn = make_w4_experts(gate_up), make_w4_experts(down)
    sg = make_w4(shared_gate_up) if shared_gate_up is not None else None
    sd = make_w4(shared_down) if shared_down is not None else None
    ws = out["workspace"]
    name = "moe_decode_bf16" if bf16 else "moe_decode"
    _check(name, getattr(lib(), name)(
        _ptr(H), _ptr(Wr), _ptr(logit_bias), T, D, E, topk, ctypes.byref(gu), ctypes.byref(dn),
        ctypes.byref(sg) if sg is not None else None, ctypes.byref(sd) if sd is not None else None,
        _ptr(out["ids"]), _ptr(out["gates"]), _ptr(ws), ws.numel(), _ptr(out["out"]),
        _stream(stream)))
    return out


def moe_decode_codec(codec: str, H, Wr, logit_bias, topk: int, gate_up: dict, down: dict,
                     shared_gate_up=None, shared_down=None, out: dict | None = None, stream=None) -> dict:
    """moe_decode_fp8 (codec "fp8") or moe_decode_nvfp4 ("nvfp4"): the decode
    layer with codec experts, fp16 H / Wr / out; returns the dict of ids,
    gates, out and workspace."""
    T, D = H.shape
    E = Wr.shape[1]
    I = int(down["K"])
    if out is None:
        out = alloc_decode_outputs(T, E, topk, D, I, H.device)
    make = _fp8_structs if codec == "fp8" else _nvfp4_structs
    gu, sg = make(gate_up, shared_gate_up)
    dn, sd = make(down, shared_down)
    ws = out["workspace"]
    name = "moe_decode_fp8" if codec == "fp8" else "moe_decode_nvfp4"
    _check(name, getattr(lib(), name)(
        _ptr(H), _ptr(Wr), _ptr(logit_bias), T, D, E, topk, ctypes.byref(gu), ctypes.byref(dn),
        ctypes.byref(sg) if sg is not None else None, ctypes.byref(sd) if sd is not None else None,
        _ptr(out["ids"]), _ptr(out["gates"]), _ptr(ws), ws.numel(), _ptr(out["out"]),
        _stream(stream)))
    return out


QL_DECODE_SCRATCH_BYTES = 1 << 20


def moe_decode_noalloc(H, Wr, logit_bias, topk: int, gate_up: dict, down: dict, shared_gate_up=None,
                       shared_down=None, ids=None, gates=None, out=None, stream=None):
    """moe_decode on the library's own device scratch (no workspace
    argument); ids, gates and out are caller-owned and allocated here only
    when not given.  Returns (ids, gates, out)."""
    import torch
    T, D = H.shape
    E = Wr.shape[1]
    if ids is None:
        ids = torch.empty((T, topk), dtype=torch.int32, device=H.device)
    if gates is None:
        gates = torch.empty((T, topk), dtype=torch.float32, device=H.device)
    if out is None:
        out = torch.empty((T, D), dtype=torch.float16, device=H.device)
    gu, dn = make_w4_experts(gate_up), make_w4_experts(down)
    sg = make_w4(shared_gate_up) if shared_gate_up is not None else None
    sd = make_w4(shared_down) if shared_down is not None else None
    _check("moe_decode_noalloc", lib().moe_decode_noalloc(
        _ptr(H), _ptr(Wr), _ptr(logit_bias), T, D, E, topk, ctypes.byref(gu), ctypes.byref(dn),
        ctypes.byref(sg) if sg is not None else None, ctypes.byref(sd) if sd is not None else None,
        _ptr(ids), _ptr(gates), _ptr(out), _stream(stream)))
    return ids, gates, out


def moe_combine(Ydown, gates, pos, T: int, topk: int, has_shared: bool, out=None, stream=None):
    import torch
    N = Ydown.shape[1]
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=Ydown.device)
    _check("moe_combine", lib().moe_combine(_ptr(Ydown), _ptr(gates), _ptr(pos), T, topk, N,
                                            1 if has_shared else 0, _ptr(out), _stream(stream)))
    return out


def to_device_w4(W: dict, device) -> dict:
    """Copy a host w4 dict (numpy, as drawn by the input generators) to the
    device as torch tensors.  Pure data movement."""
    import numpy as np
    import torch
    q = np.ascontiguousarray(W["qweight"]).view(np.int32)
    return {"qweight": torch.from_numpy(q).to(device),
            "scales": torch.from_numpy(np.ascontiguousarray(W["scales"])).to(device),
            "biases": torch.from_numpy(np.ascontiguousarray(W["biases"])).to(device),
            "K": int(W["K"]), "N": int(W["N"])}
