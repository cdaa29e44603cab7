"""ctypes binding of libcf.so: argument marshalling only.

Every function here has the name of the C entry point it calls and forwards
device pointers, sizes and the HIP stream.  All arithmetic runs in the HIP
kernels; there is no CPU fallback: if the library is missing or fails to
load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcf.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "cf.h")
HEADER_PATHS = [HEADER_PATH, os.path.join(os.path.dirname(_HERE), "include", "cf_spec.h")]

CF_OK, CF_EINVAL, CF_EUNSUPPORTED, CF_EALIGN, CF_EWORKSPACE, CF_EOCCUPANCY, CF_EHIP = range(7)
(CF_OP_STITCH_SOFTMAX, CF_OP_STITCH_LAYERNORM, CF_OP_STITCH_POW_BCAST_ADD, CF_OP_GEMM_LN, CF_OP_GEMM_SOFTMAX,
 CF_OP_GEMM_SOFTMAX_GEMM, CF_OP_STITCH_LAYERNORM_AFFINE, CF_OP_STITCH_RMSNORM, CF_OP_GEMM_ACT) = range(1, 10)
CF_ACT_NONE, CF_ACT_RELU, CF_ACT_GELU_TANH, CF_ACT_SILU, CF_ACT_SQUARE, CF_ACT_RSQRT = range(6)
ACT_IDS = {"none": CF_ACT_NONE, "relu": CF_ACT_RELU, "gelu_tanh": CF_ACT_GELU_TANH, "silu": CF_ACT_SILU,
           "square": CF_ACT_SQUARE, "rsqrt": CF_ACT_RSQRT}

_lib = None
_lock = threading.Lock()

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_ST = ctypes.c_int

class GNode(ctypes.Structure):
    """cf_gnode: one node of a captured graph (include/cf_spec.h)."""
    _fields_ = [("op", ctypes.c_int32), ("in0", ctypes.c_int32), ("in1", ctypes.c_int32),
                ("attr", ctypes.c_int32), ("slot", ctypes.c_int32), ("value", ctypes.c_double)]


# cf_gop codes by name
G_OPS = {name: i for i, name in enumerate(
    ["input", "operand", "matmul", "rowvec", "colvec", "tensor", "const", "add", "sub", "mul", "div", "pow",
     "exp", "square", "rsqrt", "relu", "gelu_tanh", "silu", "rowsum", "rowmax"])}

_SIGS = {
    "cf_workspace_bytes": (_SZ, [ctypes.c_int, _I64, _I64, _I64]),
    "cf_unfused_workspace_bytes": (_SZ, [ctypes.c_int, _I64, _I64, _I64]),
    "cf_status_str": (ctypes.c_char_p, [_ST]),
    "cf_last_plan": (ctypes.c_int, [ctypes.c_char_p, _SZ]),
    "cf_stitch_softmax": (_ST, [_P, _P, _I64, _I64, _P, _SZ, _P]),
    "cf_stitch_layernorm": (_ST, [_P, _P, _I64, _I64, _F, _P, _SZ, _P]),
    "cf_stitch_pow_bcast_add": (_ST, [_P, _P, _F, _P, _P, _I64, _I64, _P, _SZ, _P]),
    "cf_stitch_layernorm_affine": (_ST, [_P, _P, _P, _P, _I64, _I64, _F, _P, _SZ, _P]),
    "cf_stitch_rmsnorm": (_ST, [_P, _P, _P, _I64, _I64, _F, _P, _SZ, _P]),
    "cf_gemm_ln": (_ST, [_P, _P, _P, _P, _P, _P, _F, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "cf_gemm_ln_noalloc": (_ST, [_P, _P, _P, _P, _P, _P, _F, _P, _I64, _I64, _I64, _P]),
    "cf_workspace_error": (_ST, [_P, ctypes.c_int, ctypes.POINTER(ctypes.c_uint32), _P]),
    "cf_gemm_softmax": (_ST, [_P, _P, _F, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "cf_gemm_softmax_gemm": (_ST, [_P, _P, _P, _F, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P]),
    "cf_gemm_act": (_ST, [_P, _P, _P, ctypes.c_int, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "cf_unfused_stitch_softmax": (_ST, [_P, _P, _I64, _I64, _P, _SZ, _P]),
    "cf_unfused_stitch_layernorm": (_ST, [_P, _P, _I64, _I64, _F, _P, _SZ, _P]),
    "cf_unfused_stitch_pow_bcast_add": (_ST, [_P, _P, _F, _P, _P, _I64, _I64, _P, _SZ, _P]),
    "cf_unfused_stitch_layernorm_affine": (_ST, [_P, _P, _P, _P, _I64, _I64, _F, _P, _SZ, _P]),
    "cf_unfused_stitch_rmsnorm": (_ST, [_P, _P, _P, _I64, _I64, _F, _P, _SZ, _P]),
    "cf_unfused_gemm_ln": (_ST, [_P, _P, _P, _P, _P, _P, _F, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "cf_unfused_gemm_softmax": (_ST, [_P, _P, _F, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "cf_unfused_gemm_softmax_gemm": (_ST, [_P, _P, _P, _F, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P]),
    "cf_unfused_gemm_act": (_ST, [_P, _P, _P, ctypes.c_int, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "cf_graph_begin": (_ST, [_P]),
    "cf_graph_end": (_ST, [_P, ctypes.POINTER(_P)]),
    "cf_graph_launch": (_ST, [_P, _P]),
    "cf_graph_destroy": (_ST, [_P]),
    "cf_util_fill_f32": (_ST, [_P, _I64, _F, _P]),
    "cf_util_copy_f32": (_ST, [_P, _P, _I64, _P]),
    "cf_spec_build": (_ST, [ctypes.POINTER(GNode), ctypes.c_int, ctypes.c_int, _I64, _I64, _I64,
                            ctypes.POINTER(_P)]),
    "cf_spec_describe": (ctypes.c_int, [_P, ctypes.c_char_p, _SZ]),
    "cf_spec_workspace_bytes": (_SZ, [_P]),
    "cf_spec_launch": (_ST, [_P, ctypes.POINTER(_P), ctypes.c_int, _P, _P, _SZ, _P]),
    "cf_spec_free": (None, [_P]),
    "cf_auto_build": (_ST, [ctypes.POINTER(GNode), ctypes.c_int, ctypes.c_int, _I64, _I64, ctypes.POINTER(_P)]),
    "cf_auto_describe": (ctypes.c_int, [_P, ctypes.c_char_p, _SZ]),
    "cf_auto_source": (ctypes.c_int, [_P, ctypes.c_char_p, _SZ]),
    "cf_auto_launch": (_ST, [_P, ctypes.POINTER(_P), ctypes.c_int, _P, _P, _SZ, _P]),
    "cf_auto_workspace_bytes": (_SZ, [_P]),
    "cf_auto_free": (None, [_P]),
}


class CFError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call} failed: {status_str(status)}")


def header_functions() -> list[str]:
    """Names of every function the C headers declare."""
    txt = ""
    for path in HEADER_PATHS:
        with open(path) as f:
            txt += f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(cf_[a-z0-9_]+)\s*\(", txt)))


def lib() -> ctypes.CDLL:
    """Load libcf.so once; raise if it is missing (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m broadcast_subgraphs_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().cf_status_str(int(status)).decode()


def last_plan() -> str:
    buf = ctypes.create_string_buffer(1024)
    lib().cf_last_plan(buf, 1024)
    return buf.value.decode()


def _check(name: str, status: int) -> None:
    if status != CF_OK:
        raise CFError(name, status)


# ----------------------------------------------------------------- torch glue
# PyTorch only supplies device memory and the stream.

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _need(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


class Workspace:
    """A caller-owned device workspace, zero-filled once at allocation."""

    def __init__(self, nbytes: int, device=None):
        torch = _torch()
        self.nbytes = max(int(nbytes), 256)
        self.buf = torch.zeros(self.nbytes, dtype=torch.uint8, device=device or "cuda")
        torch.cuda.synchronize(self.buf.device)

    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr())

    def error_word(self) -> int:
        """Non-zero if a cross-workgroup wait gave up (read after the stream finished)."""
        return int(self.buf[:4].view(_torch().int32).item())

    def clear_error(self) -> None:
        self.buf[:4].zero_()


def cf_workspace_error(ws, clear=False, stream=None) -> int:
    """The workspace's error word through the C-ABI (waits for the stream); non-zero: a
    cross-workgroup wait of a call that used it gave up and that call's output is wrong."""
    out = ctypes.c_uint32(0)
    _check("cf_workspace_error", lib().cf_workspace_error(ws.ptr(), 1 if clear else 0, ctypes.byref(out),
                                                          _stream(stream)))
    return int(out.value)


_ws_cache: dict = {}


def _workspace(nbytes: int, device, stream) -> Workspace:
    if nbytes == 0:
        return None
    key = (device.index, int(stream.value or 0))
    ws = _ws_cache.get(key)
    if ws is None or ws.nbytes < nbytes:
        ws = Workspace(nbytes, device)
        _ws_cache[key] = ws
    return ws


def _ws_args(op, d0, d1, d2, ws, device, stream, unfused=False):
    L = lib()
    nbytes = (L.cf_unfused_workspace_bytes if unfused else L.cf_workspace_bytes)(op, d0, d1, d2)
    if nbytes == ctypes.c_size_t(-1).value:
        raise CFError("cf_workspace_bytes" if not unfused else "cf_unfused_workspace_bytes", CF_EUNSUPPORTED)
    if ws is None:
        ws = _workspace(nbytes, device, stream)
    if ws is None:
        return None, 0, None
    return ws.ptr(), ws.nbytes, ws


# ----------------------------------------------------------------- entry points

def cf_stitch_softmax(x, y, ws=None, stream=None, unfused=False):
    torch = _torch()
    _need(x, torch.float32, "x", 2)
    _need(y, torch.float32, "y", 2)
    rows, cols = x.shape
    st = _stream(stream)
    p, n, w = _ws_args(CF_OP_STITCH_SOFTMAX, rows, cols, 0, ws, x.device, st, unfused)
    name = "cf_unfused_stitch_softmax" if unfused else "cf_stitch_softmax"
    _check(name, getattr(lib(), name)(_ptr(x), _ptr(y), rows, cols, p, n, st))
    return w


def cf_stitch_layernorm(x, y, eps=1e-5, ws=None, stream=None, unfused=False):
    torch = _torch()
    _need(x, torch.float32, "x", 2)
    _need(y, torch.float32, "y", 2)
    rows, cols = x.shape
    st = _stream(stream)
    p, n, w = _ws_args(CF_OP_STITCH_LAYERNORM, rows, cols, 0, ws, x.device, st, unfused)
    name = "cf_unfused_stitch_layernorm" if unfused else "cf_stitch_layernorm"
    _check(name, getattr(lib(), name)(_ptr(x), _ptr(y), rows, cols, float(eps), p, n, st))
    return w


def cf_stitch_pow_bcast_add(x, v, p, y, y_pre=None, ws=None, stream=None, unfused=False):
    torch = _torch()
    _need(x, torch.float32, "x", 2)
    _need(v, torch.float32, "v", 1)
    _need(y, torch.float32, "y", 2)
    if y_pre is not None:
        _need(y_pre, torch.float32, "y_pre", 2)
    rows, cols = x.shape
    st = _stream(stream)
    wp, n, w = _ws_args(CF_OP_STITCH_POW_BCAST_ADD, rows, cols, 0, ws, x.device, st, unfused)
    name = "cf_unfused_stitch_pow_bcast_add" if unfused else "cf_stitch_pow_bcast_add"
    _check(name, getattr(lib(), name)(_ptr(x), _ptr(v), float(p), _ptr(y), _ptr(y_pre), rows, cols, wp, n, st))
    return w


def cf_gemm_ln(A, W, bias, R, gamma, beta, Y, eps=1e-5, ws=None, stream=None, unfused=False):
    """A [M,K], W [K,N], R [M,N] or None, Y [M,N]: bf16 tensors; bias/gamma/beta fp32 [N]."""
    torch = _torch()
    for t, nm in ((A, "A"), (W, "W"), (Y, "Y")):
        _need(t, torch.bfloat16, nm, 2)
    if R is not None:
        _need(R, torch.bfloat16, "R", 2)
    for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        _need(t, torch.float32, nm, 1)
    M, K = A.shape
    N = W.shape[1]
    st = _stream(stream)
    p, n, w = _ws_args(CF_OP_GEMM_LN, M, N, K, ws, A.device, st, unfused)
    name = "cf_unfused_gemm_ln" if unfused else "cf_gemm_ln"
    _check(name, getattr(lib(), name)(_ptr(A), _ptr(W), _ptr(bias), _ptr(R), _ptr(gamma), _ptr(beta),
                                      float(eps), _ptr(Y), M, N, K, p, n, st))
    return w


def cf_gemm_ln_noalloc(A, W, bias, R, gamma, beta, Y, eps=1e-5, stream=None):
    """cf_gemm_ln with its workspace in the library's static scratch (nothing allocated)."""
    torch = _torch()
    for t, nm in ((A, "A"), (W, "W"), (Y, "Y")):
        _need(t, torch.bfloat16, nm, 2)
    if R is not None:
        _need(R, torch.bfloat16, "R", 2)
    for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        _need(t, torch.float32, nm, 1)
    M, K = A.shape
    N = W.shape[1]
    _check("cf_gemm_ln_noalloc", lib().cf_gemm_ln_noalloc(_ptr(A), _ptr(W), _ptr(bias), _ptr(R), _ptr(gamma),
                                                          _ptr(beta), float(eps), _ptr(Y), M, N, K,
                                                          _stream(stream)))


def cf_gemm_softmax(Q, K, scale, S, ws=None, stream=None, unfused=False):
    """Q [M,D], K [N,D], S [M,N]: bf16 tensors."""
    torch = _torch()
    for t, nm in ((Q, "Q"), (K, "K"), (S, "S")):
        _need(t, torch.bfloat16, nm, 2)
    M, D = Q.shape
    N = K.shape[0]
    st = _stream(stream)
    p, n, w = _ws_args(CF_OP_GEMM_SOFTMAX, M, N, D, ws, Q.device, st, unfused)
    name = "cf_unfused_gemm_softmax" if unfused else "cf_gemm_softmax"
    _check(name, getattr(lib(), name)(_ptr(Q), _ptr(K), float(scale), _ptr(S), M, N, D, p, n, st))
    return w


def cf_stitch_layernorm_affine(x, gamma, beta, y, eps=1e-5, ws=None, stream=None, unfused=False):
    """x, y [rows, cols], gamma, beta [cols]: fp32 tensors; y = LayerNorm(x) * gamma + beta."""
    torch = _torch()
    _need(x, torch.float32, "x", 2)
    _need(y, torch.float32, "y", 2)
    _need(gamma, torch.float32, "gamma", 1)
    _need(beta, torch.float32, "beta", 1)
    rows, cols = x.shape
    st = _stream(stream)
    p, n, w = _ws_args(CF_OP_STITCH_LAYERNORM_AFFINE, rows, cols, 0, ws, x.device, st, unfused)
    name = "cf_unfused_stitch_layernorm_affine" if unfused else "cf_stitch_layernorm_affine"
    _check(name, getattr(lib(), name)(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), rows, cols, float(eps), p, n, st))
    return w


def cf_stitch_rmsnorm(x, gamma, y, eps=1e-5, ws=None, stream=None, unfused=False):
    """x, y [rows, cols] fp32, gamma [cols] fp32 or None (gain 1); y = x * rsqrt(mean(x^2) + eps) * gamma."""
    torch = _torch()
    _need(x, torch.float32, "x", 2)
    _need(y, torch.float32, "y", 2)
    if gamma is not None:
        _need(gamma, torch.float32, "gamma", 1)
    rows, cols = x.shape
    st = _stream(stream)
    p, n, w = _ws_args(CF_OP_STITCH_RMSNORM, rows, cols, 0, ws, x.device, st, unfused)
    name = "cf_unfused_stitch_rmsnorm" if unfused else "cf_stitch_rmsnorm"
    _check(name, getattr(lib(), name)(_ptr(x), _ptr(gamma), _ptr(y), rows, cols, float(eps), p, n, st))
    return w


def cf_gemm_softmax_gemm(Q, K, V, scale, O, ws=None, stream=None, unfused=False):
    """Q [M,D], K [N,D], V [N,Dv], O [M,Dv]: bf16 tensors; O = softmax(scale * Q.K^T).V."""
    torch = _torch()
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V"), (O, "O")):
        _need(t, torch.bfloat16, nm, 2)
    M, D = Q.shape
    N, Dv = V.shape
    st = _stream(stream)
    p, n, w = _ws_args(CF_OP_GEMM_SOFTMAX_GEMM, M, N, D, ws, Q.device, st, unfused)
    name = "cf_unfused_gemm_softmax_gemm" if unfused else "cf_gemm_softmax_gemm"
    _check(name, getattr(lib(), name)(_ptr(Q), _ptr(K), _ptr(V), float(scale), _ptr(O), M, N, D, Dv, p, n, st))
    return w


def cf_gemm_act(A, W, bias, act, Y, ws=None, stream=None, unfused=False):
    """A [M,K], W [K,N], Y [M,N]: bf16 tensors; bias fp32 [N] or None; act a CF_ACT_* id or its name."""
    torch = _torch()
    for t, nm in ((A, "A"), (W, "W"), (Y, "Y")):
        _need(t, torch.bfloat16, nm, 2)
    if bias is not None:
        _need(bias, torch.float32, "bias", 1)
    act_id = ACT_IDS[act] if isinstance(act, str) else int(act)
    M, K = A.shape
    N = W.shape[1]
    st = _stream(stream)
    p, n, w = _ws_args(CF_OP_GEMM_ACT, M, N, K, ws, A.device, st, unfused)
    name = "cf_unfused_gemm_act" if unfused else "cf_gemm_act"
    _check(name, getattr(lib(), name)(_ptr(A), _ptr(W), _ptr(bias), act_id, _ptr(Y), M, N, K, p, n, st))
    return w


def cf_workspace_bytes(op, d0, d1, d2=0):
    return lib().cf_workspace_bytes(op, d0, d1, d2)


def cf_unfused_workspace_bytes(op, d0, d1, d2=0):
    return lib().cf_unfused_workspace_bytes(op, d0, d1, d2)


def cf_graph_begin(stream=None):
    _check("cf_graph_begin", lib().cf_graph_begin(_stream(stream)))


def cf_graph_end(stream=None):
    h = ctypes.c_void_p()
    _check("cf_graph_end", lib().cf_graph_end(_stream(stream), ctypes.byref(h)))
    return h


def cf_graph_launch(exec_handle, stream=None):
    _check("cf_graph_launch", lib().cf_graph_launch(exec_handle, _stream(stream)))


def cf_graph_destroy(exec_handle):
    _check("cf_graph_destroy", lib().cf_graph_destroy(exec_handle))


def cf_util_fill_f32(p, value=0.0, stream=None):
    _check("cf_util_fill_f32", lib().cf_util_fill_f32(_ptr(p), p.numel(), float(value), _stream(stream)))


def cf_util_copy_f32(src, dst, stream=None):
    _check("cf_util_copy_f32", lib().cf_util_copy_f32(_ptr(src), _ptr(dst), src.numel(), _stream(stream)))


# ------------------------------------------------------------- Fusion Spec IR

class Graph:
    """A captured graph as plain node tuples (op name, in0, in1, attr, slot, value).

    Each builder method appends one node and returns its index.  Placeholders
    name the slot of their tensor in the argument list given at launch."""

    def __init__(self):
        self.nodes = []

    def _add(self, op, a=-1, b=-1, attr=0, slot=-1, value=0.0):
        self.nodes.append((op, a, b, attr, slot, float(value)))
        return len(self.nodes) - 1

    def input(self, slot):
        return self._add("input", slot=slot)

    def operand(self, slot):
        return self._add("operand", slot=slot)

    def rowvec(self, slot):
        return self._add("rowvec", slot=slot)

    def colvec(self, slot):
        return self._add("colvec", slot=slot)

    def tensor(self, slot):
        return self._add("tensor", slot=slot)

    def const(self, value):
        return self._add("const", value=value)

    def matmul(self, a, b, nt=False):
        return self._add("matmul", a, b, attr=1 if nt else 0)

    def op(self, name, a, b=-1):
        return self._add(name, a, b)


class Spec:
    """cf_spec_build over a Graph; launch() enqueues the kernel it matched."""

    def __init__(self, graph, terminal, rows, cols, k=0):
        """graph: a Graph, or a list of its node tuples."""
        nodes = graph.nodes if hasattr(graph, "nodes") else list(graph)
        arr = (GNode * max(1, len(nodes)))()
        for i, (op, a, b, attr, slot, value) in enumerate(nodes):
            arr[i] = GNode(G_OPS[op], a, b, attr, slot, value)
        h = _P()
        self._h = None
        _check("cf_spec_build", lib().cf_spec_build(arr, len(nodes), terminal, rows, cols, k, ctypes.byref(h)))
        self._h = h

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.cf_spec_free(self._h)
            self._h = None

    def describe(self) -> dict:
        import json
        n = lib().cf_spec_describe(self._h, None, 0)
        buf = ctypes.create_string_buffer(n + 1)
        lib().cf_spec_describe(self._h, buf, n + 1)
        return json.loads(buf.value.decode())

    def workspace_bytes(self) -> int:
        return int(lib().cf_spec_workspace_bytes(self._h))

    def launch(self, args, out, ws=None, stream=None):
        """args: tensors by slot (None where unused); out: the output tensor."""
        st = _stream(stream)
        nb = self.workspace_bytes()
        if nb == ctypes.c_size_t(-1).value:
            raise CFError("cf_spec_workspace_bytes", CF_EUNSUPPORTED)
        if ws is None:
            ws = _workspace(nb, out.device, st)
        ptrs = (_P * max(1, len(args)))(*[None if t is None else t.data_ptr() for t in args])
        _check("cf_spec_launch", lib().cf_spec_launch(self._h, ptrs, len(args), _ptr(out),
                                                      None if ws is None else ws.ptr(),
                                                      0 if ws is None else ws.nbytes, st))
        return ws


def _gnodes(graph):
    nodes = graph.nodes if hasattr(graph, "nodes") else list(graph)
    arr = (GNode * max(1, len(nodes)))()
    for i, (op, a, b, attr, slot, value) in enumerate(nodes):
        arr[i] = GNode(G_OPS[op], a, b, attr, slot, value)
    return arr, len(nodes)


class Auto:
    """cf_auto_build over a Graph (or its node tuples): a generated stitched kernel."""

    def __init__(self, graph, terminal, rows, cols):
        arr, n = _gnodes(graph)
        h = _P()
        self._h = None
        _check("cf_auto_build", lib().cf_auto_build(arr, n, terminal, rows, cols, ctypes.byref(h)))
        self._h = h

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.cf_auto_free(self._h)
            self._h = None

    def _text(self, fn) -> str:
        n = fn(self._h, None, 0)
        buf = ctypes.create_string_buffer(n + 1)
        fn(self._h, buf, n + 1)
        return buf.value.decode()

    def describe(self) -> dict:
        import json
        return json.loads(self._text(lib().cf_auto_describe))

    def source(self) -> str:
        return self._text(lib().cf_auto_source)

    def workspace_bytes(self) -> int:
        return int(lib().cf_auto_workspace_bytes(self._h))

    def launch(self, args, out, ws=None, stream=None, check=False):
        """args: fp32 tensors by slot (None where unused); out: fp32 [rows, cols].  A workspace is
        allocated and cached when the kernel needs one and none is given; returns it.  With
        check=True the call waits for the stream and raises CFError(CF_EOCCUPANCY) if a
        cross-workgroup wait gave up (its members were not all resident), clearing the word."""
        st = _stream(stream)
        nb = self.workspace_bytes()
        if nb == ctypes.c_size_t(-1).value:
            raise CFError("cf_auto_workspace_bytes", CF_EHIP)
        if ws is None:
            ws = _workspace(nb, out.device, st)
        ptrs = (_P * max(1, len(args)))(*[None if t is None else t.data_ptr() for t in args])
        _check("cf_auto_launch", lib().cf_auto_launch(self._h, ptrs, len(args), _ptr(out),
                                                      None if ws is None else ws.ptr(),
                                                      0 if ws is None else ws.nbytes, st))
        if check and ws is not None and cf_workspace_error(ws, clear=True, stream=st.value) != 0:
            raise CFError("cf_auto_launch", CF_EOCCUPANCY)
        return ws
