"""Thin ctypes binding of libarl2.so (include/arl2.h).

Argument marshalling only: every step of the hybrid attention layer runs in
the library's HIP kernels. torch provides device memory (tensor data
pointers) and streams (torch.cuda.current_stream() unless one is given).
There is no fallback: if libarl2.so is missing or fails to load, importing
this module raises.

Function names mirror the C entry points without the ``arl2_`` prefix.
"""
from __future__ import annotations

import ctypes
import dataclasses
import functools
import os

import torch  # loaded first: libarl2 then binds to the HIP runtime torch carries

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libarl2.so")

# ARL2_ABI_VERSION of include/arl2.h that these signatures follow
ABI_VERSION = 2

F32 = 0
BF16 = 1
OP_READ, OP_CLEAN_PASS, OP_COMMIT, OP_STATE_COMMIT, OP_READ_PREPARED = 0, 1, 2, 3, 4
OP_CLEAN_PASS_PREPARED = 5
OP_TOKEN_LEVEL = 6
OP_INTRA_ATTN_BACKWARD, OP_READ_BACKWARD, OP_COMMIT_BACKWARD = 7, 8, 9

STATUS_NAMES = {
    0: "ARL2_OK", 1: "ARL2_E_NULL", 2: "ARL2_E_SHAPE", 3: "ARL2_E_DTYPE",
    4: "ARL2_E_LAYOUT", 5: "ARL2_E_ALIAS", 6: "ARL2_E_WORKSPACE", 7: "ARL2_E_HIP",
}

# Every entry point the header declares, with its ctypes signature.
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class _Shape(ctypes.Structure):
    _fields_ = [("B", _i32), ("H", _i32), ("T", _i32), ("D", _i32),
                ("act_dtype", _i32), ("softmax_scale", ctypes.c_float)]


_SP = ctypes.POINTER(_Shape)
SIGNATURES = {
    "arl2_feature_map": (_i32, [_SP, _vp, _vp, _vp, _i32, _vp]),
    "arl2_intra_attn": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp]),
    "arl2_intra_attn_lse": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp, _vp]),
    "arl2_inter_read": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp]),
    "arl2_state_commit": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "arl2_read": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "arl2_read_noalloc": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "arl2_commit": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "arl2_clean_pass": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _sz, _vp]),
    "arl2_fullkv_attn": (_i32, [_SP, _vp, _vp, _vp, _i64, _i64, _vp, _vp]),
    "arl2_prepared_bytes": (_sz, [_SP]),
    "arl2_read_prepare": (_i32, [_SP, _vp, _vp, _vp, _vp]),
    "arl2_read_prepared": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "arl2_clean_pass_prepared": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "arl2_token_read": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _sz, _vp]),
    "arl2_token_clean_pass": (_i32, [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp, _sz, _vp]),
    "arl2_intra_attn_backward": (_i32, [_SP] + [_vp] * 9 + [_i32, _vp, _sz, _vp]),
    "arl2_read_backward": (_i32, [_SP] + [_vp] * 13 + [_i32, _vp, _sz, _vp]),
    "arl2_commit_backward": (_i32, [_SP] + [_vp] * 15 + [_i32, _vp, _sz, _vp]),
    "arl2_state_scan": (_i32, [_SP, _i32] + [_vp] * 9 + [_sz, _vp]),
    "arl2_workspace_bytes": (_sz, [_SP, _i32]),
    "arl2_status_string": (ctypes.c_char_p, [_i32]),
    "arl2_last_error": (ctypes.c_char_p, []),
    "arl2_abi_version": (_i32, []),
}


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python -m hybrid_linear_memory_amd.build` "
            "(the ARL2 path has no non-HIP fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    got = lib.arl2_abi_version()
    if got != ABI_VERSION:
        raise ImportError(f"{_LIB_PATH} has ABI version {got}, the binding expects "
                          f"{ABI_VERSION}; rebuild with `python -m hybrid_linear_memory_amd.build`")
    return lib


_lib = _load()


class Arl2Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, f"status {status}")
        super().__init__(f"{self.name}: {detail}")


@dataclasses.dataclass(frozen=True)
class Shape:
    B: int
    H: int
    T: int
    D: int
    act_dtype: int = BF16
    softmax_scale: float = 0.0

    def c(self) -> _Shape:
        # one C struct per Shape object, kept on it (the library only reads it)
        try:
            return self.__dict__["_c"]
        except KeyError:
            c = _c_shape_cached(self)
            object.__setattr__(self, "_c", c)
            return c

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.act_dtype == BF16 else torch.float32


def _check(status: int):
    if status != 0:
        raise Arl2Error(status, _lib.arl2_last_error().decode())


def _ptr(t, name, dtype=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


_ACT = ("q", "k", "v", "o", "o_intra", "o_inter", "x", "x_out", "q_prime", "k_prime", "v_prime",
        "d_o", "dq", "dk", "dv")
_PHI = ("phi", "phi_q", "phi_k", "phi_v", "dphi_q", "dphi_k", "dphi_v")
_STATE = ("S", "S_prev", "S_next", "dS", "dS_next", "dS_prev", "S0", "states")


@functools.lru_cache(maxsize=256)
def _c_shape_cached(shape: "Shape") -> _Shape:
    # one C struct per shape, never modified (the library only reads it)
    return _Shape(shape.B, shape.H, shape.T, shape.D, shape.act_dtype, shape.softmax_scale)


@functools.lru_cache(maxsize=256)
def _sizes(shape: "Shape", frames: int, state_frames: int):
    B, H, T, D = shape.B, shape.H, shape.T, shape.D
    sizes = {}
    sizes.update({n: B * H * T * D * frames for n in _ACT})
    sizes.update({n: H * D * D for n in _PHI})
    sizes.update({n: B * H * D * D * state_frames for n in _STATE})
    sizes.update({"beta": B * H * T * frames, "dbeta": B * H * T, "alpha": B * H * frames,
                  "dalpha": B * H, "lse": B * H * T})
    min_bytes = {"prepared": prepared_bytes(shape), "prepared_next": prepared_bytes(shape)}
    return sizes, min_bytes


def _checker(shape: "Shape", frames: int = 1, state_frames: int = 1):
    """_ptr that also checks each tensor's element count against the shape
    (the library sees only pointers: a short tensor would be read past its
    end). `frames` multiplies the per-frame inputs (k, v, beta, alpha) of a
    multi-frame call, `state_frames` the state-shaped tensors."""
    memo = shape.__dict__.get("_sizes")
    if memo is None:
        memo = {}
        object.__setattr__(shape, "_sizes", memo)
    key = (frames, state_frames)
    got = memo.get(key)
    if got is None:
        got = memo[key] = _sizes(shape, frames, state_frames)
    sizes, min_bytes = got

    def ck(t, name, dtype=None, optional=False):
        ptr = _ptr(t, name, dtype, optional)
        if t is not None:
            want = sizes.get(name)
            if want is not None and t.numel() != want:
                raise ValueError(f"{name} has {t.numel()} elements, the shape needs {want}")
            mb = min_bytes.get(name)
            if mb is not None and t.numel() * t.element_size() < mb:
                raise ValueError(f"{name} has {t.numel() * t.element_size()} bytes, the shape "
                                 f"needs {mb}")
        return ptr
    return ck


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None and _cur_device is not None:
        return _raw_stream(_cur_device())
    return torch.cuda.current_stream().cuda_stream


def abi_version() -> int:
    return _lib.arl2_abi_version()


def status_string(status: int) -> str:
    return _lib.arl2_status_string(status).decode()


def last_error() -> str:
    return _lib.arl2_last_error().decode()


def workspace_bytes(shape: Shape, op: int) -> int:
    return _lib.arl2_workspace_bytes(ctypes.byref(shape.c()), op)


def alloc_workspace(shape: Shape, op: int, device=None) -> torch.Tensor:
    n = max(workspace_bytes(shape, op), 16)
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def feature_map(shape: Shape, x, phi, x_out, normalize_rows=False, stream=None):
    ck = _checker(shape)
    a = shape.torch_dtype
    _check(_lib.arl2_feature_map(ctypes.byref(shape.c()), ck(x, "x", a), ck(phi, "phi", a),
                                 ck(x_out, "x_out", a), int(bool(normalize_rows)),
                                 _stream(stream)))


def intra_attn(shape: Shape, q, k, v, o_intra, stream=None):
    ck = _checker(shape)
    a = shape.torch_dtype
    _check(_lib.arl2_intra_attn(ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a),
                                ck(v, "v", a), ck(o_intra, "o_intra", a), _stream(stream)))


def intra_attn_lse(shape: Shape, q, k, v, o_intra, lse, stream=None):
    """intra_attn, plus each row's log-sum-exp of the scaled scores (natural
    log, float32 [B, H, T]) for the backward calls."""
    ck = _checker(shape)
    a = shape.torch_dtype
    _check(_lib.arl2_intra_attn_lse(ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a),
                                    ck(v, "v", a), ck(o_intra, "o_intra", a),
                                    ck(lse, "lse", torch.float32), _stream(stream)))


def inter_read(shape: Shape, q_prime, S, o_intra, o, stream=None):
    ck = _checker(shape)
    a = shape.torch_dtype
    _check(_lib.arl2_inter_read(ctypes.byref(shape.c()), ck(q_prime, "q_prime", a),
                                ck(S, "S", torch.float32),
                                ck(o_intra, "o_intra", a, optional=True), ck(o, "o", a),
                                _stream(stream)))


def state_commit(shape: Shape, k_prime, v_prime, beta, alpha, S_prev, S_next, ws, stream=None):
    ck = _checker(shape)
    a, f = shape.torch_dtype, torch.float32
    _check(_lib.arl2_state_commit(
        ctypes.byref(shape.c()), ck(k_prime, "k_prime", a), ck(v_prime, "v_prime", a),
        ck(beta, "beta", f), ck(alpha, "alpha", f), ck(S_prev, "S_prev", f),
        ck(S_next, "S_next", f), ck(ws, "ws", optional=True),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def read(shape: Shape, q, k, v, phi_q, S, o, o_intra=None, o_inter=None, ws=None, stream=None):
    ck = _checker(shape)
    a = shape.torch_dtype
    _check(_lib.arl2_read(
        ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a), ck(v, "v", a),
        ck(phi_q, "phi_q", a), ck(S, "S", torch.float32), ck(o, "o", a),
        ck(o_intra, "o_intra", a, optional=True), ck(o_inter, "o_inter", a, optional=True),
        ck(ws, "ws", optional=True), ws.numel() * ws.element_size() if ws is not None else 0,
        _stream(stream)))


# bytes of the library's fixed scratch that arl2_read_noalloc uses
NOALLOC_SCRATCH_BYTES = 8 << 20


def read_noalloc(shape: Shape, q, k, v, phi_q, S, o, o_intra=None, o_inter=None, stream=None):
    """read() without a workspace: the library's fixed device scratch holds
    its intermediates (for callers that cannot allocate)."""
    ck = _checker(shape)
    a = shape.torch_dtype
    _check(_lib.arl2_read_noalloc(
        ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a), ck(v, "v", a),
        ck(phi_q, "phi_q", a), ck(S, "S", torch.float32), ck(o, "o", a),
        ck(o_intra, "o_intra", a, optional=True), ck(o_inter, "o_inter", a, optional=True),
        _stream(stream)))


def prepared_bytes(shape: Shape) -> int:
    return _lib.arl2_prepared_bytes(ctypes.byref(shape.c()))


def alloc_prepared(shape: Shape, device=None) -> torch.Tensor:
    return torch.empty(max(prepared_bytes(shape), 16), dtype=torch.uint8, device=device or "cuda")


def read_prepare(shape: Shape, phi_q, S, prepared, stream=None):
    ck = _checker(shape)
    _check(_lib.arl2_read_prepare(ctypes.byref(shape.c()), ck(phi_q, "phi_q", shape.torch_dtype),
                                  ck(S, "S", torch.float32), ck(prepared, "prepared"),
                                  _stream(stream)))


def read_prepared(shape: Shape, q, k, v, prepared, o, o_intra=None, o_inter=None, ws=None,
                  stream=None):
    ck = _checker(shape)
    a = shape.torch_dtype
    _check(_lib.arl2_read_prepared(
        ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a), ck(v, "v", a),
        ck(prepared, "prepared"), ck(o, "o", a), ck(o_intra, "o_intra", a, optional=True),
        ck(o_inter, "o_inter", a, optional=True), ck(ws, "ws", optional=True),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def clean_pass_prepared(shape: Shape, q, k, v, prepared, phi_k, phi_v, beta, alpha, S_prev,
                        S_next, o, o_intra=None, o_inter=None, ws=None, stream=None, phi_q=None,
                        prepared_next=None):
    ck = _checker(shape)
    a, f = shape.torch_dtype, torch.float32
    _check(_lib.arl2_clean_pass_prepared(
        ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a), ck(v, "v", a),
        ck(prepared, "prepared"), ck(phi_q, "phi_q", a, optional=True),
        ck(phi_k, "phi_k", a), ck(phi_v, "phi_v", a), ck(beta, "beta", f),
        ck(alpha, "alpha", f), ck(S_prev, "S_prev", f), ck(S_next, "S_next", f),
        ck(prepared_next, "prepared_next", optional=True), ck(o, "o", a),
        ck(o_intra, "o_intra", a, optional=True), ck(o_inter, "o_inter", a, optional=True),
        ck(ws, "ws", optional=True), ws.numel() * ws.element_size() if ws is not None else 0,
        _stream(stream)))


def commit(shape: Shape, k, v, phi_k, phi_v, beta, alpha, S_prev, S_next, ws, stream=None):
    ck = _checker(shape)
    a, f = shape.torch_dtype, torch.float32
    _check(_lib.arl2_commit(
        ctypes.byref(shape.c()), ck(k, "k", a), ck(v, "v", a), ck(phi_k, "phi_k", a),
        ck(phi_v, "phi_v", a), ck(beta, "beta", f), ck(alpha, "alpha", f),
        ck(S_prev, "S_prev", f), ck(S_next, "S_next", f), ck(ws, "ws", optional=True),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def clean_pass(shape: Shape, q, k, v, phi_q, phi_k, phi_v, beta, alpha, S_prev, S_next, o,
               o_intra=None, o_inter=None, ws=None, stream=None):
    ck = _checker(shape)
    a, f = shape.torch_dtype, torch.float32
    _check(_lib.arl2_clean_pass(
        ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a), ck(v, "v", a),
        ck(phi_q, "phi_q", a), ck(phi_k, "phi_k", a), ck(phi_v, "phi_v", a),
        ck(beta, "beta", f), ck(alpha, "alpha", f), ck(S_prev, "S_prev", f),
        ck(S_next, "S_next", f), ck(o, "o", a), ck(o_intra, "o_intra", a, optional=True),
        ck(o_inter, "o_inter", a, optional=True), ck(ws, "ws", optional=True),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def token_read(shape: Shape, q, k, v, phi_q, phi_k, phi_v, beta, S, o, o_intra=None,
               o_inter=None, ws=None, stream=None):
    """Read under token-level access (token t sees the frame's earlier tokens)."""
    ck = _checker(shape)
    a, f = shape.torch_dtype, torch.float32
    _check(_lib.arl2_token_read(
        ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a), ck(v, "v", a),
        ck(phi_q, "phi_q", a), ck(phi_k, "phi_k", a), ck(phi_v, "phi_v", a),
        ck(beta, "beta", f), ck(S, "S", f), ck(o, "o", a),
        ck(o_intra, "o_intra", a, optional=True), ck(o_inter, "o_inter", a, optional=True),
        ck(ws, "ws", optional=True), ws.numel() * ws.element_size() if ws is not None else 0,
        _stream(stream)))


def token_clean_pass(shape: Shape, q, k, v, phi_q, phi_k, phi_v, beta, alpha, S_prev, S_next, o,
                     o_intra=None, o_inter=None, ws=None, stream=None):
    """Clean pass under token-level access: the read, then S_next from its end state."""
    ck = _checker(shape)
    a, f = shape.torch_dtype, torch.float32
    _check(_lib.arl2_token_clean_pass(
        ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a), ck(v, "v", a),
        ck(phi_q, "phi_q", a), ck(phi_k, "phi_k", a), ck(phi_v, "phi_v", a),
        ck(beta, "beta", f), ck(alpha, "alpha", f), ck(S_prev, "S_prev", f),
        ck(S_next, "S_next", f), ck(o, "o", a), ck(o_intra, "o_intra", a, optional=True),
        ck(o_inter, "o_inter", a, optional=True), ck(ws, "ws", optional=True),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def _ws(ws):
    return _ptr(ws, "ws", optional=True), ws.numel() * ws.element_size() if ws is not None else 0


def intra_attn_backward(shape: Shape, q, k, v, o_intra, d_o, dq, dk, dv, accumulate=False,
                        ws=None, stream=None, lse=None):
    """dq, dk, dv of the intra-frame softmax from its output o_intra and
    dL/dO_intra (lse: the rows' log-sum-exp from intra_attn_lse, or None)."""
    ck = _checker(shape)
    a = shape.torch_dtype
    _check(_lib.arl2_intra_attn_backward(
        ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a), ck(v, "v", a),
        ck(o_intra, "o_intra", a), ck(lse, "lse", torch.float32, optional=True),
        ck(d_o, "d_o", a), ck(dq, "dq", a), ck(dk, "dk", a), ck(dv, "dv", a),
        1 if accumulate else 0, *_ws(ws), _stream(stream)))


def read_backward(shape: Shape, q, k, v, phi_q, S, o_intra, d_o, dq, dk, dv, dphi_q, dS,
                  accumulate=False, ws=None, stream=None, lse=None):
    """Gradients of a read O = O_intra + (Q Phi_q) S given dL/dO (lse: the
    rows' log-sum-exp from intra_attn_lse, or None)."""
    ck = _checker(shape)
    a, f = shape.torch_dtype, torch.float32
    _check(_lib.arl2_read_backward(
        ctypes.byref(shape.c()), ck(q, "q", a), ck(k, "k", a), ck(v, "v", a),
        ck(phi_q, "phi_q", a), ck(S, "S", f), ck(o_intra, "o_intra", a),
        ck(lse, "lse", f, optional=True),
        ck(d_o, "d_o", a), ck(dq, "dq", a), ck(dk, "dk", a), ck(dv, "dv", a),
        ck(dphi_q, "dphi_q", f), ck(dS, "dS", f), 1 if accumulate else 0, *_ws(ws),
        _stream(stream)))


def commit_backward(shape: Shape, k, v, phi_k, phi_v, beta, alpha, S_prev, dS_next, dk, dv,
                    dphi_k, dphi_v, dbeta, dalpha, dS_prev, accumulate=False, ws=None,
                    stream=None):
    """Gradients of the commit given dL/dS_next."""
    ck = _checker(shape)
    a, f = shape.torch_dtype, torch.float32
    _check(_lib.arl2_commit_backward(
        ctypes.byref(shape.c()), ck(k, "k", a), ck(v, "v", a), ck(phi_k, "phi_k", a),
        ck(phi_v, "phi_v", a), ck(beta, "beta", f), ck(alpha, "alpha", f),
        ck(S_prev, "S_prev", f), ck(dS_next, "dS_next", f), ck(dk, "dk", a),
        ck(dv, "dv", a), ck(dphi_k, "dphi_k", f), ck(dphi_v, "dphi_v", f),
        ck(dbeta, "dbeta", f), ck(dalpha, "dalpha", f), ck(dS_prev, "dS_prev", f),
        1 if accumulate else 0, *_ws(ws), _stream(stream)))


def state_scan(shape: Shape, k, v, phi_k, phi_v, beta, alpha, S0, states, ws=None, stream=None):
    """states[0] = S0 and states[f + 1] = the commit of frame f (k, v: [F, B, H, T, D])."""
    ck = _checker(shape, frames=int(k.shape[0]), state_frames=int(k.shape[0]) + 1)
    a, f = shape.torch_dtype, torch.float32
    n_frames = int(k.shape[0])
    if tuple(states.shape[:1]) != (n_frames + 1,):
        raise ValueError("states needs n_frames + 1 entries")
    _check(_lib.arl2_state_scan(
        ctypes.byref(shape.c()), n_frames, ck(k, "k", a), ck(v, "v", a),
        ck(phi_k, "phi_k", a), ck(phi_v, "phi_v", a), ck(beta, "beta", f),
        ck(alpha, "alpha", f), _checker(shape)(S0, "S0", f), ck(states, "states", f), *_ws(ws),
        _stream(stream)))


def fullkv_attn(shape: Shape, q, k_cache, v_cache, n_kv: int, o, stream=None):
    ck = _checker(shape)
    a = shape.torch_dtype
    cap = k_cache.shape[2]
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache shapes differ")
    _check(_lib.arl2_fullkv_attn(ctypes.byref(shape.c()), ck(q, "q", a),
                                 ck(k_cache, "k_cache", a), ck(v_cache, "v_cache", a),
                                 int(n_kv), int(cap), ck(o, "o", a), _stream(stream)))


def raw_call(name: str, *args):
    """Call an entry point with raw ctypes arguments and return its status
    (used by the ABI error-path tests)."""
    return getattr(_lib, name)(*args)


def c_shape(shape: Shape):
    return ctypes.byref(shape.c())
