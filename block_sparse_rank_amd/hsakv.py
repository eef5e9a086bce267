"""ctypes binding of libhsakv.so: the C ABI of include/hsakv.h, same names.

Argument marshalling only. Tensors are torch tensors (device memory and the
current stream are the only things taken from torch); each entry point
passes `tensor.data_ptr()` and the current HIP stream and raises HsakvError
on a non-zero status. Every step of the path runs in the library's HIP
kernels; there is no fallback of any kind: if the library is missing, the
import of this module fails.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhsakv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m block_sparse_rank_amd.build` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

c_int32 = ctypes.c_int32
c_void_p = ctypes.c_void_p
c_size_t = ctypes.c_size_t

# status codes and constants (include/hsakv.h)
OK = 0
ERR_NULL_ARG = -1
ERR_BAD_DIMS = -2
ERR_BAD_DTYPE = -3
ERR_BAD_TAU = -4
ERR_WORKSPACE = -5
ERR_MISALIGNED = -6
ERR_HIP = -7
ERR_UNSUPPORTED = -8
F32 = 0
BF16 = 1
ENTRY_GATHER = 1
ENTRY_SELECT = 2
ENTRY_SPARSE = 3
ENTRY_LINEAR = 4
ENTRY_FORWARD = 6

EXPORTS = [
    "hsakv_version", "hsakv_status_str", "hsakv_last_hip_error", "hsakv_validate",
    "hsakv_workspace_bytes", "hkv_page_summary", "hkv_gather", "hsa_select", "hsa_sparse_attn",
    "hsa_linear_branch", "hsa_fuse", "hsa_forward",
]


class Dims(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "H", "d", "Lq", "tokens_per_frame", "Psize", "P", "Kp", "Binter", "Bintra", "Bq", "r",
        "dtype")]

    @property
    def Tp(self) -> int:
        return self.Psize * self.tokens_per_frame

    @property
    def NQB(self) -> int:
        return -(-self.Lq // self.Bq)

    @property
    def NBc(self) -> int:
        return -(-self.Lq // self.Bintra)

    @property
    def NB_max(self) -> int:
        return -(-(self.Kp * self.Tp) // self.Binter) + self.NBc

    @property
    def L(self) -> int:
        return self.Kp * self.Tp + self.Lq


class Inputs(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "q", "k_intra", "v_intra", "pool_k", "pool_v", "page_kmean", "page_prompt", "E", "F",
        "w_g", "b_g")]


class Outputs(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "out", "page_idx", "n_sel", "k_hist", "v_hist", "sel_count", "sel_idx", "o_sparse",
        "o_linear", "gate")]


_P = c_void_p
_D = ctypes.POINTER(Dims)
_sig = {
    "hsakv_version": (c_int32, []),
    "hsakv_status_str": (ctypes.c_char_p, [c_int32]),
    "hsakv_last_hip_error": (c_int32, []),
    "hsakv_validate": (c_int32, [_D]),
    "hsakv_workspace_bytes": (c_size_t, [_D, c_int32]),
    "hkv_page_summary": (c_int32, [_D, _P, _P, _P]),
    "hkv_gather": (c_int32, [_D, _P, _P, _P, _P, c_int32, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "hsa_select": (c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "hsa_sparse_attn": (c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "hsa_linear_branch": (c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "hsa_fuse": (c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P]),
    "hsa_forward": (c_int32, [_D, _P, c_int32, ctypes.POINTER(Inputs), ctypes.POINTER(Outputs), _P,
                              c_size_t, _P]),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class HsakvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        hip = _lib.hsakv_last_hip_error() if status == ERR_HIP else 0
        msg = f"{fn}: {status_str(status)} ({status})"
        if hip:
            msg += f", hipError {hip}"
        super().__init__(msg)
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise HsakvError(fn, status)


def _ptr(t) -> Optional[int]:
    """Device (or host) address of a tensor, an int address, or None for NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _host_f32(x) -> ctypes.Array:
    vals = [float(v) for v in (x.tolist() if hasattr(x, "tolist") else x)]
    return (ctypes.c_float * len(vals))(*vals)


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


# ---- helpers -----------------------------------------------------------------

def version() -> int:
    return _lib.hsakv_version()


def status_str(status: int) -> str:
    return _lib.hsakv_status_str(status).decode()


def validate(dims: Dims) -> int:
    return _lib.hsakv_validate(ctypes.byref(dims))


def workspace_bytes(dims: Dims, entry: int) -> int:
    return _lib.hsakv_workspace_bytes(ctypes.byref(dims), entry)


def make_dims(*, H, d, Lq, tokens_per_frame, Psize, P, Kp, Binter, Bintra, Bq, r, dtype) -> Dims:
    dt = {"f32": F32, "bf16": BF16}.get(dtype, dtype)
    return Dims(H, d, Lq, tokens_per_frame, Psize, P, Kp, Binter, Bintra, Bq, r, dt)


# ---- entry points ------------------------------------------------------------

def hkv_page_summary(dims: Dims, pool_k, page_kmean, stream=None) -> None:
    _check("hkv_page_summary", _lib.hkv_page_summary(
        ctypes.byref(dims), _ptr(pool_k), _ptr(page_kmean), _stream(stream)))


def hkv_gather(dims: Dims, pool_k, pool_v, page_kmean, page_prompt, cur_prompt: int, q, page_idx,
               n_sel, k_hist, v_hist, ws, stream=None) -> None:
    w, wb = _ws(ws)
    _check("hkv_gather", _lib.hkv_gather(
        ctypes.byref(dims), _ptr(pool_k), _ptr(pool_v), _ptr(page_kmean), _ptr(page_prompt),
        int(cur_prompt), _ptr(q), _ptr(page_idx), _ptr(n_sel), _ptr(k_hist), _ptr(v_hist), w, wb,
        _stream(stream)))


def hsa_select(dims: Dims, q, k_hist, k_intra, n_sel, tau, sel_count, sel_idx, sel_mask=None,
               block_mass=None, ws=None, stream=None) -> None:
    w, wb = _ws(ws)
    _check("hsa_select", _lib.hsa_select(
        ctypes.byref(dims), _ptr(q), _ptr(k_hist), _ptr(k_intra), _ptr(n_sel),
        ctypes.cast(_host_f32(tau), c_void_p), _ptr(sel_count), _ptr(sel_idx), _ptr(sel_mask),
        _ptr(block_mass), w, wb, _stream(stream)))


def hsa_sparse_attn(dims: Dims, q, k_hist, v_hist, k_intra, v_intra, n_sel, sel_count, sel_idx,
                    o_sparse, ws=None, stream=None) -> None:
    w, wb = _ws(ws)
    _check("hsa_sparse_attn", _lib.hsa_sparse_attn(
        ctypes.byref(dims), _ptr(q), _ptr(k_hist), _ptr(v_hist), _ptr(k_intra), _ptr(v_intra),
        _ptr(n_sel), _ptr(sel_count), _ptr(sel_idx), _ptr(o_sparse), w, wb, _stream(stream)))


def hsa_linear_branch(dims: Dims, q, k_hist, v_hist, k_intra, v_intra, n_sel, E, F, o_linear,
                      k_low=None, v_low=None, ws=None, stream=None) -> None:
    w, wb = _ws(ws)
    _check("hsa_linear_branch", _lib.hsa_linear_branch(
        ctypes.byref(dims), _ptr(q), _ptr(k_hist), _ptr(v_hist), _ptr(k_intra), _ptr(v_intra),
        _ptr(n_sel), _ptr(E), _ptr(F), _ptr(o_linear), _ptr(k_low), _ptr(v_low), w, wb,
        _stream(stream)))


def hsa_fuse(dims: Dims, q, w_g, b_g, o_sparse, o_linear, out, gate=None, stream=None) -> None:
    _check("hsa_fuse", _lib.hsa_fuse(
        ctypes.byref(dims), _ptr(q), _ptr(w_g), _ptr(b_g), _ptr(o_sparse), _ptr(o_linear),
        _ptr(out), _ptr(gate), _stream(stream)))


def hsa_forward(dims: Dims, tau, cur_prompt: int, inputs: dict, outputs: dict, ws,
                stream=None) -> None:
    ins = Inputs(*[_ptr(inputs.get(n)) for n, _ in Inputs._fields_])
    outs = Outputs(*[_ptr(outputs.get(n)) for n, _ in Outputs._fields_])
    w, wb = _ws(ws)
    _check("hsa_forward", _lib.hsa_forward(
        ctypes.byref(dims), ctypes.cast(_host_f32(tau), c_void_p), int(cur_prompt),
        ctypes.byref(ins), ctypes.byref(outs), w, wb, _stream(stream)))
