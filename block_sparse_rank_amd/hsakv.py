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
ERR_TOO_LARGE = -9
STATIC_SCRATCH_BYTES = 128 << 20
F32 = 0
BF16 = 1
ENTRY_GATHER = 1
ENTRY_SELECT = 2
ENTRY_SPARSE = 3
ENTRY_LINEAR = 4
ENTRY_FORWARD = 6
ENTRY_SUMMARY = 7
ENTRY_COMMIT = 8
ENTRY_BACKWARD = 9
ENTRY_SPARSE_STATIC = 10

EXPORTS = [
    "hsakv_version", "hsakv_status_str", "hsakv_last_hip_error", "hsakv_validate",
    "hsakv_workspace_bytes", "hkv_page_summary", "hkv_gather", "hsa_select", "hsa_sparse_attn",
    "hsa_linear_branch", "hsa_fuse", "hsa_forward", "hsakv_fork_create", "hsakv_fork_destroy",
    "hsa_sparse_attn_static", "hkv_page_commit", "hsa_sparse_plan", "hsa_sparse_compute",
    "hsakv_host_alloc", "hsakv_host_free", "hkv_tier_plan", "hkv_tier_apply", "hsa_backward_params",
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


POLICIES = {"two_stage": 0, "page_only": 1, "prompt_only": 2, "recent": 3, "random": 4, "mismatched": 5}


class Retrieval(ctypes.Structure):
    """hsakv_retrieval: retrieval policy and the seed of the random policy."""
    _fields_ = [("policy", c_int32), ("reserved", c_int32), ("seed", ctypes.c_uint64)]


def _retrieval(policy, seed):
    if policy is None:
        return None
    pid = POLICIES[policy] if isinstance(policy, str) else int(policy)
    return ctypes.byref(Retrieval(pid, 0, int(seed)))


class Tiers(ctypes.Structure):
    """hsakv_tiers: device page table and the device addresses of the pinned host store."""
    _fields_ = [("page_slot", c_void_p), ("host_k", c_void_p), ("host_v", c_void_p)]


def make_tiers(page_slot, host_k, host_v) -> Tiers:
    return Tiers(_ptr(page_slot), _ptr(host_k), _ptr(host_v))


def _tiers(t):
    return ctypes.byref(t) if t is not None else None


class Fork(ctypes.Structure):
    """hsakv_fork: a caller-owned second stream and two events (hipStream_t,
    hipEvent_t handles) for hsa_forward's low-rank branch."""
    _fields_ = [("stream", c_void_p), ("fork", c_void_p), ("join", c_void_p)]


_P = c_void_p
_D = ctypes.POINTER(Dims)
_sig = {
    "hsakv_version": (c_int32, []),
    "hsakv_status_str": (ctypes.c_char_p, [c_int32]),
    "hsakv_last_hip_error": (c_int32, []),
    "hsakv_validate": (c_int32, [_D]),
    "hsakv_workspace_bytes": (c_size_t, [_D, c_int32]),
    "hkv_page_summary": (c_int32, [_D, _P, _P, _P, c_size_t, _P]),
    "hkv_gather": (c_int32, [_D, _P, _P, _P, _P, c_int32, ctypes.POINTER(Retrieval), ctypes.POINTER(Tiers), _P,
                             _P, _P, _P, _P, _P, c_size_t, _P]),
    "hsa_select": (c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "hsa_sparse_attn": (c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "hsa_linear_branch": (c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "hsa_fuse": (c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P]),
    "hsa_forward": (c_int32, [_D, _P, c_int32, ctypes.POINTER(Retrieval), ctypes.POINTER(Tiers),
                              ctypes.POINTER(Inputs), ctypes.POINTER(Outputs), _P, c_size_t, _P,
                              ctypes.POINTER(Fork)]),
    "hsakv_host_alloc": (c_int32, [c_size_t, ctypes.POINTER(c_void_p), ctypes.POINTER(c_void_p)]),
    "hsakv_host_free": (c_int32, [_P]),
    "hsa_backward_params": (c_int32, [_D] + [_P] * 18 + [c_size_t, _P, _P]),
    "hkv_tier_plan": (c_int32, [c_int32, c_int32, _P, _P, _P, ctypes.c_int64, _P, c_int32, _P, _P, _P, _P, _P,
                                _P]),
    "hkv_tier_apply": (c_int32, [_D, ctypes.POINTER(Tiers), _P, _P, c_int32, _P, _P, c_int32, _P, _P, c_int32,
                                 _P]),
    "hsa_sparse_attn_static": (c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "hsa_sparse_plan": (c_int32, [_D, _P, _P, _P, _P, c_size_t, _P]),
    "hsa_sparse_compute": (c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "hkv_page_commit": (c_int32, [_D, _P, _P, _P, _P, _P, _P, c_int32, ctypes.c_int64, c_int32, _P, c_size_t,
                                  _P]),
    "hsakv_fork_create": (c_int32, [ctypes.POINTER(Fork)]),
    "hsakv_fork_destroy": (c_int32, [ctypes.POINTER(Fork)]),
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


def _scratch(nbytes: int, like):
    """A device byte buffer for a workspace, on the device of tensor `like`
    (None when `like` is not a tensor: the library then rejects the call on
    the host)."""
    if not hasattr(like, "device") or nbytes <= 0:
        return None
    import torch
    return torch.empty(nbytes, dtype=torch.uint8, device=like.device)


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

def hkv_page_summary(dims: Dims, pool_k, page_kmean, ws=None, stream=None) -> None:
    """ws: a device buffer of workspace_bytes(dims, ENTRY_SUMMARY) bytes (allocated
    here through torch when None)."""
    if ws is None:
        ws = _scratch(workspace_bytes(dims, ENTRY_SUMMARY), page_kmean)
    w, wb = _ws(ws)
    _check("hkv_page_summary", _lib.hkv_page_summary(
        ctypes.byref(dims), _ptr(pool_k), _ptr(page_kmean), w, wb, _stream(stream)))


def hkv_page_commit(dims: Dims, pool_k, pool_v, page_kmean, page_prompt, k_chunk, v_chunk,
                    n_tokens: int, fill: int, cur_prompt: int, ws=None, stream=None) -> None:
    """ws: a device buffer of workspace_bytes(dims, ENTRY_COMMIT) bytes (allocated
    here through torch when None)."""
    if ws is None:
        ws = _scratch(workspace_bytes(dims, ENTRY_COMMIT), page_kmean)
    w, wb = _ws(ws)
    _check("hkv_page_commit", _lib.hkv_page_commit(
        ctypes.byref(dims), _ptr(pool_k), _ptr(pool_v), _ptr(page_kmean), _ptr(page_prompt),
        _ptr(k_chunk), _ptr(v_chunk), int(n_tokens), int(fill), int(cur_prompt), w, wb,
        _stream(stream)))


def hkv_gather(dims: Dims, pool_k, pool_v, page_kmean, page_prompt, cur_prompt: int, q, page_idx,
               n_sel, k_hist, v_hist, ws, stream=None, policy=None, seed: int = 0,
               tiers: Optional[Tiers] = None) -> None:
    w, wb = _ws(ws)
    _check("hkv_gather", _lib.hkv_gather(
        ctypes.byref(dims), _ptr(pool_k), _ptr(pool_v), _ptr(page_kmean), _ptr(page_prompt),
        int(cur_prompt), _retrieval(policy, seed), _tiers(tiers), _ptr(q), _ptr(page_idx), _ptr(n_sel),
        _ptr(k_hist), _ptr(v_hist), w, wb, _stream(stream)))


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


def hsa_sparse_plan(dims: Dims, n_sel, sel_count, sel_idx, ws, stream=None) -> None:
    w, wb = _ws(ws)
    _check("hsa_sparse_plan", _lib.hsa_sparse_plan(
        ctypes.byref(dims), _ptr(n_sel), _ptr(sel_count), _ptr(sel_idx), w, wb, _stream(stream)))


def hsa_sparse_compute(dims: Dims, q, k_hist, v_hist, k_intra, v_intra, n_sel, o_sparse, ws,
                       stream=None) -> None:
    w, wb = _ws(ws)
    _check("hsa_sparse_compute", _lib.hsa_sparse_compute(
        ctypes.byref(dims), _ptr(q), _ptr(k_hist), _ptr(v_hist), _ptr(k_intra), _ptr(v_intra),
        _ptr(n_sel), _ptr(o_sparse), w, wb, _stream(stream)))


def hsa_sparse_attn_static(dims: Dims, q, k_hist, v_hist, k_intra, v_intra, n_sel, sel_count,
                           sel_idx, o_sparse, stream=None) -> None:
    """hsa_sparse_attn with its scratch in the library's fixed device array:
    no workspace, no allocation."""
    _check("hsa_sparse_attn_static", _lib.hsa_sparse_attn_static(
        ctypes.byref(dims), _ptr(q), _ptr(k_hist), _ptr(v_hist), _ptr(k_intra), _ptr(v_intra),
        _ptr(n_sel), _ptr(sel_count), _ptr(sel_idx), _ptr(o_sparse), _stream(stream)))


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


def fork_create() -> Fork:
    """A new fork (second stream and two events) on the current device."""
    f = Fork()
    _check("hsakv_fork_create", _lib.hsakv_fork_create(ctypes.byref(f)))
    return f


def fork_destroy(f: Fork) -> None:
    _check("hsakv_fork_destroy", _lib.hsakv_fork_destroy(ctypes.byref(f)))


def hsa_forward(dims: Dims, tau, cur_prompt: int, inputs: dict, outputs: dict, ws,
                stream=None, fork: Optional[Fork] = None, policy=None, seed: int = 0,
                tiers: Optional[Tiers] = None) -> None:
    ins = Inputs(*[_ptr(inputs.get(n)) for n, _ in Inputs._fields_])
    outs = Outputs(*[_ptr(outputs.get(n)) for n, _ in Outputs._fields_])
    w, wb = _ws(ws)
    _check("hsa_forward", _lib.hsa_forward(
        ctypes.byref(dims), ctypes.cast(_host_f32(tau), c_void_p), int(cur_prompt),
        _retrieval(policy, seed), _tiers(tiers), ctypes.byref(ins), ctypes.byref(outs), w, wb,
        _stream(stream), ctypes.byref(fork) if fork is not None else None))


def hsa_backward_params(dims: Dims, q, k_hist, v_hist, k_intra, v_intra, n_sel, w_g, b_g, k_low, v_low,
                        o_sparse, o_linear, d_out, d_wg, d_bg, d_E, d_F, ws, stream=None, fork=None) -> None:
    w, wb = _ws(ws)
    _check("hsa_backward_params", _lib.hsa_backward_params(
        ctypes.byref(dims), *[_ptr(x) for x in (q, k_hist, v_hist, k_intra, v_intra, n_sel, w_g, b_g, k_low,
                                                v_low, o_sparse, o_linear, d_out, d_wg, d_bg, d_E, d_F)],
        w, wb, _stream(stream), ctypes.byref(fork) if fork is not None else None))


# ---- page tiers ---------------------------------------------------------------

class HostStore:
    """Pinned, device-mapped host memory from hsakv_host_alloc: `array` is a
    numpy view for the host, `device` the address kernels read."""

    def __init__(self, shape, dtype):
        import numpy as np
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        h, d = c_void_p(), c_void_p()
        _check("hsakv_host_alloc", _lib.hsakv_host_alloc(n, ctypes.byref(h), ctypes.byref(d)))
        self.host, self.device = h.value, d.value
        buf = (ctypes.c_char * n).from_address(self.host)
        self.array = np.frombuffer(buf, dtype=dtype).reshape(shape)

    def free(self):
        if self.host:
            self.array = None
            _check("hsakv_host_free", _lib.hsakv_host_free(self.host))
            self.host = self.device = None


class TierPlacement:
    """Host copy of the HBM slot placement for hkv_tier_plan (int32/int64 numpy arrays)."""

    def __init__(self, P: int, slots: int):
        import numpy as np
        self.P, self.slots = P, slots
        self.slot_of_page = np.full(P, -1, np.int32)
        self.page_of_slot = np.full(slots, -1, np.int32)
        self.last_use = np.zeros(P, np.int64)


def hkv_tier_plan(pl: TierPlacement, now: int, want):
    """Returns (promote_page, promote_slot, upd_page, upd_value) numpy arrays."""
    import numpy as np
    want = np.ascontiguousarray(np.asarray(want, np.int32))
    cap = max(1, min(len(want), pl.slots))
    pp, ps = np.zeros(cap, np.int32), np.zeros(cap, np.int32)
    up, uv = np.zeros(2 * cap, np.int32), np.zeros(2 * cap, np.int32)
    npro, nupd = ctypes.c_int32(), ctypes.c_int32()
    P = lambda a: a.ctypes.data_as(c_void_p)  # noqa: E731
    _check("hkv_tier_plan", _lib.hkv_tier_plan(
        pl.P, pl.slots, P(pl.slot_of_page), P(pl.page_of_slot), P(pl.last_use), int(now), P(want),
        len(want), P(pp), P(ps), ctypes.byref(npro), P(up), P(uv), ctypes.byref(nupd)))
    return pp[:npro.value].copy(), ps[:npro.value].copy(), up[:nupd.value].copy(), uv[:nupd.value].copy()


def hkv_tier_apply(dims: Dims, tiers: Tiers, pool_k, pool_v, slots: int, promote_page, promote_slot,
                   upd_page, upd_value, stream=None) -> None:
    import numpy as np
    a = [np.ascontiguousarray(np.asarray(x, np.int32)) for x in (promote_page, promote_slot, upd_page, upd_value)]
    P = lambda x: x.ctypes.data_as(c_void_p) if len(x) else None  # noqa: E731
    _check("hkv_tier_apply", _lib.hkv_tier_apply(
        ctypes.byref(dims), ctypes.byref(tiers), _ptr(pool_k), _ptr(pool_v), int(slots), P(a[0]), P(a[1]),
        len(a[0]), P(a[2]), P(a[3]), len(a[2]), _stream(stream)))
