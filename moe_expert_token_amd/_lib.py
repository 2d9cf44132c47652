"""ctypes binding of libmoe_shuffle.so: argument marshalling only.

Every function here has the name of the C function it calls and only turns
torch tensors into pointers, streams into handles and status codes into
exceptions.  All computation happens in the HIP kernels of the library; if
the library is missing or fails to load, this module raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_shuffle.so")

OK, E_INVALID_ARG, E_ALIGN, E_WORKSPACE, E_BAD_INDEX, E_HIP, E_OVERFLOW = 0, -1, -2, -3, -4, -5, -6

# Every function the header declares.
EXPORTS = (
    "moe_shuffle_workspace_size", "moe_shuffle_plan", "moe_shuffle_dispatch", "moe_shuffle_dispatch_send",
    "moe_shuffle_dispatch_fanout", "moe_shuffle_combine", "moe_shuffle_plan_query",
    "moe_shuffle_plan_arrays_get", "moe_shuffle_plan_destroy", "moe_shuffle_strerror",
    "moe_shuffle_last_hip_error", "moe_shuffle_sum_expert_rows", "moe_shuffle_sum_rank_rows",
    "moe_shuffle_dispatch_backward", "moe_shuffle_combine_rank_partial", "moe_shuffle_combine_backward",
    "moe_shuffle_dispatch_range", "moe_shuffle_combine_range", "moe_shuffle_combine_rank_partial_f32",
    "moe_shuffle_copy_reference", "moe_shuffle_plan_static",
)

STATIC_WORKSPACE_BYTES = 64 << 20  # MOE_SHUFFLE_STATIC_WORKSPACE_BYTES


class MoeShuffleError(RuntimeError):
    def __init__(self, func: str, code: int, text: str, hip: int = 0):
        msg = f"{func}: {text} ({code})"
        if code == E_HIP:
            msg += f", hipError {hip}"
        super().__init__(msg)
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("num_ranks", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_rank_rows", ctypes.c_int32), ("n_expert_rows", ctypes.c_int32), ("status", ctypes.c_int32),
                ("max_rank_rows", ctypes.c_int32)]


_vp = ctypes.c_void_p


class PlanStorage(ctypes.Structure):
    """Host storage for the handle of moe_shuffle_plan_static."""
    _fields_ = [("opaque", ctypes.c_uint64 * 64)]


class PlanArrays(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("expert_count", "expert_offset", "rank_count", "rank_offset", "send_token",
                                   "tok_rank_row", "fan_src", "fan_dst", "comb_row", "rank_segs", "expert_segs",
                                   "status", "n_rank_rows")] + \
               [("tok_rank_width", ctypes.c_int32), ("fan_dst_width", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it is absent or does not load)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m moe_expert_token_amd.build`")
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    sig = {
        "moe_shuffle_workspace_size": (ctypes.c_int, [ctypes.POINTER(Dims), ctypes.POINTER(ctypes.c_size_t)]),
        "moe_shuffle_plan": (ctypes.c_int, [ctypes.POINTER(Dims), _vp, _vp, ctypes.c_size_t, _vp, ctypes.POINTER(_vp)]),
        "moe_shuffle_dispatch": (ctypes.c_int, [_vp, _vp, _vp, i64, _vp, _vp]),
        "moe_shuffle_dispatch_send": (ctypes.c_int, [_vp, _vp, _vp, i64, _vp]),
        "moe_shuffle_dispatch_fanout": (ctypes.c_int, [_vp, _vp, i64, _vp, _vp]),
        "moe_shuffle_combine": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp]),
        "moe_shuffle_plan_query": (ctypes.c_int, [_vp, _vp, ctypes.POINTER(PlanInfo)]),
        "moe_shuffle_plan_arrays_get": (ctypes.c_int, [_vp, ctypes.POINTER(PlanArrays)]),
        "moe_shuffle_plan_destroy": (None, [_vp]),
        "moe_shuffle_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_shuffle_last_hip_error": (ctypes.c_int, []),
        "moe_shuffle_sum_expert_rows": (ctypes.c_int, [_vp, _vp, _vp, _vp, i64, _vp]),
        "moe_shuffle_sum_rank_rows": (ctypes.c_int, [_vp, _vp, i64, _vp, _vp]),
        "moe_shuffle_dispatch_backward": (ctypes.c_int, [_vp, _vp, _vp, i64, _vp, _vp]),
        "moe_shuffle_combine_rank_partial": (ctypes.c_int, [_vp, _vp, _vp, _vp, i64, _vp, _vp]),
        "moe_shuffle_combine_rank_partial_f32": (ctypes.c_int, [_vp, _vp, _vp, _vp, i64, _vp, _vp]),
        "moe_shuffle_combine_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
        "moe_shuffle_dispatch_range": (ctypes.c_int, [_vp, _vp, _vp, i64, _vp, ctypes.c_int32, ctypes.c_int32, _vp]),
        "moe_shuffle_combine_range": (ctypes.c_int, [_vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp]),
        "moe_shuffle_copy_reference": (ctypes.c_int, [_vp, _vp, ctypes.c_size_t, _vp]),
        "moe_shuffle_plan_static": (ctypes.c_int, [ctypes.POINTER(Dims), _vp, _vp, ctypes.POINTER(PlanStorage),
                                                   ctypes.POINTER(_vp)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


def _check(func: str, rc: int):
    if rc != OK:
        lib = load()
        raise MoeShuffleError(func, rc, lib.moe_shuffle_strerror(rc).decode(), lib.moe_shuffle_last_hip_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


# The current stream's raw handle without building a torch Stream object
# (several microseconds per call, which small batches feel).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream):
    if stream is None:
        if _raw_stream is not None and _cur_device is not None:
            return _raw_stream(_cur_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def dims_of(T: int, H: int, E: int, k: int, R: int) -> Dims:
    return Dims(int(T), int(H), int(E), int(k), int(R))


class Plan:
    """Host handle returned by moe_shuffle_plan (freed on destroy / GC)."""

    def __init__(self, handle: int, dims: Dims, workspace, idx):
        self.handle = handle
        self.dims = dims
        self.workspace = workspace  # keep the workspace (and the ids the kernels read) alive
        self._idx = idx

    @property
    def T(self):
        return self.dims.num_tokens

    @property
    def H(self):
        return self.dims.hidden

    @property
    def k(self):
        return self.dims.top_k

    @property
    def KR(self):
        return min(self.dims.top_k, self.dims.num_ranks)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.moe_shuffle_plan_destroy(self.handle)
            self.handle = None


def moe_shuffle_workspace_size(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_shuffle_workspace_size", load().moe_shuffle_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def moe_shuffle_plan(dims: Dims, topk_idx, workspace, stream=None) -> Plan:
    h = _vp(0)
    nbytes = workspace.numel() * workspace.element_size()
    rc = load().moe_shuffle_plan(ctypes.byref(dims), _ptr(topk_idx), _ptr(workspace), nbytes, _stream(stream),
                                 ctypes.byref(h))
    _check("moe_shuffle_plan", rc)
    return Plan(h.value, dims, workspace, topk_idx)


def moe_shuffle_plan_static(dims: Dims, topk_idx, stream=None) -> Plan:
    """The plan in the library's static workspace (no device allocation); the
    returned Plan holds the handle's storage.  A later static plan on the same
    GPU invalidates this one."""
    h = _vp(0)
    storage = PlanStorage()
    rc = load().moe_shuffle_plan_static(ctypes.byref(dims), _ptr(topk_idx), _stream(stream), ctypes.byref(storage),
                                        ctypes.byref(h))
    _check("moe_shuffle_plan_static", rc)
    plan = Plan(h.value, dims, None, topk_idx)
    plan.storage = storage
    return plan


def moe_shuffle_dispatch(plan: Plan, x, xr, xe, stream=None):
    _check("moe_shuffle_dispatch", load().moe_shuffle_dispatch(plan.handle, _ptr(x), _ptr(xr), xr.shape[0],
                                                               _ptr(xe), _stream(stream)))


def moe_shuffle_dispatch_send(plan: Plan, x, xr, stream=None):
    _check("moe_shuffle_dispatch_send", load().moe_shuffle_dispatch_send(plan.handle, _ptr(x), _ptr(xr),
                                                                         xr.shape[0], _stream(stream)))


def moe_shuffle_dispatch_fanout(plan: Plan, xr, xe, stream=None):
    _check("moe_shuffle_dispatch_fanout", load().moe_shuffle_dispatch_fanout(plan.handle, _ptr(xr), xr.shape[0],
                                                                             _ptr(xe), _stream(stream)))


def moe_shuffle_combine(plan: Plan, ye, topk_w, out, stream=None):
    _check("moe_shuffle_combine", load().moe_shuffle_combine(plan.handle, _ptr(ye), _ptr(topk_w), _ptr(out),
                                                             _stream(stream)))


def moe_shuffle_copy_reference(src, dst, nbytes=None, stream=None):
    """The reference streaming copy (a bandwidth yardstick, not a step of the
    shuffle): the first nbytes (default: all of src) of src into dst."""
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    _check("moe_shuffle_copy_reference", load().moe_shuffle_copy_reference(_ptr(src), _ptr(dst), int(nbytes),
                                                                           _stream(stream)))


def moe_shuffle_sum_expert_rows(plan: Plan, expert_rows, topk_w, rank_rows, stream=None):
    _check("moe_shuffle_sum_expert_rows", load().moe_shuffle_sum_expert_rows(
        plan.handle, _ptr(expert_rows), _ptr(topk_w), _ptr(rank_rows), rank_rows.shape[0], _stream(stream)))


def moe_shuffle_sum_rank_rows(plan: Plan, rank_rows, out, stream=None):
    _check("moe_shuffle_sum_rank_rows", load().moe_shuffle_sum_rank_rows(
        plan.handle, _ptr(rank_rows), rank_rows.shape[0], _ptr(out), _stream(stream)))


def moe_shuffle_dispatch_backward(plan: Plan, grad_xe, grad_xr, grad_x, stream=None):
    _check("moe_shuffle_dispatch_backward", load().moe_shuffle_dispatch_backward(
        plan.handle, _ptr(grad_xe), _ptr(grad_xr), grad_xr.shape[0], _ptr(grad_x), _stream(stream)))


def moe_shuffle_combine_rank_partial(plan: Plan, ye, topk_w, partial, out, stream=None):
    _check("moe_shuffle_combine_rank_partial", load().moe_shuffle_combine_rank_partial(
        plan.handle, _ptr(ye), _ptr(topk_w), _ptr(partial), partial.shape[0], _ptr(out), _stream(stream)))


def moe_shuffle_combine_rank_partial_f32(plan: Plan, ye, topk_w, partial, out, stream=None):
    """As moe_shuffle_combine_rank_partial with fp32 partial rows (partial: float32 [rows, H])."""
    _check("moe_shuffle_combine_rank_partial_f32", load().moe_shuffle_combine_rank_partial_f32(
        plan.handle, _ptr(ye), _ptr(topk_w), _ptr(partial), partial.shape[0], _ptr(out), _stream(stream)))


def moe_shuffle_combine_backward(plan: Plan, grad_out, ye, topk_w, grad_ye, grad_w, stream=None):
    _check("moe_shuffle_combine_backward", load().moe_shuffle_combine_backward(
        plan.handle, _ptr(grad_out), _ptr(ye), _ptr(topk_w), _ptr(grad_ye), _ptr(grad_w), _stream(stream)))


def moe_shuffle_dispatch_range(plan: Plan, x, xr, xe, t0: int, t1: int, stream=None):
    _check("moe_shuffle_dispatch_range", load().moe_shuffle_dispatch_range(
        plan.handle, _ptr(x), _ptr(xr), xr.shape[0], _ptr(xe), int(t0), int(t1), _stream(stream)))


def moe_shuffle_combine_range(plan: Plan, ye, topk_w, out, t0: int, t1: int, stream=None):
    _check("moe_shuffle_combine_range", load().moe_shuffle_combine_range(
        plan.handle, _ptr(ye), _ptr(topk_w), _ptr(out), int(t0), int(t1), _stream(stream)))


def moe_shuffle_plan_query(plan: Plan, stream=None) -> dict:
    info = PlanInfo()
    rc = load().moe_shuffle_plan_query(plan.handle, _stream(stream), ctypes.byref(info))
    if rc not in (OK, E_BAD_INDEX):
        _check("moe_shuffle_plan_query", rc)
    return {"status": info.status, "N": info.n_rank_rows, "n_expert_rows": info.n_expert_rows,
            "max_rank_rows": info.max_rank_rows}


def moe_shuffle_plan_arrays_get(plan: Plan) -> dict:
    a = PlanArrays()
    _check("moe_shuffle_plan_arrays_get", load().moe_shuffle_plan_arrays_get(plan.handle, ctypes.byref(a)))
    out = {n: getattr(a, n) for n, _ in PlanArrays._fields_}
    return out


def moe_shuffle_plan_destroy(plan: Plan):
    if plan.handle:
        load().moe_shuffle_plan_destroy(plan.handle)
        plan.handle = None


def moe_shuffle_strerror(code: int) -> str:
    return load().moe_shuffle_strerror(code).decode()


def moe_shuffle_last_hip_error() -> int:
    return load().moe_shuffle_last_hip_error()


def plan_array_views(plan: Plan, N: int | None = None) -> dict:
    """int32 views of the plan arrays inside the workspace tensor (no copy)."""
    if plan.workspace is None:
        raise ValueError("a plan of moe_shuffle_plan_static lives in the library's static buffer, not in a "
                         "workspace tensor; read its arrays through moe_shuffle_plan_arrays_get")
    a = moe_shuffle_plan_arrays_get(plan)
    ws = plan.workspace
    base = ws.data_ptr()
    d = plan.dims
    T, k, E, R = d.num_tokens, d.top_k, d.num_experts, d.num_ranks
    KR, D = a["tok_rank_width"], a["fan_dst_width"]
    if N is None:
        N = T * KR
    shapes = {
        "expert_count": (E,), "expert_offset": (E + 1,), "rank_count": (R,), "rank_offset": (R + 1,),
        "send_token": (N,), "tok_rank_row": (T, KR), "fan_src": (T * k,), "fan_dst": (N, D),
        "comb_row": (T, k), "rank_segs": (R, 4), "expert_segs": (E, 4), "status": (1,), "n_rank_rows": (1,),
    }
    i32 = ws.view(torch.int32) if ws.dtype != torch.int32 else ws
    views = {}
    for name, shape in shapes.items():
        off = a[name] - base
        assert off % 4 == 0
        n = 1
        for s in shape:
            n *= s
        views[name] = i32[off // 4: off // 4 + n].view(*shape)
    return views
