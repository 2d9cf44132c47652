"""Python access to the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
bench's CPU-baseline leg, never by the product package.  Arrays are numpy;
bf16 tensors are uint16 bit patterns.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, E_INVALID_ARG, E_ALIGN, E_WORKSPACE, E_BAD_INDEX, E_HIP, E_OVERFLOW = 0, -1, -2, -3, -4, -5, -6

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (no fast-math, no contraction)."""
    cmd = ["gcc", *CFLAGS, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class _Dims(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("num_ranks", ctypes.c_int32)]


_P = ctypes.POINTER(ctypes.c_int32)


class _PlanOut(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("expert_count", "expert_offset", "rank_count", "rank_offset",
                                  "send_token", "tok_rank_row", "fan_src", "fan_dst", "comb_row",
                                  "rank_segs", "expert_segs", "n_rank_rows")]


class Oracle:
    """One loaded copy of the oracle library (path may point at a variant)."""

    def __init__(self, path: str = _LIB):
        if path == _LIB and not os.path.exists(path):
            build()
        self.lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        self.lib.oracle_check_dims.argtypes = [ctypes.POINTER(_Dims)]
        self.lib.oracle_plan.argtypes = [ctypes.POINTER(_Dims), vp, ctypes.POINTER(_PlanOut)]
        self.lib.oracle_dispatch.argtypes = [ctypes.POINTER(_Dims), vp, vp, ctypes.c_int32, vp, vp, vp]
        self.lib.oracle_combine.argtypes = [ctypes.POINTER(_Dims), vp, vp, vp, vp]
        self.lib.oracle_dispatch_backward.argtypes = [ctypes.POINTER(_Dims), vp, vp, ctypes.c_int32, vp, vp, vp]
        self.lib.oracle_combine_backward.argtypes = [ctypes.POINTER(_Dims), vp, vp, vp, vp, vp, vp]
        self.lib.oracle_combine_rank_partial.argtypes = [ctypes.POINTER(_Dims), vp, vp, vp, ctypes.c_int32, vp, vp,
                                                         vp, vp]
        self.lib.oracle_combine_rank_partial_f32.argtypes = self.lib.oracle_combine_rank_partial.argtypes
        self.lib.oracle_round_bf16.argtypes = [vp, vp, ctypes.c_int64]
        self.lib.oracle_round_bf16.restype = None
        for f in (self.lib.oracle_check_dims, self.lib.oracle_plan, self.lib.oracle_dispatch,
                  self.lib.oracle_combine, self.lib.oracle_dispatch_backward, self.lib.oracle_combine_backward,
                  self.lib.oracle_combine_rank_partial, self.lib.oracle_combine_rank_partial_f32):
            f.restype = ctypes.c_int

    @staticmethod
    def dims(T, H, E, k, R):
        return _Dims(int(T), int(H), int(E), int(k), int(R))

    def check_dims(self, T, H, E, k, R) -> int:
        d = self.dims(T, H, E, k, R)
        return self.lib.oracle_check_dims(ctypes.byref(d))

    def plan(self, idx: np.ndarray, H: int, E: int, R: int):
        """Returns (status, dict of plan arrays)."""
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, k = idx.shape
        d = self.dims(T, H, E, k, R)
        rc = self.lib.oracle_check_dims(ctypes.byref(d))
        if rc:
            return rc, None
        Epr = E // R
        KR, D = min(k, R), min(k, Epr)
        a = {
            "expert_count": np.zeros(E, np.int32), "expert_offset": np.zeros(E + 1, np.int32),
            "rank_count": np.zeros(R, np.int32), "rank_offset": np.zeros(R + 1, np.int32),
            "send_token": np.full(max(T * KR, 1), -7, np.int32),
            "tok_rank_row": np.full((T, KR), -7, np.int32),
            "fan_src": np.full(max(T * k, 1), -7, np.int32),
            "fan_dst": np.full((max(T * KR, 1), D), -7, np.int32),
            "comb_row": np.full((T, k), -7, np.int32),
            "rank_segs": np.zeros((R, 4), np.int32), "expert_segs": np.zeros((E, 4), np.int32),
            "n_rank_rows": np.zeros(1, np.int32),
        }
        o = _PlanOut(*[a[n].ctypes.data_as(_P) for n, _ in _PlanOut._fields_])
        rc = self.lib.oracle_plan(ctypes.byref(d), idx.ctypes.data, ctypes.byref(o))
        if rc:
            return rc, None
        N = int(a["n_rank_rows"][0])
        a["N"] = N
        a["send_token"] = a["send_token"][:N]
        a["fan_src"] = a["fan_src"][:T * k]
        a["fan_dst"] = a["fan_dst"][:N]
        return rc, a

    def round_bf16(self, bits: np.ndarray) -> np.ndarray:
        """The fp32 -> bf16 rounding step alone, on fp32 bit patterns (uint32)."""
        bits = np.ascontiguousarray(bits, dtype=np.uint32)
        out = np.zeros(bits.shape, np.uint16)
        self.lib.oracle_round_bf16(bits.ctypes.data, out.ctypes.data, bits.size)
        return out

    def dispatch(self, plan: dict, x: np.ndarray, E: int, k: int, R: int):
        x = np.ascontiguousarray(x, dtype=np.uint16)
        T, H = x.shape
        N = plan["N"]
        d = self.dims(T, H, E, k, R)
        xr = np.zeros((N, H), np.uint16)
        xe = np.zeros((T * k, H), np.uint16)
        st = np.ascontiguousarray(plan["send_token"], dtype=np.int32)
        fs = np.ascontiguousarray(plan["fan_src"], dtype=np.int32)
        rc = self.lib.oracle_dispatch(ctypes.byref(d), st.ctypes.data, fs.ctypes.data, N,
                                      x.ctypes.data, xr.ctypes.data, xe.ctypes.data)
        if rc:
            raise RuntimeError(f"oracle_dispatch: {rc}")
        return xr, xe

    def combine(self, comb_row: np.ndarray, ye: np.ndarray, w: np.ndarray, E: int, R: int):
        comb_row = np.ascontiguousarray(comb_row, dtype=np.int32)
        ye = np.ascontiguousarray(ye, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        T, k = comb_row.shape
        H = ye.shape[1]
        d = self.dims(T, H, E, k, R)
        out = np.zeros((T, H), np.uint16)
        rc = self.lib.oracle_combine(ctypes.byref(d), comb_row.ctypes.data, ye.ctypes.data,
                                     w.ctypes.data, out.ctypes.data)
        if rc:
            raise RuntimeError(f"oracle_combine: {rc}")
        return out


    def dispatch_backward(self, plan: dict, grad_xe: np.ndarray, T: int, E: int, k: int, R: int):
        """Returns (grad_xr [N,H], grad_x [T,H]) as bf16 bits."""
        grad_xe = np.ascontiguousarray(grad_xe, dtype=np.uint16)
        H = grad_xe.shape[1]
        N = plan["N"]
        d = self.dims(T, H, E, k, R)
        gxr = np.zeros((N, H), np.uint16)
        gx = np.zeros((T, H), np.uint16)
        fd = np.ascontiguousarray(plan["fan_dst"], dtype=np.int32)
        tr = np.ascontiguousarray(plan["tok_rank_row"], dtype=np.int32)
        rc = self.lib.oracle_dispatch_backward(ctypes.byref(d), fd.ctypes.data, tr.ctypes.data, N,
                                               grad_xe.ctypes.data, gxr.ctypes.data, gx.ctypes.data)
        if rc:
            raise RuntimeError(f"oracle_dispatch_backward: {rc}")
        return gxr, gx

    def combine_backward(self, comb_row: np.ndarray, grad_out: np.ndarray, ye: np.ndarray, w: np.ndarray,
                         E: int, R: int):
        """Returns (grad_ye [T*k,H] bf16 bits, grad_w [T,k] float64)."""
        comb_row = np.ascontiguousarray(comb_row, dtype=np.int32)
        grad_out = np.ascontiguousarray(grad_out, dtype=np.uint16)
        ye = np.ascontiguousarray(ye, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        T, k = comb_row.shape
        H = grad_out.shape[1]
        d = self.dims(T, H, E, k, R)
        gye = np.zeros((T * k, H), np.uint16)
        gw = np.zeros((T, k), np.float64)
        rc = self.lib.oracle_combine_backward(ctypes.byref(d), comb_row.ctypes.data, grad_out.ctypes.data,
                                              ye.ctypes.data, w.ctypes.data, gye.ctypes.data, gw.ctypes.data)
        if rc:
            raise RuntimeError(f"oracle_combine_backward: {rc}")
        return gye, gw

    def combine_rank_partial(self, plan: dict, ye: np.ndarray, w: np.ndarray, E: int, R: int):
        """Returns (partial [N,H], out [T,H]) as bf16 bits."""
        ye = np.ascontiguousarray(ye, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        T, k = w.shape
        H = ye.shape[1]
        N = plan["N"]
        d = self.dims(T, H, E, k, R)
        part = np.zeros((N, H), np.uint16)
        out = np.zeros((T, H), np.uint16)
        fd = np.ascontiguousarray(plan["fan_dst"], dtype=np.int32)
        tr = np.ascontiguousarray(plan["tok_rank_row"], dtype=np.int32)
        cr = np.ascontiguousarray(plan["comb_row"], dtype=np.int32)
        rc = self.lib.oracle_combine_rank_partial(ctypes.byref(d), fd.ctypes.data, tr.ctypes.data, cr.ctypes.data,
                                                  N, ye.ctypes.data, w.ctypes.data, part.ctypes.data,
                                                  out.ctypes.data)
        if rc:
            raise RuntimeError(f"oracle_combine_rank_partial: {rc}")
        return part, out


    def combine_rank_partial_f32(self, plan: dict, ye: np.ndarray, w: np.ndarray, E: int, R: int):
        """Returns (partial [N,H] fp32, out [T,H] bf16 bits): partials kept in fp32."""
        ye = np.ascontiguousarray(ye, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        T, k = w.shape
        H = ye.shape[1]
        N = plan["N"]
        d = self.dims(T, H, E, k, R)
        part = np.zeros((N, H), np.float32)
        out = np.zeros((T, H), np.uint16)
        fd = np.ascontiguousarray(plan["fan_dst"], dtype=np.int32)
        tr = np.ascontiguousarray(plan["tok_rank_row"], dtype=np.int32)
        cr = np.ascontiguousarray(plan["comb_row"], dtype=np.int32)
        rc = self.lib.oracle_combine_rank_partial_f32(ctypes.byref(d), fd.ctypes.data, tr.ctypes.data,
                                                      cr.ctypes.data, N, ye.ctypes.data, w.ctypes.data,
                                                      part.ctypes.data, out.ctypes.data)
        if rc:
            raise RuntimeError(f"oracle_combine_rank_partial_f32: {rc}")
        return part, out


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
