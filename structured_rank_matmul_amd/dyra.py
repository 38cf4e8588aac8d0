"""Python binding of libdyra (ctypes).  Argument marshalling only.

Every step of the DyRA forward path runs in the HIP library; this module only
checks tensor placement, allocates outputs and workspaces with PyTorch, and
passes raw device pointers and the current HIP stream to the C ABI declared in
include/dyra.h.  If libdyra.so is missing or fails to load, every call raises:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdyra.so")

DYRA_F32 = 0
DYRA_BF16 = 1
_DTYPES = {"f32": DYRA_F32, "float32": DYRA_F32, "bf16": DYRA_BF16, "bfloat16": DYRA_BF16}

# Every symbol include/dyra.h declares.
EXPORTED = (
    "dyra_status_str", "dyra_factorize_host", "dyra_prepare", "dyra_prepare_ex", "dyra_plan_destroy",
    "dyra_plan_info",
    "dyra_workspace_bytes", "dyra_forward", "dyra_forward_ex", "dyra_forward_status", "dyra_dense_ref",
    "dyra_forward_timed", "dyra_stage_name", "dyra_prepare_blast", "dyra_factorize_blast_host",
    "dyra_forward_noalloc", "dyra_noalloc_scratch_bytes",
)


class DyraError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


_lib = None


def load() -> ctypes.CDLL:
    """Loads libdyra.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
    vp, dp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
    L.dyra_status_str.argtypes = [ctypes.c_int]
    L.dyra_status_str.restype = ctypes.c_char_p
    L.dyra_factorize_host.argtypes = [vp, i64, i64, i32, i32, f64, dp, dp, dp, dp, dp]
    L.dyra_factorize_host.restype = ctypes.c_int
    L.dyra_prepare.argtypes = [vp, i64, i64, i32, i32, f32, ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp)]
    L.dyra_prepare.restype = ctypes.c_int
    L.dyra_prepare_ex.argtypes = [vp, i64, i64, i32, i32, f32, ctypes.c_int, ctypes.c_int, vp, i32, i32,
                                  ctypes.POINTER(vp)]
    L.dyra_prepare_ex.restype = ctypes.c_int
    L.dyra_prepare_blast.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, i32, f32, ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(vp)]
    L.dyra_prepare_blast.restype = ctypes.c_int
    L.dyra_factorize_blast_host.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, i32, f64, dp, dp, dp]
    L.dyra_factorize_blast_host.restype = ctypes.c_int
    L.dyra_plan_destroy.argtypes = [vp]
    L.dyra_plan_destroy.restype = None
    L.dyra_plan_info.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i32),
                                 ctypes.POINTER(i32), ctypes.POINTER(f32), ctypes.POINTER(ctypes.c_int),
                                 ctypes.POINTER(ctypes.c_int)]
    L.dyra_plan_info.restype = ctypes.c_int
    L.dyra_workspace_bytes.argtypes = [vp, i64, i64]
    L.dyra_workspace_bytes.restype = ctypes.c_size_t
    L.dyra_forward.argtypes = [vp, i64, i64, vp, vp, vp, ctypes.c_size_t, vp]
    L.dyra_forward.restype = ctypes.c_int
    L.dyra_forward_ex.argtypes = [vp, i64, i64, vp, vp, f32, vp, vp, ctypes.c_size_t, vp]
    L.dyra_forward_ex.restype = ctypes.c_int
    L.dyra_forward_status.argtypes = [vp, i64, i64, vp, vp, ctypes.POINTER(i32)]
    L.dyra_forward_status.restype = ctypes.c_int
    L.dyra_dense_ref.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, vp, vp]
    L.dyra_dense_ref.restype = ctypes.c_int
    L.dyra_forward_timed.argtypes = [vp, i64, i64, vp, vp, vp, ctypes.c_size_t, vp, ctypes.POINTER(vp), i32,
                                     ctypes.POINTER(i32)]
    L.dyra_forward_timed.restype = ctypes.c_int
    L.dyra_forward_noalloc.argtypes = [vp, i64, i64, vp, vp, vp]
    L.dyra_forward_noalloc.restype = ctypes.c_int
    L.dyra_noalloc_scratch_bytes.argtypes = []
    L.dyra_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.dyra_stage_name.argtypes = [vp, i64, i32]
    L.dyra_stage_name.restype = ctypes.c_char_p
    _lib = L
    return L


def status_str(status: int) -> str:
    return load().dyra_status_str(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise DyraError(status, what)


def _dtype_code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    key = str(dtype).replace("torch.", "")
    if key not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype!r}")
    return _DTYPES[key]


# ------------------------------------------------------------------ host factorisation

def dyra_factorize_host(W: np.ndarray, r: int, k: int, lam: float = 0.0) -> Dict[str, np.ndarray]:
    """Float64 factors of W ([c1, c2] float32, X @ W orientation) from the library's host SVD."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    c1, c2 = W.shape
    out = {"A_s": np.zeros((c1, r)), "V_s": np.zeros((c2, r)), "R0": np.zeros((k, c2)),
           "P_L": np.zeros((c1, k)), "sigma": np.zeros(r + k)}
    ptr = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))  # noqa: E731
    st = load().dyra_factorize_host(W.ctypes.data, c1, c2, int(r), int(k), float(lam), ptr(out["A_s"]),
                                    ptr(out["V_s"]), ptr(out["R0"]), ptr(out["P_L"]), ptr(out["sigma"]))
    _check(st, "dyra_factorize_host")
    return out


# ------------------------------------------------------------------ plan

class Plan:
    """A prepared layer (owns the library's device buffers)."""

    def __init__(self, handle: int, c1: int, c2: int, r: int, k: int, lam: float, dtype: int, device: int):
        self.handle = handle
        self.c1, self.c2, self.r, self.k = c1, c2, r, k
        self.lam = lam
        self.dtype = dtype
        self.device = device

    @property
    def torch_dtype(self):
        import torch
        return torch.bfloat16 if self.dtype == DYRA_BF16 else torch.float32

    def close(self) -> None:
        if self.handle:
            load().dyra_plan_destroy(ctypes.c_void_p(self.handle))
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def info(self) -> dict:
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        c1, c2, r, k = i64(), i64(), i32(), i32()
        lam, dt, dev = ctypes.c_float(), ctypes.c_int(), ctypes.c_int()
        _check(load().dyra_plan_info(ctypes.c_void_p(self.handle), ctypes.byref(c1), ctypes.byref(c2),
                                     ctypes.byref(r), ctypes.byref(k), ctypes.byref(lam), ctypes.byref(dt),
                                     ctypes.byref(dev)), "dyra_plan_info")
        return {"c1": c1.value, "c2": c2.value, "r": r.value, "k": k.value, "lambda": lam.value,
                "dtype": dt.value, "device": dev.value}


def dyra_prepare(W: np.ndarray, r: int, k: int, lam: float = 0.0, dtype="bf16", device: int = 0) -> Plan:
    """Algorithm 1 Offline Preparation in the library; W is [c1, c2] float32 on the host."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    c1, c2 = W.shape
    code = _dtype_code(dtype)
    h = ctypes.c_void_p()
    st = load().dyra_prepare(W.ctypes.data, c1, c2, int(r), int(k), float(lam), code, int(device), ctypes.byref(h))
    _check(st, "dyra_prepare")
    return Plan(h.value, c1, c2, int(r), int(k), float(lam), code, int(device))


def dyra_prepare_ex(W: np.ndarray, r: int, k: int, lam: float = 0.0, dtype="bf16", device: int = 0,
                    R0: Optional[np.ndarray] = None, als_half_steps: int = 2, ns_iters: int = 0) -> Plan:
    """dyra_prepare with a given R^(0) ([k, c2], e.g. Gaussian), the number of
    single ALS updates (2 = t 1, 3 = t 1.5, 4 = t 2) and the SPD solve (0 =
    Cholesky, > 0 = that many Newton-Schulz steps)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    c1, c2 = W.shape
    code = _dtype_code(dtype)
    r0 = None
    if R0 is not None:
        r0 = np.ascontiguousarray(R0, dtype=np.float32)
        if r0.shape != (int(k), c2):
            raise ValueError(f"R0 must be [{k}, {c2}]")
    h = ctypes.c_void_p()
    st = load().dyra_prepare_ex(W.ctypes.data, c1, c2, int(r), int(k), float(lam), code, int(device),
                                r0.ctypes.data if r0 is not None else None, int(als_half_steps), int(ns_iters),
                                ctypes.byref(h))
    _check(st, "dyra_prepare_ex")
    return Plan(h.value, c1, c2, int(r), int(k), float(lam), code, int(device))


def dyra_factorize_blast_host(W: np.ndarray, U: np.ndarray, S: np.ndarray, V: np.ndarray, nb: int, k: int,
                              lam: float = 0.0) -> Dict[str, np.ndarray]:
    """The library's host BLAST preparation alone: W_res, R0, P_L (float64)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    U = np.ascontiguousarray(U, dtype=np.float32)
    S = np.ascontiguousarray(S, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    c1, c2 = W.shape
    rb = U.shape[1]
    out = {"W_res": np.zeros((c1, c2)), "R0": np.zeros((k, c2)), "P_L": np.zeros((c1, k))}
    dp = ctypes.POINTER(ctypes.c_double)
    st = load().dyra_factorize_blast_host(W.ctypes.data, c1, c2, int(nb), int(rb), U.ctypes.data, S.ctypes.data,
                                          V.ctypes.data, int(k), float(lam),
                                          *[out[n].ctypes.data_as(dp) for n in ("W_res", "R0", "P_L")])
    _check(st, "dyra_factorize_blast_host")
    return out


def dyra_prepare_blast(W: np.ndarray, U: np.ndarray, S: np.ndarray, V: np.ndarray, nb: int, k: int,
                       lam: float = 0.0, dtype="bf16", device: int = 0) -> Plan:
    """Offline Preparation with a BLAST W_hat from the given factors: U [c1, rb],
    S [nb, nb, rb] (diagonal couplings), V [c2, rb]; all float32 on the host."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    c1, c2 = W.shape
    U = np.ascontiguousarray(U, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    S = np.ascontiguousarray(S, dtype=np.float32)
    rb = U.shape[1] if U.ndim == 2 else -1
    if U.shape != (c1, rb) or V.shape != (c2, rb) or S.shape != (int(nb), int(nb), rb):
        raise ValueError(f"BLAST factors must be U [{c1}, rb], S [{nb}, {nb}, rb], V [{c2}, rb]")
    code = _dtype_code(dtype)
    h = ctypes.c_void_p()
    st = load().dyra_prepare_blast(W.ctypes.data, c1, c2, int(nb), int(rb), U.ctypes.data, S.ctypes.data,
                                   V.ctypes.data, int(k), float(lam), code, int(device), ctypes.byref(h))
    _check(st, "dyra_prepare_blast")
    return Plan(h.value, c1, c2, int(rb), int(k), float(lam), code, int(device))


def dyra_workspace_bytes(plan: Plan, B: int, n: int) -> int:
    return int(load().dyra_workspace_bytes(ctypes.c_void_p(plan.handle), int(B), int(n)))


def _stream_ptr(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev_ptr(t) -> int:
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def alloc_workspace(plan: Plan, B: int, n: int):
    import torch
    nbytes = max(dyra_workspace_bytes(plan, B, n), 16)
    return torch.empty(nbytes, dtype=torch.uint8, device=f"cuda:{plan.device}")


def _on_stream(t, stream) -> None:
    """A tensor allocated here on the current stream but used by work enqueued
    on another one: tell the caching allocator, so that its memory is not
    handed out again before that stream's work has finished."""
    import torch
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)


def dyra_forward(X, B: int, n: int, plan: Plan, Y=None, workspace=None, stream=None):
    """Algorithm 1 Inference for B instances of n tokens: X [B*n, c1] -> Y [B*n, c2] (device tensors)."""
    import torch
    if X.dtype != plan.torch_dtype:
        raise ValueError(f"X dtype {X.dtype} does not match the plan's {plan.torch_dtype}")
    if tuple(X.shape) != (B * n, plan.c1):
        raise ValueError(f"X shape {tuple(X.shape)} != ({B * n}, {plan.c1})")
    if Y is None:
        Y = torch.empty((B * n, plan.c2), dtype=X.dtype, device=X.device)
        _on_stream(Y, stream)
    if workspace is None:
        workspace = alloc_workspace(plan, B, n)
        _on_stream(workspace, stream)
    st = load().dyra_forward(_dev_ptr(X), int(B), int(n), ctypes.c_void_p(plan.handle), _dev_ptr(Y),
                             _dev_ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream_ptr(stream))
    _check(st, "dyra_forward")
    return Y


def dyra_forward_ex(X, B: int, n: int, plan: Plan, bias=None, alpha: float = 1.0, Y=None, workspace=None,
                    stream=None):
    """§2.4's fused linear layer: Y = X A_s V_s^T + bias + alpha L1 R1 (bias [c2] device tensor or None)."""
    import torch
    if X.dtype != plan.torch_dtype:
        raise ValueError(f"X dtype {X.dtype} does not match the plan's {plan.torch_dtype}")
    if tuple(X.shape) != (B * n, plan.c1):
        raise ValueError(f"X shape {tuple(X.shape)} != ({B * n}, {plan.c1})")
    if bias is not None and (bias.dtype != X.dtype or tuple(bias.shape) != (plan.c2,)):
        raise ValueError(f"bias must be [{plan.c2}] in {X.dtype}")
    if Y is None:
        Y = torch.empty((B * n, plan.c2), dtype=X.dtype, device=X.device)
        _on_stream(Y, stream)
    if workspace is None:
        workspace = alloc_workspace(plan, B, n)
        _on_stream(workspace, stream)
    st = load().dyra_forward_ex(_dev_ptr(X), int(B), int(n), ctypes.c_void_p(plan.handle),
                                _dev_ptr(bias) if bias is not None else None, float(alpha), _dev_ptr(Y),
                                _dev_ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream_ptr(stream))
    _check(st, "dyra_forward_ex")
    return Y


def dyra_forward_noalloc(X, B: int, n: int, plan: Plan, Y, stream=None):
    """dyra_forward with the library's built-in per-GPU scratch as workspace
    (the caller passes X and Y; nothing is allocated).  Calls overlapping on
    one GPU race on that scratch."""
    if X.dtype != plan.torch_dtype or Y.dtype != plan.torch_dtype:
        raise ValueError(f"X and Y must be {plan.torch_dtype}")
    if tuple(X.shape) != (B * n, plan.c1) or tuple(Y.shape) != (B * n, plan.c2):
        raise ValueError(f"X must be ({B * n}, {plan.c1}) and Y ({B * n}, {plan.c2})")
    st = load().dyra_forward_noalloc(_dev_ptr(X), int(B), int(n), ctypes.c_void_p(plan.handle), _dev_ptr(Y),
                                     _stream_ptr(stream))
    _check(st, "dyra_forward_noalloc")
    return Y


def dyra_noalloc_scratch_bytes() -> int:
    return int(load().dyra_noalloc_scratch_bytes())


def dyra_forward_status(plan: Plan, B: int, n: int, workspace, stream=None) -> int:
    fails = ctypes.c_int32()
    st = load().dyra_forward_status(ctypes.c_void_p(plan.handle), int(B), int(n), _dev_ptr(workspace),
                                    _stream_ptr(stream), ctypes.byref(fails))
    _check(st, "dyra_forward_status")
    return int(fails.value)


def dyra_forward_timed(X, B: int, n: int, plan: Plan, Y, workspace, events, stream=None) -> int:
    """dyra_forward that records `events` (torch.cuda.Event, enable_timing) around each kernel."""
    for e in events:
        if not e.cuda_event:   # torch creates the HIP event on first record
            e.record(stream)
    ptrs = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    rec = ctypes.c_int32()
    st = load().dyra_forward_timed(_dev_ptr(X), int(B), int(n), ctypes.c_void_p(plan.handle), _dev_ptr(Y),
                                   _dev_ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream_ptr(stream), ptrs, len(events), ctypes.byref(rec))
    _check(st, "dyra_forward_timed")
    return int(rec.value)


def dyra_stage_name(plan: Plan, n: int, i: int) -> Optional[str]:
    s = load().dyra_stage_name(ctypes.c_void_p(plan.handle), int(n), int(i))
    return s.decode() if s is not None else None


def stage_names(plan: Plan, n: int):
    out, i = [], 0
    while True:
        s = dyra_stage_name(plan, n, i)
        if s is None:
            return out
        out.append(s)
        i += 1


def dyra_dense_ref(X, Wt, Y=None, stream=None):
    """Exact product Y = X W with Wt = W^T [c2, c1] (device tensors, same dtype)."""
    import torch
    N, c1 = X.shape
    c2 = Wt.shape[0]
    if Wt.shape[1] != c1 or Wt.dtype != X.dtype:
        raise ValueError("Wt must be [c2, c1] in X's dtype")
    if Y is None:
        Y = torch.empty((N, c2), dtype=X.dtype, device=X.device)
        _on_stream(Y, stream)
    st = load().dyra_dense_ref(_dev_ptr(X), _dev_ptr(Wt), N, c1, c2, _dtype_code(X.dtype), _dev_ptr(Y),
                               _stream_ptr(stream))
    _check(st, "dyra_dense_ref")
    return Y
