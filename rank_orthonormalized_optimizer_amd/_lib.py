"""ctypes view of the C ABI in include/dion.h (argument marshalling only).

The shared library must have been built (``python -m
rank_orthonormalized_optimizer_amd.build``); there is no fallback path.
torch, when present, is imported first so that the library binds to the HIP
runtime torch already loaded (both carry the soname libamdhip64.so.7) and
torch's device pointers and streams are valid in it.
"""
from __future__ import annotations

import ctypes
import os

try:  # one HIP runtime per process: let torch load it first
    import torch  # noqa: F401
except ImportError:  # the library itself does not need torch
    torch = None

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdion_mi355x.so")

# mirrors of the enums in include/dion.h
F32, BF16 = 0, 1
OK = 0
ERR_NULL, ERR_SHAPE, ERR_RANK, ERR_HYPER, ERR_ALIGN = -1, -2, -3, -4, -5
ERR_OVERLAP, ERR_WORKSPACE, ERR_DTYPE, ERR_OPTION, ERR_SCRATCH, ERR_HIP = -6, -7, -8, -9, -10, -100
NOALLOC_SCRATCH_BYTES = 64 << 20
OPT_STICKY_F64, OPT_FORCE_F64, OPT_FORCE_F32, OPT_HOUSEHOLDER, OPT_SPECTRAL_SHIFT = 1, 2, 4, 16, 32
OPT_EXACT_PRODUCTS = 64
OPT_CHUNKS_SHIFT = 8


def opt_chunks(n: int) -> int:
    """Option bits asking for n concurrent chunks (1 = everything on the caller's stream)."""
    return (int(n) & 15) << OPT_CHUNKS_SHIFT
FLAG_F64, FLAG_NONFINITE, FLAG_SHIFTED, FLAG_HOUSEHOLDER = 1, 2, 4, 8

NUM_PHASES = 10
PHASES = ("init", "f32_product", "f32_qr", "f32_backproject", "f64_product", "f64_qr", "f64_backproject",
          "norms", "update", "flags")

EXPORTS = ("dion_workspace_size", "dion_step_batched", "dion_step_batched_profiled", "dion_step_batched_ex",
           "dion_step_batched_noalloc",
           "dion_adamw_step",
           "dion_lion_step", "dion_lambda_max_workspace_size", "dion_lambda_max_batched", "dion_strerror",
           "dion_version")


class StepOutputs(ctypes.Structure):
    """dion_step_outputs: optional phase events and the per-matrix momentum-change output."""
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("rmmc", ctypes.c_void_p)]


class DionError(RuntimeError):
    def __init__(self, status: int, what: str = "dion_step_batched"):
        super().__init__(f"{what} failed with status {status}: {strerror(status)}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the library (once) and declare the signatures; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m rank_orthonormalized_optimizer_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.dion_workspace_size.restype = ctypes.c_size_t
    lib.dion_workspace_size.argtypes = [i64, i64, i64, i64]
    lib.dion_step_batched.restype = ctypes.c_int
    lib.dion_step_batched.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64,
                                      ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                      ctypes.c_int, ctypes.c_int, vp, ctypes.c_size_t,
                                      vp, ctypes.c_uint32, vp]
    lib.dion_step_batched_profiled.restype = ctypes.c_int
    lib.dion_step_batched_profiled.argtypes = lib.dion_step_batched.argtypes + [ctypes.POINTER(ctypes.c_void_p)]
    lib.dion_step_batched_ex.restype = ctypes.c_int
    lib.dion_step_batched_ex.argtypes = lib.dion_step_batched.argtypes + [ctypes.POINTER(StepOutputs)]
    f32, i32 = ctypes.c_float, ctypes.c_int
    lib.dion_step_batched_noalloc.restype = ctypes.c_int
    lib.dion_step_batched_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f32, f32, f32, i32, i32, vp,
                                              ctypes.c_uint32, vp]
    lib.dion_adamw_step.restype = ctypes.c_int
    lib.dion_adamw_step.argtypes = [vp, vp, vp, vp, i64, i64, f32, f32, f32, f32, f32, i32, i32, vp]
    lib.dion_lion_step.restype = ctypes.c_int
    lib.dion_lion_step.argtypes = [vp, vp, vp, i64, f32, f32, f32, f32, i32, i32, vp]
    lib.dion_lambda_max_workspace_size.restype = ctypes.c_size_t
    lib.dion_lambda_max_workspace_size.argtypes = [i64, i64, i32]
    lib.dion_lambda_max_batched.restype = ctypes.c_int
    lib.dion_lambda_max_batched.argtypes = [vp, i64, i64, vp, i32, i32, vp, vp, ctypes.c_size_t, vp]
    lib.dion_strerror.restype = ctypes.c_char_p
    lib.dion_strerror.argtypes = [ctypes.c_int]
    lib.dion_version.restype = ctypes.c_int
    lib.dion_version.argtypes = []
    _lib = lib
    return lib


def workspace_size(m: int, n: int, batch: int, rank: int) -> int:
    return int(load().dion_workspace_size(m, n, batch, rank))


def strerror(status: int) -> str:
    return load().dion_strerror(int(status)).decode()


def version() -> int:
    return int(load().dion_version())


def step_batched_raw(X: int, G: int, M: int, Q: int, m: int, n: int, batch: int, rank: int,
                     mu: float, lr: float, eps: float, x_dtype: int, g_dtype: int,
                     workspace: int, workspace_bytes: int, flags: int, options: int, stream: int,
                     events=None, rmmc: int = 0) -> int:
    """dion_step_batched (or, with ``events`` or ``rmmc``, the extended entry) with integer addresses.

    ``events``: sequence of NUM_PHASES + 1 hipEvent_t handles (ints); ``rmmc``: address of a
    device fp32 [batch] array for the momentum-change statistic.  Returns the status code.
    """
    args = (X or None, G or None, M or None, Q or None, m, n, batch, rank, mu, lr, eps, x_dtype, g_dtype,
            workspace or None, workspace_bytes, flags or None, options, stream or None)
    if events is None and not rmmc:
        return int(load().dion_step_batched(*args))
    out = StepOutputs()
    if events is not None:
        arr = (ctypes.c_void_p * (NUM_PHASES + 1))(*[int(e) for e in events])
        out.events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    out.rmmc = rmmc or None
    return int(load().dion_step_batched_ex(*args, ctypes.byref(out)))


def step_batched_noalloc_raw(X: int, G: int, M: int, Q: int, m: int, n: int, batch: int, rank: int,
                             mu: float, lr: float, eps: float, x_dtype: int, g_dtype: int, flags: int, options: int,
                             stream: int) -> int:
    """dion_step_batched_noalloc (the built-in scratch, no workspace) with integer addresses; returns the
    status code."""
    return int(load().dion_step_batched_noalloc(X or None, G or None, M or None, Q or None, m, n, batch, rank, mu,
                                                lr, eps, x_dtype, g_dtype, flags or None, options, stream or None))


def adamw_step_raw(param: int, grad: int, exp_avg: int, exp_avg_sq: int, n: int, t: int, lr: float, beta1: float,
                   beta2: float, eps: float, weight_decay: float, p_dtype: int, g_dtype: int, stream: int) -> int:
    """dion_adamw_step with integer addresses; returns the status code."""
    return int(load().dion_adamw_step(param or None, grad or None, exp_avg or None, exp_avg_sq or None, n, t,
                                      lr, beta1, beta2, eps, weight_decay, p_dtype, g_dtype, stream or None))


def lion_step_raw(param: int, grad: int, exp_avg: int, n: int, lr: float, beta1: float, beta2: float,
                  weight_decay: float, p_dtype: int, g_dtype: int, stream: int) -> int:
    """dion_lion_step with integer addresses; returns the status code."""
    return int(load().dion_lion_step(param or None, grad or None, exp_avg or None, n, lr, beta1, beta2,
                                     weight_decay, p_dtype, g_dtype, stream or None))


def lambda_max_workspace_size(r: int, batch: int, k: int) -> int:
    return int(load().dion_lambda_max_workspace_size(r, batch, k))


def lambda_max_raw(W: int, r: int, batch: int, V0: int, k: int, iters: int, lam: int, workspace: int,
                   workspace_bytes: int, stream: int) -> int:
    """dion_lambda_max_batched with integer addresses; returns the status code."""
    return int(load().dion_lambda_max_batched(W or None, r, batch, V0 or None, k, iters, lam or None,
                                              workspace or None, workspace_bytes, stream or None))
