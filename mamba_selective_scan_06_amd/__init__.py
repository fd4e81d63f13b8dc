"""MI355X (gfx950) selective-SSM scan: thin Python binding over libssm_scan.so.

Every step of the scan runs in the library's HIP kernels.  This module only
checks and marshals arguments (torch tensors -> device pointers, shapes,
dtype, the current HIP stream), allocates outputs and the time-split
workspace with torch, and raises on a non-zero status.  There is no CPU or
PyTorch fallback: if the library is not built or cannot be loaded, import of
the scan entry points fails loudly.

The operation (page youngju.dev "Mamba 논문 리뷰", sections 2.2, 3.1, 3.3, 3.4):
    delta = softplus(delta_raw + delta_bias)
    h_t   = exp(delta A) * h_{t-1} + delta * B_t * x_t       (per channel d, state n)
    y_t   = (C_t . h_t + D * x_t) * SiLU(z_t)
with x, delta, z of shape (B, L, D), A (D, N), B and C (B, L, N), D and
delta_bias (D), h0/hT (B, D, N) fp32.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm_scan.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "ssm_scan.h")

DTYPE_F32, DTYPE_BF16 = 0, 1
VARIANTS = {"auto": 0, "nsplit": 1, "lane": 2, "decode": 3}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}
FLAG_GENERIC_A = 1

# Exported symbols the header declares (checked by the tests).
EXPORTS = ("ssm_scan_fwd", "ssm_scan_workspace_bytes", "ssm_scan_plan", "ssm_scan_strerror",
           "ssm_scan_abi_version")


class ScanArgs(ctypes.Structure):
    """Mirror of ssm_scan_args in include/ssm_scan.h."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p), ("C", ctypes.c_void_p), ("D", ctypes.c_void_p),
        ("z", ctypes.c_void_p), ("delta_bias", ctypes.c_void_p), ("h0", ctypes.c_void_p),
        ("hT", ctypes.c_void_p), ("y", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_int64), ("variant", ctypes.c_int32),
        ("time_splits", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mamba_selective_scan_06_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(ScanArgs)
        L.ssm_scan_fwd.argtypes = [P, ctypes.c_void_p]
        L.ssm_scan_fwd.restype = ctypes.c_int
        L.ssm_scan_workspace_bytes.argtypes = [P]
        L.ssm_scan_workspace_bytes.restype = ctypes.c_int64
        L.ssm_scan_plan.argtypes = [P]
        L.ssm_scan_plan.restype = ctypes.c_int64
        L.ssm_scan_strerror.argtypes = [ctypes.c_int]
        L.ssm_scan_strerror.restype = ctypes.c_char_p
        L.ssm_scan_abi_version.argtypes = []
        L.ssm_scan_abi_version.restype = ctypes.c_int
        if L.ssm_scan_abi_version() != 1:
            raise RuntimeError("libssm_scan ABI version mismatch")
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().ssm_scan_strerror(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(name, t, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_args(x, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, hT=None, y=None,
              workspace=None, variant="auto", time_splits=0, generic_a=False) -> ScanArgs:
    """Check shapes/dtypes/devices of torch tensors and fill an ssm_scan_args."""
    if x.dim() != 3:
        raise ValueError("x must be (B, L, D)")
    bsz, L, dim = x.shape
    if A.dim() != 2 or A.shape[0] != dim:
        raise ValueError("A must be (D, N)")
    N = A.shape[1]
    io = x.dtype
    if io not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    f32 = torch.float32
    _check("x", x, (bsz, L, dim), io, dev)
    _check("delta", delta, (bsz, L, dim), io, dev)
    _check("A", A, (dim, N), f32, dev)
    _check("B", B, (bsz, L, N), io, dev)
    _check("C", C, (bsz, L, N), io, dev)
    _check("D", D, (dim,), f32, dev)
    _check("z", z, (bsz, L, dim), io, dev)
    _check("delta_bias", delta_bias, (dim,), f32, dev)
    _check("h0", h0, (bsz, dim, N), f32, dev)
    _check("hT", hT, (bsz, dim, N), f32, dev)
    _check("y", y, (bsz, L, dim), io, dev)
    if variant not in VARIANTS:
        raise ValueError(f"variant must be one of {sorted(VARIANTS)}")
    a = ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate = bsz, L, dim, N
    a.dtype = DTYPE_F32 if io == torch.float32 else DTYPE_BF16
    a.flags = FLAG_GENERIC_A if generic_a else 0
    a.x, a.delta, a.A, a.B, a.C = _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C)
    a.D, a.z, a.delta_bias, a.h0, a.hT, a.y = _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(h0), _ptr(hT), _ptr(y)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.variant = VARIANTS[variant]
    a.time_splits = int(time_splits)
    return a


def plan(args: ScanArgs):
    """(variant name, time splits) the library would use for these arguments."""
    r = lib().ssm_scan_plan(ctypes.byref(args))
    if r < 0:
        raise RuntimeError(f"ssm_scan_plan: {strerror(int(r))}")
    return VARIANT_NAMES[int(r) // 65536], int(r) % 65536


def workspace_bytes(args: ScanArgs) -> int:
    r = lib().ssm_scan_workspace_bytes(ctypes.byref(args))
    if r < 0:
        raise RuntimeError(f"ssm_scan_workspace_bytes: {strerror(int(r))}")
    return int(r)


def scan_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, *,
             return_final_state=False, out=None, final_state_out=None, workspace=None,
             variant="auto", time_splits=0, generic_a=False):
    """Selective scan forward on the GPU.  Returns y, or (y, hT) with
    return_final_state=True.  `final_state_out` may be h0 itself (in-place state
    update).  Launches on torch's current HIP stream and does not synchronise."""
    if not x.is_cuda:
        raise ValueError("scan_fwd runs on the GPU only: move the tensors to a HIP device")
    L_ = lib()
    y = out if out is not None else torch.empty_like(x)
    hT = final_state_out
    if hT is None and return_final_state:
        hT = torch.empty((x.shape[0], x.shape[2], A.shape[1]), dtype=torch.float32, device=x.device)
    args = make_args(x, delta, A, B, C, D, z, delta_bias, h0, hT, y, None, variant, time_splits, generic_a)
    if workspace is None:
        nbytes = L_.ssm_scan_workspace_bytes(ctypes.byref(args))
        if nbytes < 0:
            raise RuntimeError(f"ssm_scan_fwd: {strerror(int(nbytes))}")
        if nbytes > 0:
            workspace = torch.empty(int(nbytes), dtype=torch.uint8, device=x.device)
    if workspace is not None:
        args.workspace = _ptr(workspace)
        args.workspace_bytes = workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = L_.ssm_scan_fwd(ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"ssm_scan_fwd: {strerror(rc)}")
    if return_final_state or final_state_out is not None:
        return y, hT
    return y


__all__ = ["scan_fwd", "make_args", "plan", "workspace_bytes", "lib", "strerror", "ScanArgs", "EXPORTS"]
