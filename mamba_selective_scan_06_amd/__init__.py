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
FLAG_ZOH = 2
FLAG_CARRY_SCAN = 4
ABI_VERSION = 4  # SSM_SCAN_ABI_VERSION of include/ssm_scan.h

# Exported symbols the header declares (checked by the tests).
EXPORTS = ("ssm_scan_fwd", "ssm_scan_fwd_noalloc", "ssm_scan_workspace_bytes", "ssm_scan_plan",
           "ssm_scan_checkpoint_bytes", "ssm_scan_bwd",
           "ssm_scan_bwd_workspace_bytes", "ssm_scan_bwd_plan", "ssm_conv1d_silu_fwd", "ssm_ssd_fwd",
           "ssm_ssd_workspace_bytes", "ssm_ssd_plan", "ssm_gla_fwd", "ssm_gla_workspace_bytes", "ssm_gla_plan",
           "ssm_scan_strerror", "ssm_scan_abi_version")


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
        ("time_splits", ctypes.c_int32), ("checkpoints", ctypes.c_void_p),
    ]


class ScanBwdArgs(ctypes.Structure):
    """Mirror of ssm_scan_bwd_args in include/ssm_scan.h."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p), ("C", ctypes.c_void_p), ("D", ctypes.c_void_p),
        ("z", ctypes.c_void_p), ("delta_bias", ctypes.c_void_p), ("h0", ctypes.c_void_p),
        ("dy", ctypes.c_void_p), ("dhT", ctypes.c_void_p),
        ("dx", ctypes.c_void_p), ("ddelta", ctypes.c_void_p), ("dA", ctypes.c_void_p),
        ("dB", ctypes.c_void_p), ("dC", ctypes.c_void_p), ("dD", ctypes.c_void_p),
        ("dz", ctypes.c_void_p), ("ddelta_bias", ctypes.c_void_p), ("dh0", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
        ("time_splits", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("checkpoints", ctypes.c_void_p),
    ]


class ConvArgs(ctypes.Structure):
    """Mirror of ssm_conv_args in include/ssm_scan.h."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
        ("width", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("state", ctypes.c_void_p), ("u", ctypes.c_void_p), ("state_out", ctypes.c_void_p),
    ]


class SsdArgs(ctypes.Structure):
    """Mirror of ssm_ssd_args in include/ssm_scan.h."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("time_splits", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p), ("C", ctypes.c_void_p), ("D", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p), ("h0", ctypes.c_void_p), ("hT", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
    ]


class GlaArgs(ctypes.Structure):
    """Mirror of ssm_gla_args in include/ssm_scan.h."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("feature_map", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("log_f", ctypes.c_void_p), ("in_gate", ctypes.c_void_p),
        ("h0", ctypes.c_void_p), ("hT", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
        ("time_splits", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


# Gradient outputs of the backward: name of the input they belong to -> struct field.
GRAD_FIELDS = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
               "delta_bias": "ddelta_bias", "h0": "dh0"}

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
        L.ssm_scan_fwd_noalloc.argtypes = [P, ctypes.c_void_p]
        L.ssm_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssm_scan_workspace_bytes.argtypes = [P]
        L.ssm_scan_workspace_bytes.restype = ctypes.c_int64
        L.ssm_scan_plan.argtypes = [P]
        L.ssm_scan_plan.restype = ctypes.c_int64
        L.ssm_scan_checkpoint_bytes.argtypes = [P]
        L.ssm_scan_checkpoint_bytes.restype = ctypes.c_int64
        PB = ctypes.POINTER(ScanBwdArgs)
        L.ssm_scan_bwd.argtypes = [PB, ctypes.c_void_p]
        L.ssm_scan_bwd.restype = ctypes.c_int
        L.ssm_scan_bwd_workspace_bytes.argtypes = [PB]
        L.ssm_scan_bwd_workspace_bytes.restype = ctypes.c_int64
        L.ssm_scan_bwd_plan.argtypes = [PB]
        L.ssm_scan_bwd_plan.restype = ctypes.c_int64
        L.ssm_ssd_fwd.argtypes = [ctypes.POINTER(SsdArgs), ctypes.c_void_p]
        L.ssm_ssd_fwd.restype = ctypes.c_int
        L.ssm_gla_fwd.argtypes = [ctypes.POINTER(GlaArgs), ctypes.c_void_p]
        L.ssm_gla_fwd.restype = ctypes.c_int
        L.ssm_ssd_workspace_bytes.argtypes = [ctypes.POINTER(SsdArgs)]
        L.ssm_ssd_workspace_bytes.restype = ctypes.c_int64
        L.ssm_ssd_plan.argtypes = [ctypes.POINTER(SsdArgs)]
        L.ssm_ssd_plan.restype = ctypes.c_int
        L.ssm_gla_workspace_bytes.argtypes = [ctypes.POINTER(GlaArgs)]
        L.ssm_gla_workspace_bytes.restype = ctypes.c_int64
        L.ssm_gla_plan.argtypes = [ctypes.POINTER(GlaArgs)]
        L.ssm_gla_plan.restype = ctypes.c_int
        L.ssm_conv1d_silu_fwd.argtypes = [ctypes.POINTER(ConvArgs), ctypes.c_void_p]
        L.ssm_conv1d_silu_fwd.restype = ctypes.c_int
        L.ssm_scan_strerror.argtypes = [ctypes.c_int]
        L.ssm_scan_strerror.restype = ctypes.c_char_p
        L.ssm_scan_abi_version.argtypes = []
        L.ssm_scan_abi_version.restype = ctypes.c_int
        if L.ssm_scan_abi_version() != ABI_VERSION:
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
              workspace=None, variant="auto", time_splits=0, generic_a=False, zoh=False,
              carry_scan=False, checkpoints=None) -> ScanArgs:
    """Check shapes/dtypes/devices of torch tensors and fill an ssm_scan_args
    (zoh: zero-order-hold input term instead of the Euler one; checkpoints: a
    float32 tensor of checkpoint_shape(...) for the backward, or None)."""
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
    _check("checkpoints", checkpoints, checkpoint_shape(bsz, L, dim, N), f32, dev)
    if variant not in VARIANTS:
        raise ValueError(f"variant must be one of {sorted(VARIANTS)}")
    a = ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate = bsz, L, dim, N
    a.dtype = DTYPE_F32 if io == torch.float32 else DTYPE_BF16
    a.flags = (FLAG_GENERIC_A if generic_a else 0) | (FLAG_ZOH if zoh else 0) | (FLAG_CARRY_SCAN if carry_scan else 0)
    a.x, a.delta, a.A, a.B, a.C = _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C)
    a.D, a.z, a.delta_bias, a.h0, a.hT, a.y = _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(h0), _ptr(hT), _ptr(y)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.variant = VARIANTS[variant]
    a.time_splits = int(time_splits)
    a.checkpoints = _ptr(checkpoints)
    return a


def checkpoint_tokens(dstate: int) -> int:
    """Tokens between the checkpoints a forward writes for the backward."""
    return 16 if dstate <= 4 else 8


def checkpoint_shape(batch: int, seqlen: int, dim: int, dstate: int):
    """Shape of the checkpoints of one call: (B, ceil(L / T) - 1, 4, D, M),
    M = ceil(N / 4); entry i is the state after token (i + 1) T - 1, state n
    of channel d at [.., i, n // M, d, n % M]."""
    T = checkpoint_tokens(dstate)
    return (batch, max((seqlen + T - 1) // T - 1, 0), 4, dim, (dstate + 3) // 4)


def checkpoint_states(ck, dstate: int):
    """The states of checkpoints `ck` as a (B, entries, D, N) tensor."""
    b, e, _, dim, m = ck.shape
    return ck.permute(0, 1, 3, 2, 4).reshape(b, e, dim, 4 * m)[..., :dstate]


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
             variant="auto", time_splits=0, generic_a=False, zoh=False, carry_scan=False, checkpoints=None):
    """Selective scan forward on the GPU.  Returns y, or (y, hT) with
    return_final_state=True.  `final_state_out` may be h0 itself (in-place state
    update).  zoh=True discretises the input term with the zero-order hold,
    (exp(delta A) - 1) / A * B x, instead of delta B x.  carry_scan=True makes a
    time-split call compose the segment summaries with the wave-level
    associative scan launch instead of folding them serially in each block.
    `checkpoints` (a float32 tensor of checkpoint_shape(...)) receives the
    states the backward can start from (scan_bwd(..., checkpoints=...)).
    Launches on torch's current HIP stream and does not synchronise."""
    if not x.is_cuda:
        raise ValueError("scan_fwd runs on the GPU only: move the tensors to a HIP device")
    L_ = lib()
    y = out if out is not None else torch.empty_like(x)
    hT = final_state_out
    if hT is None and return_final_state:
        hT = torch.empty((x.shape[0], x.shape[2], A.shape[1]), dtype=torch.float32, device=x.device)
    args = make_args(x, delta, A, B, C, D, z, delta_bias, h0, hT, y, None, variant, time_splits, generic_a, zoh,
                     carry_scan, checkpoints)
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


def make_bwd_args(x, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, *, dy, dhT=None,
                  grads=None, workspace=None, time_splits=0, generic_a=False, zoh=False,
                  checkpoints=None) -> ScanBwdArgs:
    """Check shapes/dtypes/devices and fill an ssm_scan_bwd_args.  `grads` maps
    input names (x, delta, A, B, C, D, z, delta_bias, h0) to output tensors."""
    fa = make_args(x, delta, A, B, C, D, z, delta_bias, h0, generic_a=generic_a, zoh=zoh, checkpoints=checkpoints)
    bsz, L, dim = x.shape
    N = A.shape[1]
    io, dev, f32 = x.dtype, x.device, torch.float32
    _check("dy", dy, (bsz, L, dim), io, dev)
    _check("dhT", dhT, (bsz, dim, N), f32, dev)
    grads = grads or {}
    shapes = {"x": ((bsz, L, dim), io), "delta": ((bsz, L, dim), io), "A": ((dim, N), f32),
              "B": ((bsz, L, N), io), "C": ((bsz, L, N), io), "D": ((dim,), f32), "z": ((bsz, L, dim), io),
              "delta_bias": ((dim,), f32), "h0": ((bsz, dim, N), f32)}
    a = ScanBwdArgs()
    for f, _ in ScanArgs._fields_:
        if f in dict(ScanBwdArgs._fields_) and f not in ("workspace", "workspace_bytes", "time_splits"):
            # (checkpoints: the forward's, passed through as an input here)
            setattr(a, f, getattr(fa, f))
    a.dy, a.dhT = _ptr(dy), _ptr(dhT)
    for k, t in grads.items():
        if k not in GRAD_FIELDS:
            raise ValueError(f"no gradient for {k!r}")
        _check("d" + k, t, *shapes[k], dev)
        setattr(a, GRAD_FIELDS[k], _ptr(t))
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.time_splits = int(time_splits)
    a.reserved = 0
    return a


def bwd_workspace_bytes(args: ScanBwdArgs) -> int:
    r = lib().ssm_scan_bwd_workspace_bytes(ctypes.byref(args))
    if r < 0:
        raise RuntimeError(f"ssm_scan_bwd_workspace_bytes: {strerror(int(r))}")
    return int(r)


def bwd_plan(args: ScanBwdArgs) -> int:
    """Number of time segments the backward would use."""
    r = lib().ssm_scan_bwd_plan(ctypes.byref(args))
    if r < 0:
        raise RuntimeError(f"ssm_scan_bwd_plan: {strerror(int(r))}")
    return int(r)


def scan_bwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, *, dy, dhT=None,
             wanted=None, workspace=None, time_splits=0, generic_a=False, zoh=False, checkpoints=None):
    """Backward selective scan on the GPU: gradients of sum(dy * y) + sum(dhT * hT)
    with respect to the inputs, as a dict keyed like the inputs (x, delta, A, B,
    C, h0 always; D, z, delta_bias when given).  `wanted` restricts the outputs
    to those names; zoh=True differentiates the zero-order-hold forward;
    `checkpoints` are those a scan_fwd call on the same inputs wrote (the
    forward recurrence is then not run again).  Launches on torch's current HIP stream and does not
    synchronise."""
    if not x.is_cuda:
        raise ValueError("scan_bwd runs on the GPU only: move the tensors to a HIP device")
    L_ = lib()
    given = {"x": x, "delta": delta, "A": A, "B": B, "C": C, "D": D, "z": z, "delta_bias": delta_bias}
    names = ["x", "delta", "A", "B", "C", "h0"] + [k for k in ("D", "z", "delta_bias") if given[k] is not None]
    if wanted is not None:
        names = [k for k in names if k in set(wanted)]
    bsz, _, dim = x.shape
    N = A.shape[1]
    grads = {}
    for k in names:
        if k == "h0":
            grads[k] = torch.empty((bsz, dim, N), dtype=torch.float32, device=x.device)
        else:
            grads[k] = torch.empty_like(given[k])
    args = make_bwd_args(x, delta, A, B, C, D, z, delta_bias, h0, dy=dy, dhT=dhT, grads=grads,
                         time_splits=time_splits, generic_a=generic_a, zoh=zoh, checkpoints=checkpoints)
    if workspace is None:
        nbytes = L_.ssm_scan_bwd_workspace_bytes(ctypes.byref(args))
        if nbytes < 0:
            raise RuntimeError(f"ssm_scan_bwd: {strerror(int(nbytes))}")
        workspace = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=x.device)
    args.workspace = _ptr(workspace)
    args.workspace_bytes = workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = L_.ssm_scan_bwd(ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"ssm_scan_bwd: {strerror(rc)}")
    return grads


def make_conv_args(x, weight, bias=None, state=None, u=None, state_out=None) -> ConvArgs:
    """Check shapes/dtypes/devices and fill an ssm_conv_args."""
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be (B, L, D) and weight (D, W)")
    bsz, L, dim = x.shape
    W = weight.shape[1]
    io, dev, f32 = x.dtype, x.device, torch.float32
    if io not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _check("weight", weight, (dim, W), f32, dev)
    _check("bias", bias, (dim,), f32, dev)
    _check("state", state, (bsz, W - 1, dim), io, dev)
    _check("u", u, (bsz, L, dim), io, dev)
    _check("state_out", state_out, (bsz, W - 1, dim), io, dev)
    _check("x", x, (bsz, L, dim), io, dev)
    a = ConvArgs()
    a.batch, a.seqlen, a.dim, a.width = bsz, L, dim, W
    a.dtype = DTYPE_F32 if io == torch.float32 else DTYPE_BF16
    a.x, a.weight, a.bias, a.state = _ptr(x), _ptr(weight), _ptr(bias), _ptr(state)
    a.u, a.state_out = _ptr(u), _ptr(state_out)
    return a


def conv1d_silu(x, weight, bias=None, state=None, *, return_state=False, out=None, state_out=None):
    """Depthwise causal conv1d + SiLU on the GPU: u = SiLU(bias + sum_k weight[:, k] x[t-(W-1)+k]).
    `state` (B, W-1, D) carries the previous call's last W-1 input rows.  Returns u,
    or (u, state_out) with return_state=True.  Launches on torch's current HIP
    stream and does not synchronise."""
    if not x.is_cuda:
        raise ValueError("conv1d_silu runs on the GPU only: move the tensors to a HIP device")
    L_ = lib()
    u = out if out is not None else torch.empty_like(x)
    so = state_out
    if so is None and return_state:
        so = torch.empty((x.shape[0], weight.shape[1] - 1, x.shape[2]), dtype=x.dtype, device=x.device)
    args = make_conv_args(x, weight, bias, state, u, so)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = L_.ssm_conv1d_silu_fwd(ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"ssm_conv1d_silu_fwd: {strerror(rc)}")
    if return_state or state_out is not None:
        return u, so
    return u


def make_ssd_args(x, dt, A, B, C, D=None, dt_bias=None, h0=None, hT=None, y=None, time_splits=0) -> SsdArgs:
    """Check shapes/dtypes/devices and fill an ssm_ssd_args."""
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be (B, L, H, P) and B, C (B, L, G, N)")
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    bf, f32, dev = torch.bfloat16, torch.float32, x.device
    _check("x", x, (bsz, L, H, P), bf, dev)
    _check("dt", dt, (bsz, L, H), bf, dev)
    _check("A", A, (H,), f32, dev)
    _check("B", B, (bsz, L, G, N), bf, dev)
    _check("C", C, (bsz, L, G, N), bf, dev)
    _check("D", D, (H,), f32, dev)
    _check("dt_bias", dt_bias, (H,), f32, dev)
    _check("h0", h0, (bsz, H, P, N), f32, dev)
    _check("hT", hT, (bsz, H, P, N), f32, dev)
    _check("y", y, (bsz, L, H, P), bf, dev)
    a = SsdArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.ngroups, a.dstate = bsz, L, H, P, G, N
    a.dtype, a.time_splits = DTYPE_BF16, int(time_splits)
    a.x, a.dt, a.A, a.B, a.C = _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C)
    a.D, a.dt_bias, a.h0, a.hT, a.y = _ptr(D), _ptr(dt_bias), _ptr(h0), _ptr(hT), _ptr(y)
    return a


def _attach_workspace(args, query, workspace, device, name):
    """Size (query) and allocate a workspace when none is given; an empty tensor declines it."""
    if workspace is None:
        nbytes = query(ctypes.byref(args))
        if nbytes < 0:
            raise RuntimeError(f"{name}: {strerror(int(nbytes))}")
        if nbytes > 0:
            workspace = torch.empty(int(nbytes), dtype=torch.uint8, device=device)
    if workspace is not None and workspace.numel() > 0:
        args.workspace = _ptr(workspace)
        args.workspace_bytes = workspace.numel() * workspace.element_size()
    return workspace


def ssd_workspace_bytes(args: SsdArgs) -> int:
    """Bytes of workspace ssm_ssd_fwd uses for time-segment summaries (0: no split)."""
    r = lib().ssm_ssd_workspace_bytes(ctypes.byref(args))
    if r < 0:
        raise RuntimeError(f"ssm_ssd_workspace_bytes: {strerror(int(r))}")
    return int(r)


def ssd_plan(args: SsdArgs) -> int:
    """Time segments ssm_ssd_fwd would run with these arguments (1: no split)."""
    r = lib().ssm_ssd_plan(ctypes.byref(args))
    if r < 0:
        raise RuntimeError(f"ssm_ssd_plan: {strerror(int(r))}")
    return int(r)


def ssd_fwd(x, dt, A, B, C, D=None, dt_bias=None, h0=None, *, return_final_state=False, out=None,
            final_state_out=None, time_splits=0, workspace=None):
    """Mamba-2 SSD layer forward on the GPU (chunked matrix form on the matrix
    cores).  Returns y, or (y, hT) with return_final_state=True.  time_splits:
    0 lets the library cut the sequence into time segments when batch x heads
    leaves compute units idle, 1 never, S > 1 asks for S; the segment summaries
    go to `workspace` (allocated here when None; an empty tensor declines it).
    Launches on torch's current HIP stream and does not synchronise."""
    if not x.is_cuda:
        raise ValueError("ssd_fwd runs on the GPU only: move the tensors to a HIP device")
    L_ = lib()
    y = out if out is not None else torch.empty_like(x)
    hT = final_state_out
    if hT is None and return_final_state:
        hT = torch.empty((x.shape[0], x.shape[2], x.shape[3], B.shape[3]), dtype=torch.float32, device=x.device)
    args = make_ssd_args(x, dt, A, B, C, D, dt_bias, h0, hT, y, time_splits)
    _attach_workspace(args, L_.ssm_ssd_workspace_bytes, workspace, x.device, "ssm_ssd_fwd")
    stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = L_.ssm_ssd_fwd(ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"ssm_ssd_fwd: {strerror(rc)}")
    if return_final_state or final_state_out is not None:
        return y, hT
    return y


def make_gla_args(q, k, v, log_f=None, in_gate=None, h0=None, hT=None, y=None, feature_map=False,
                  time_splits=0) -> GlaArgs:
    """Check shapes/dtypes/devices and fill an ssm_gla_args."""
    if v.dim() != 4 or k.dim() != 4:
        raise ValueError("v must be (B, L, H, P) and q, k (B, L, G, N)")
    bsz, L, H, P = v.shape
    G, N = k.shape[2], k.shape[3]
    bf, f32, dev = torch.bfloat16, torch.float32, v.device
    _check("q", q, (bsz, L, G, N), bf, dev)
    _check("k", k, (bsz, L, G, N), bf, dev)
    _check("v", v, (bsz, L, H, P), bf, dev)
    _check("log_f", log_f, (bsz, L, H), f32, dev)
    _check("in_gate", in_gate, (bsz, L, H), f32, dev)
    _check("h0", h0, (bsz, H, P, N), f32, dev)
    _check("hT", hT, (bsz, H, P, N), f32, dev)
    _check("y", y, (bsz, L, H, P), bf, dev)
    a = GlaArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.ngroups, a.dstate = bsz, L, H, P, G, N
    a.dtype, a.feature_map = DTYPE_BF16, int(bool(feature_map))
    a.time_splits, a.reserved = int(time_splits), 0
    a.q, a.k, a.v, a.log_f, a.in_gate = _ptr(q), _ptr(k), _ptr(v), _ptr(log_f), _ptr(in_gate)
    a.h0, a.hT, a.y = _ptr(h0), _ptr(hT), _ptr(y)
    return a


def gla_workspace_bytes(args: GlaArgs) -> int:
    """Bytes of workspace ssm_gla_fwd uses: the feature map applied once per
    call, then the time-segment summaries."""
    r = lib().ssm_gla_workspace_bytes(ctypes.byref(args))
    if r < 0:
        raise RuntimeError(f"ssm_gla_workspace_bytes: {strerror(int(r))}")
    return int(r)


def gla_plan(args: GlaArgs) -> int:
    """Time segments ssm_gla_fwd would run with these arguments (1: no split)."""
    r = lib().ssm_gla_plan(ctypes.byref(args))
    if r < 0:
        raise RuntimeError(f"ssm_gla_plan: {strerror(int(r))}")
    return int(r)


def gla_fwd(q, k, v, log_f=None, in_gate=None, h0=None, *, feature_map=False, return_final_state=False, out=None,
            final_state_out=None, workspace=None, time_splits=0):
    """Gated linear attention / mLSTM matrix-state recurrence on the GPU:
    S_t = exp(log_f) S_{t-1} + in_gate v_t phi(k_t)^T, y_t = S_t phi(q_t), phi the
    identity or elu + 1 (feature_map=True).  Returns y, or (y, hT) with
    return_final_state=True.  A workspace (allocated here when None; an empty
    tensor declines it) lets the library apply phi once per call and hold the
    time-segment summaries (time_splits as for ssd_fwd).  Launches on torch's
    current HIP stream and does not synchronise."""
    if not v.is_cuda:
        raise ValueError("gla_fwd runs on the GPU only: move the tensors to a HIP device")
    L_ = lib()
    y = out if out is not None else torch.empty_like(v)
    hT = final_state_out
    if hT is None and return_final_state:
        hT = torch.empty((v.shape[0], v.shape[2], v.shape[3], k.shape[3]), dtype=torch.float32, device=v.device)
    args = make_gla_args(q, k, v, log_f, in_gate, h0, hT, y, feature_map, time_splits)
    _attach_workspace(args, L_.ssm_gla_workspace_bytes, workspace, v.device, "ssm_gla_fwd")
    stream = torch.cuda.current_stream(v.device).cuda_stream
    rc = L_.ssm_gla_fwd(ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"ssm_gla_fwd: {strerror(rc)}")
    if return_final_state or final_state_out is not None:
        return y, hT
    return y


__all__ = ["scan_fwd", "scan_bwd", "conv1d_silu", "ssd_fwd", "gla_fwd", "make_gla_args", "GlaArgs", "gla_workspace_bytes", "gla_plan", "make_ssd_args", "SsdArgs", "ssd_workspace_bytes", "ssd_plan", "make_conv_args", "ConvArgs", "make_args", "make_bwd_args", "plan", "bwd_plan", "workspace_bytes",
           "bwd_workspace_bytes", "checkpoint_shape", "checkpoint_states", "checkpoint_tokens", "lib", "strerror", "ScanArgs", "ScanBwdArgs", "EXPORTS"]
