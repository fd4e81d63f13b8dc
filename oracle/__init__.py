"""Plain fp64 CPU oracle for the selective-SSM scan (ctypes over ssm_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the HIP implementation; both sides receive the same seeded inputs
from the `workloads` module.

The arithmetic lives in ssm_oracle.c, which cites the passages it follows
(page "Mamba 논문 리뷰: Selective State Space Models로 Transformer를 넘어서",
sections 2.2, 3.1, 3.3 and 3.4).  This wrapper only widens inputs to fp64,
lays them out densely and calls the C entry points.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_BUILD = os.path.join(_HERE, "_build")

_dp = ctypes.POINTER(ctypes.c_double)


class _Args(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("x", _dp), ("delta", _dp), ("A", _dp), ("Bm", _dp), ("Cm", _dp),
        ("Dskip", _dp), ("z", _dp), ("delta_bias", _dp), ("h0", _dp),
        ("y", _dp), ("hT", _dp),
    ]


class _Grads(ctypes.Structure):
    _fields_ = [
        ("dy", _dp), ("dhT", _dp),
        ("dx", _dp), ("ddelta", _dp), ("dA", _dp), ("dB", _dp), ("dC", _dp),
        ("dD", _dp), ("dz", _dp), ("ddelta_bias", _dp), ("dh0", _dp),
    ]


class _SsdArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("x", _dp), ("dt", _dp), ("A", _dp), ("Bm", _dp), ("Cm", _dp),
        ("Dskip", _dp), ("dt_bias", _dp), ("s0", _dp), ("y", _dp), ("sT", _dp),
    ]


class _GlaArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("feature_map", ctypes.c_int64),
        ("q", _dp), ("k", _dp), ("v", _dp), ("log_f", _dp), ("in_gate", _dp), ("s0", _dp),
        ("y", _dp), ("sT", _dp),
    ]


def lib_path(mutant: int = 0, out_dir: str | None = None) -> str:
    d = out_dir or _BUILD
    name = "liboracle.so" if mutant == 0 else f"liboracle_mutant{mutant}.so"
    return os.path.join(d, name)


def build(mutant: int = 0, out_dir: str | None = None) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE fp64 throughout)."""
    out = lib_path(mutant, out_dir)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", f"-DORACLE_MUTANT={int(mutant)}", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """Handle on one compiled oracle library (the real one, or a test mutant)."""

    def __init__(self, path: str):
        self.path = path
        self._lib = ctypes.CDLL(path)
        self._lib.oracle_scan_f64.argtypes = [ctypes.POINTER(_Args), ctypes.c_int]
        self._lib.oracle_scan_f64.restype = ctypes.c_int
        self._lib.oracle_scan_zoh_f64.argtypes = [ctypes.POINTER(_Args), ctypes.c_int]
        self._lib.oracle_scan_zoh_f64.restype = ctypes.c_int
        self._lib.oracle_assoc_scan_f64.argtypes = [ctypes.POINTER(_Args)]
        self._lib.oracle_assoc_scan_f64.restype = ctypes.c_int
        self._lib.oracle_scan_bwd_f64.argtypes = [ctypes.POINTER(_Args), ctypes.POINTER(_Grads)]
        self._lib.oracle_scan_bwd_f64.restype = ctypes.c_int
        self._lib.oracle_scan_bwd_zoh_f64.argtypes = [ctypes.POINTER(_Args), ctypes.POINTER(_Grads)]
        self._lib.oracle_scan_bwd_zoh_f64.restype = ctypes.c_int
        i64 = ctypes.c_int64
        self._lib.oracle_ssd_f64.argtypes = [ctypes.POINTER(_SsdArgs)]
        self._lib.oracle_ssd_f64.restype = ctypes.c_int
        self._lib.oracle_gla_f64.argtypes = [ctypes.POINTER(_GlaArgs)]
        self._lib.oracle_gla_f64.restype = ctypes.c_int
        self._lib.oracle_conv1d_silu_f64.argtypes = [i64, i64, i64, i64, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        self._lib.oracle_conv1d_silu_f64.restype = ctypes.c_int
        self._lib.oracle_softplus_vec.argtypes = [_dp, _dp, ctypes.c_int64]
        self._lib.oracle_softplus_vec.restype = None
        self._lib.oracle_mutant_id.restype = ctypes.c_int
        self.mutant = self._lib.oracle_mutant_id()

    # -- helpers -------------------------------------------------------------
    @staticmethod
    def _f64(a):
        if a is None:
            return None
        if hasattr(a, "detach"):  # torch tensor (CPU): widen exactly
            a = a.detach().cpu().to(dtype=__import__("torch").float64).numpy()
        return np.ascontiguousarray(np.asarray(a, dtype=np.float64))

    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data_as(_dp)

    def _pack(self, x, delta, A, B, C, D, z, delta_bias, h0, want_state):
        x, delta, A, B, C = (self._f64(t) for t in (x, delta, A, B, C))
        D, z, delta_bias, h0 = (self._f64(t) for t in (D, z, delta_bias, h0))
        bsz, L, dim = x.shape
        N = A.shape[1]
        assert delta.shape == x.shape and A.shape == (dim, N)
        assert B.shape == (bsz, L, N) and C.shape == (bsz, L, N)
        assert D is None or D.shape == (dim,)
        assert z is None or z.shape == x.shape
        assert delta_bias is None or delta_bias.shape == (dim,)
        assert h0 is None or h0.shape == (bsz, dim, N)
        y = np.zeros((bsz, L, dim), dtype=np.float64)
        hT = np.zeros((bsz, dim, N), dtype=np.float64) if want_state else None
        keep = (x, delta, A, B, C, D, z, delta_bias, h0, y, hT)
        args = _Args(bsz, L, dim, N, *(self._ptr(t) for t in keep))
        return args, keep, y, hT

    # -- entry points --------------------------------------------------------
    def scan(self, x, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None,
             threads: int | None = None, timing: dict | None = None, zoh: bool = False):
        """Sequential fp64 scan.  Returns (y, hT) as float64 numpy arrays.
        zoh=True uses the zero-order-hold input term instead of the Euler one.
        If `timing` is a dict, the wall time of the C call alone (inputs already
        widened to fp64) and the thread count are stored in it."""
        args, keep, y, hT = self._pack(x, delta, A, B, C, D, z, delta_bias, h0, True)
        nt = threads if threads is not None else (os.cpu_count() or 1)
        t0 = time.perf_counter()
        fn = self._lib.oracle_scan_zoh_f64 if zoh else self._lib.oracle_scan_f64
        rc = fn(ctypes.byref(args), int(nt))
        t1 = time.perf_counter()
        if rc != 0:
            raise RuntimeError("oracle_scan_f64 failed")
        if timing is not None:
            timing["seconds"] = t1 - t0
            timing["threads"] = int(nt)
        del keep
        return y, hT

    def assoc_scan(self, x, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None):
        """Associative-scan twin (log-depth prefix over (a, b) pairs); small inputs."""
        args, keep, y, hT = self._pack(x, delta, A, B, C, D, z, delta_bias, h0, True)
        rc = self._lib.oracle_assoc_scan_f64(ctypes.byref(args))
        if rc != 0:
            raise RuntimeError("oracle_assoc_scan_f64 failed")
        del keep
        return y, hT

    def scan_bwd(self, x, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, *, dy, dhT=None,
                 zoh: bool = False):
        """Gradients of the scalar loss sum(dy * y) + sum(dhT * hT) with respect
        to every input, as a dict of float64 numpy arrays (keys x, delta, A, B,
        C, D, z, delta_bias, h0; an absent optional input has no entry, except
        h0, whose gradient is always returned).  zoh=True differentiates the
        zero-order-hold forward."""
        args, keep, _, _ = self._pack(x, delta, A, B, C, D, z, delta_bias, h0, False)
        xx, dd, AA, BB, CC, DD, zz, bb, hh = keep[:9]
        dy = self._f64(dy)
        dhT = self._f64(dhT)
        assert dy.shape == xx.shape and (dhT is None or dhT.shape == (xx.shape[0], xx.shape[2], AA.shape[1]))
        out = {"x": np.zeros_like(xx), "delta": np.zeros_like(dd), "A": np.zeros_like(AA),
               "B": np.zeros_like(BB), "C": np.zeros_like(CC),
               "h0": np.zeros((xx.shape[0], xx.shape[2], AA.shape[1]), dtype=np.float64)}
        if DD is not None:
            out["D"] = np.zeros_like(DD)
        if zz is not None:
            out["z"] = np.zeros_like(zz)
        if bb is not None:
            out["delta_bias"] = np.zeros_like(bb)
        p = self._ptr
        g = _Grads(p(dy), p(dhT), p(out["x"]), p(out["delta"]), p(out["A"]), p(out["B"]), p(out["C"]),
                   p(out.get("D")), p(out.get("z")), p(out.get("delta_bias")), p(out["h0"]))
        fn = self._lib.oracle_scan_bwd_zoh_f64 if zoh else self._lib.oracle_scan_bwd_f64
        rc = fn(ctypes.byref(args), ctypes.byref(g))
        if rc != 0:
            raise RuntimeError("oracle_scan_bwd_f64 failed")
        del keep
        return out

    def conv1d_silu(self, x, w, bias=None, state=None):
        """Depthwise causal conv1d + SiLU over x (B, L, D) with taps w (D, W),
        optional bias (D) and state (B, W-1, D) (the previous call's last W-1
        input rows).  Returns (u, pre, state_out) as float64 numpy arrays."""
        x = self._f64(x)
        w = self._f64(w)
        bias = self._f64(bias)
        state = self._f64(state)
        Bn, L, D = x.shape
        W = w.shape[1]
        assert w.shape == (D, W) and (bias is None or bias.shape == (D,))
        assert state is None or state.shape == (Bn, W - 1, D)
        u = np.empty_like(x)
        pre = np.empty_like(x)
        state_out = np.empty((Bn, W - 1, D), dtype=np.float64)
        p = self._ptr
        rc = self._lib.oracle_conv1d_silu_f64(Bn, L, D, W, p(x), p(w), p(bias), p(state), p(pre), p(u),
                                             p(state_out))
        if rc != 0:
            raise RuntimeError("oracle_conv1d_silu_f64 failed")
        return u, pre, state_out

    def ssd(self, x, dt, A, B, C, D=None, dt_bias=None, s0=None):
        """Mamba-2 SSD layer, recurrent form: x (B, L, H, P), dt (B, L, H), A (H),
        B and C (B, L, G, N), D and dt_bias (H), s0 (B, H, P, N).  Returns
        (y, sT) as float64 numpy arrays."""
        x, dt, A, B, C = (self._f64(t) for t in (x, dt, A, B, C))
        D, dt_bias, s0 = (self._f64(t) for t in (D, dt_bias, s0))
        Bn, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        assert dt.shape == (Bn, L, H) and A.shape == (H,) and B.shape == C.shape == (Bn, L, G, N)
        assert s0 is None or s0.shape == (Bn, H, P, N)
        y = np.empty_like(x)
        sT = np.empty((Bn, H, P, N), dtype=np.float64)
        p = self._ptr
        a = _SsdArgs(Bn, L, H, P, G, N, p(x), p(dt), p(A), p(B), p(C), p(D), p(dt_bias), p(s0), p(y), p(sT))
        if self._lib.oracle_ssd_f64(ctypes.byref(a)) != 0:
            raise RuntimeError("oracle_ssd_f64 failed")
        return y, sT

    def gla(self, q, k, v, log_f=None, in_gate=None, s0=None, feature_map=False):
        """Gated linear attention / mLSTM recurrence: q and k (B, L, G, N), v
        (B, L, H, P), log_f and in_gate (B, L, H), s0 (B, H, P, N); feature_map
        applies elu + 1 to q and k.  Returns (y, sT) as float64 numpy arrays."""
        q, k, v = (self._f64(t) for t in (q, k, v))
        log_f, in_gate, s0 = (self._f64(t) for t in (log_f, in_gate, s0))
        Bn, L, H, P = v.shape
        G, N = k.shape[2], k.shape[3]
        assert q.shape == k.shape == (Bn, L, G, N)
        assert log_f is None or log_f.shape == (Bn, L, H)
        assert in_gate is None or in_gate.shape == (Bn, L, H)
        assert s0 is None or s0.shape == (Bn, H, P, N)
        y = np.empty_like(v)
        sT = np.empty((Bn, H, P, N), dtype=np.float64)
        p = self._ptr
        a = _GlaArgs(Bn, L, H, P, G, N, int(bool(feature_map)), p(q), p(k), p(v), p(log_f), p(in_gate), p(s0),
                     p(y), p(sT))
        if self._lib.oracle_gla_f64(ctypes.byref(a)) != 0:
            raise RuntimeError("oracle_gla_f64 failed")
        return y, sT

    def softplus(self, v):
        v = self._f64(v)
        out = np.empty_like(v)
        self._lib.oracle_softplus_vec(self._ptr(v), self._ptr(out), v.size)
        return out


_lock = threading.Lock()
_default: Oracle | None = None


def get(rebuild: bool = False) -> Oracle:
    """The oracle, building it with gcc on first use if it is not built."""
    global _default
    with _lock:
        if _default is None or rebuild:
            path = lib_path()
            if rebuild or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
                build()
            _default = Oracle(path)
        return _default


def scan(*args, **kw):
    return get().scan(*args, **kw)


def assoc_scan(*args, **kw):
    return get().assoc_scan(*args, **kw)


def scan_bwd(*args, **kw):
    return get().scan_bwd(*args, **kw)


def conv1d_silu(*args, **kw):
    return get().conv1d_silu(*args, **kw)


def ssd(*args, **kw):
    return get().ssd(*args, **kw)


def gla(*args, **kw):
    return get().gla(*args, **kw)


def softplus(v):
    return get().softplus(v)
