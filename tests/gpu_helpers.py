"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and the fp64 oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import os

import numpy as np
import torch

import mamba_selective_scan_06_amd as ssm
import oracle
import workloads

DEV = "cuda:0"
TENSORS = ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")


def to_dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


def gpu_scan(dinp, **kw):
    """(y, hT) from the HIP kernels, as float64 numpy arrays."""
    y, hT = ssm.scan_fwd(dinp["x"], dinp["delta"], dinp["A"], dinp["B"], dinp["C"], dinp.get("D"),
                         dinp.get("z"), dinp.get("delta_bias"), dinp.get("h0"), return_final_state=True, **kw)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy(), hT.cpu().double().numpy()


# oracle threads: the host's share of a one-GPU machine is 16 cores
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def oracle_scan(inp, **kw):
    kw.setdefault("threads", ORACLE_THREADS)
    return oracle.scan(*(inp.get(k) for k in TENSORS), **kw)


def select(inp, bidx, didx):
    """Sub-problem on batch rows bidx and channels didx (chains are independent)."""
    bi = torch.as_tensor(bidx, dtype=torch.long)
    di = torch.as_tensor(didx, dtype=torch.long)
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
        elif k in ("x", "delta", "z"):
            out[k] = v.index_select(0, bi).index_select(2, di)
        elif k in ("B", "C"):
            out[k] = v.index_select(0, bi)
        elif k == "A":
            out[k] = v.index_select(0, di)
        elif k in ("D", "delta_bias"):
            out[k] = v.index_select(0, di)
        elif k == "h0":
            out[k] = v.index_select(0, bi).index_select(1, di)
    return out


def check(name, got, ref, dtype):
    tol = workloads.tolerance(dtype)
    err = workloads.rel_err(got, ref)
    mabs = float(np.max(np.abs(np.asarray(got) - np.asarray(ref)))) if np.size(ref) else 0.0
    print(f"  {name}: rel_err={err:.3e} max_abs={mabs:.3e} tol={tol:g}", flush=True)
    assert err <= tol, f"{name}: rel_err {err:.3e} > {tol}"
    return err


def sample_channels(dim, k=48, seed=0):
    """Channels spanning block edges (0, 63, 64, ...), the last channel, and random ones."""
    g = np.random.default_rng(seed)
    edge = [0, 1, 63, 64, 65, 127, 128, dim - 65, dim - 64, dim - 2, dim - 1]
    rnd = g.choice(dim, size=min(k, dim), replace=False).tolist()
    return sorted({c for c in edge + rnd if 0 <= c < dim})
