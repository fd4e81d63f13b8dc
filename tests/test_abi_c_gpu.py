"""A C program that calls libssm_scan.so through its C ABI alone (hipMalloc,
plain device pointers, its own HIP stream; no Python or torch on its side)
gives the oracle's results.

The program (tests/abi_c/scan_abi_check.cpp, compiled by the build step next
to its source) reads raw input files that this test writes from the shared
seeded generator, and writes y and hT back.  It also checks that a missing x is
rejected with SSM_ERR_NULL and that the library's ABI version matches the
header it was compiled against.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import check, oracle_scan

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_c", "scan_abi_check")


def _raw(t: torch.Tensor) -> bytes:
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().tobytes()
    return t.to(torch.float32).numpy().tobytes()


def _run(tmp_path, inp, dtype):
    if not os.path.exists(EXE):
        raise RuntimeError(f"{EXE} is not built: run __graft_entry__.build() first")
    files = {"x": "x", "delta": "delta", "A": "A", "B": "B", "C": "C", "D": "D", "z": "z",
             "delta_bias": "bias", "h0": "h0"}
    for k, name in files.items():
        if inp.get(k) is not None:
            (tmp_path / f"{name}.bin").write_bytes(_raw(inp[k]))
    Bn, L, D = inp["x"].shape
    N = inp["A"].shape[1]
    code = 0 if dtype == torch.float32 else 1
    print(f"  scan_abi_check B={Bn} L={L} D={D} N={N} dtype={code}", flush=True)
    r = subprocess.run([EXE, str(tmp_path), str(Bn), str(L), str(D), str(N), str(code)],
                       capture_output=True, text=True, timeout=60)
    print(r.stdout.strip(), r.stderr.strip(), flush=True)
    assert r.returncode == 0, f"exit {r.returncode}: {r.stderr}"
    yb = (tmp_path / "y.bin").read_bytes()
    if dtype == torch.float32:
        y = np.frombuffer(yb, dtype=np.float32)
    else:
        y = torch.from_numpy(np.frombuffer(yb, dtype=np.int16).copy()).view(torch.bfloat16).float().numpy()
    hT = np.frombuffer((tmp_path / "hT.bin").read_bytes(), dtype=np.float32)
    return y.reshape(Bn, L, D).astype(np.float64), hT.reshape(Bn, D, N).astype(np.float64), r.stdout


CASES = [
    # (workload index, shape overrides, drop): fp32 at full size; bf16 ragged;
    # bf16 long enough on few channels that the plan splits time (workspace > 0)
    (0, dict(), ()),
    (1, dict(batch=2, seqlen=333, dim=200), ()),
    (1, dict(batch=1, seqlen=4096, dim=128), ("z",)),
]


@pytest.mark.parametrize("wi,shape,drop", CASES, ids=["fp32-full", "bf16-ragged", "bf16-split"])
def test_c_caller_matches_oracle(tmp_path, wi, shape, drop):
    w = workloads.WORKLOADS[wi]
    inp = workloads.make_inputs(w, **shape)
    for k in drop:
        inp[k] = None
    g = np.random.default_rng(11)
    Bn, _, D = inp["x"].shape
    inp["h0"] = torch.from_numpy(g.normal(0, 0.5, size=(Bn, D, w.dstate)).astype(np.float32))
    y, hT, out = _run(tmp_path, inp, w.dtype)
    if wi == 1 and shape["seqlen"] == 4096:
        plan = int(out.split("plan=")[1].split()[0])
        ws = int(out.split("workspace=")[1].split()[0])
        assert ws > 0 and plan % 65536 > 1, f"expected a time-split plan with a workspace, got {out!r}"
    yr, hr = oracle_scan(inp)
    check("y", y, yr, w.dtype)
    check("hT", hT, hr, w.dtype)
