"""The SSD layer's C ABI on the CPU: argument checks that fail on the host
before any HIP call (fake, aligned, never dereferenced pointers)."""
import ctypes

import pytest

import mamba_selective_scan_06_amd as ssm

FAKE = 0x7F0000000000


def _args(**kw):
    a = ssm.SsdArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.ngroups, a.dstate = kw.pop("shape", (2, 64, 8, 64, 2, 128))
    a.dtype = kw.pop("dtype", 1)
    a.reserved = kw.pop("reserved", 0)
    base = FAKE
    for name in ("x", "dt", "A", "B", "C", "D", "dt_bias", "h0", "hT", "y"):
        setattr(a, name, kw.pop(name, base))
        base += 1 << 32
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _ssd(a):
    return ssm.lib().ssm_ssd_fwd(ctypes.byref(a), None)


@pytest.mark.parametrize("mut,code", [
    (dict(shape=(-1, 64, 8, 64, 2, 128)), -2),
    (dict(shape=(2, 64, 0, 64, 1, 128)), -2),
    (dict(shape=(70000, 64, 8, 64, 2, 128)), -2),
    (dict(shape=(2**40, 2**20, 2**10, 64, 1, 128)), -2),
    (dict(dtype=0), -9),              # fp32 not in this version
    (dict(dtype=5), -4),
    (dict(shape=(2, 64, 8, 32, 2, 128)), -9),   # headdim 32
    (dict(shape=(2, 64, 8, 64, 3, 128)), -9),   # groups must divide heads
    (dict(shape=(2, 64, 8, 64, 2, 96)), -9),    # dstate 96
    (dict(reserved=1), -9),
    (dict(x=0), -1), (dict(dt=0), -1), (dict(A=0), -1), (dict(B=0), -1), (dict(C=0), -1), (dict(y=0), -1),
    (dict(x=FAKE + 2), -5), (dict(h0=FAKE + 8), -5),
])
def test_invalid_arguments_rejected_on_host(mut, code):
    assert _ssd(_args(**mut)) == code


def test_aliasing_rejected():
    a = _args()
    a.y = a.x
    assert _ssd(a) == -6
    a = _args()
    a.hT = a.h0
    assert _ssd(a) == -6
    a = _args()
    a.hT = a.y
    assert _ssd(a) == -6


def test_null_args_and_empty_batch():
    assert ssm.lib().ssm_ssd_fwd(None, None) == -1
    assert _ssd(_args(shape=(0, 64, 8, 64, 2, 128))) == 0
