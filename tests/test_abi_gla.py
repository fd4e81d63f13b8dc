"""The gated-linear-attention entry point's C ABI on the CPU: argument checks
that fail on the host before any HIP call (fake, aligned, never dereferenced
pointers)."""
import ctypes

import pytest

import mamba_selective_scan_06_amd as ssm

FAKE = 0x7F0000000000


def _args(**kw):
    a = ssm.GlaArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.ngroups, a.dstate = kw.pop("shape", (2, 64, 8, 64, 2, 128))
    a.dtype = kw.pop("dtype", 1)
    a.feature_map = kw.pop("feature_map", 0)
    base = FAKE
    for name in ("q", "k", "v", "log_f", "in_gate", "h0", "hT", "y"):
        setattr(a, name, kw.pop(name, base))
        base += 1 << 32
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _gla(a):
    return ssm.lib().ssm_gla_fwd(ctypes.byref(a), None)


@pytest.mark.parametrize("mut,code", [
    (dict(shape=(-1, 64, 8, 64, 2, 128)), -2),
    (dict(shape=(2, 64, 0, 64, 1, 128)), -2),
    (dict(shape=(70000, 64, 8, 64, 2, 128)), -2),
    (dict(shape=(2**40, 2**20, 2**10, 64, 1, 128)), -2),
    (dict(dtype=0), -9),              # fp32 not in this version
    (dict(dtype=5), -4),
    (dict(feature_map=2), -9),
    (dict(feature_map=-1), -9),
    (dict(shape=(2, 64, 8, 128, 2, 128)), -9),  # headdim 128
    (dict(shape=(2, 64, 8, 64, 3, 128)), -9),   # groups must divide heads
    (dict(shape=(2, 64, 8, 64, 2, 32)), -9),    # dstate 32
    (dict(reserved=1), -9), (dict(time_splits=-1), -9), (dict(time_splits=65536), -9),
    (dict(q=0), -1), (dict(k=0), -1), (dict(v=0), -1), (dict(y=0), -1),
    (dict(v=FAKE + 2), -5), (dict(log_f=FAKE + 4), -5), (dict(hT=FAKE + 8), -5),
])
def test_invalid_arguments_rejected_on_host(mut, code):
    assert _gla(_args(**mut)) == code


def test_optional_inputs_may_be_null():
    # with no tokens nothing is launched, so fake pointers and NULL gates pass the checks
    assert _gla(_args(shape=(0, 64, 8, 64, 2, 128), log_f=0, in_gate=0, h0=0, hT=0)) == 0


def test_aliasing_rejected():
    for src, dst in (("v", "y"), ("q", "y"), ("log_f", "y"), ("h0", "hT"), ("in_gate", "hT"), ("y", "hT")):
        a = _args()
        setattr(a, dst, getattr(a, src))
        assert _gla(a) == -6, (src, dst)


def test_null_args_and_empty_batch():
    assert ssm.lib().ssm_gla_fwd(None, None) == -1
    assert _gla(_args(shape=(0, 64, 8, 64, 2, 128))) == 0


def _ws_bytes(a):
    return ssm.lib().ssm_gla_workspace_bytes(ctypes.byref(a))


def test_workspace_query():
    """phi(k) and phi(q), each (B, L, G, N) bf16 rounded up to 256 bytes; none
    without the feature map or with nothing to do."""
    assert _ws_bytes(_args()) == 0
    n = 2 * 64 * 2 * 128 * 2
    assert _ws_bytes(_args(feature_map=1)) == 2 * ((n + 255) // 256 * 256)
    assert _ws_bytes(_args(feature_map=1, shape=(2, 0, 8, 64, 2, 128))) == 0
    assert _ws_bytes(_args(feature_map=2)) == -9


def test_workspace_checked_on_host():
    far = FAKE + (40 << 32)
    big = 1 << 20
    # misaligned workspace
    assert _gla(_args(feature_map=1, workspace=far + 8, workspace_bytes=big)) == -5
    # a workspace overlapping an input or an output
    assert _gla(_args(feature_map=1, workspace=FAKE + (2 << 32), workspace_bytes=big)) == -6   # v
    assert _gla(_args(feature_map=1, workspace=FAKE + (7 << 32), workspace_bytes=big)) == -6   # y
    assert _gla(_args(feature_map=1, workspace=FAKE - 256, workspace_bytes=big)) == -6         # q


def test_workspace_with_time_segments():
    """The segment summaries follow phi(k) and phi(q) in the workspace; a
    workspace too small for both drops an automatic split first."""
    up = lambda n: (n + 255) // 256 * 256
    shape = (1, 4096, 16, 64, 1, 64)  # 64 chunks, B*H = 16 -> 16 segments of 4 chunks
    phi = 2 * up(4096 * 64 * 2)
    summ = up(15 * 16 * 64 * 64 * 4) + up(15 * 16 * 4)
    assert _ws_bytes(_args(shape=shape)) == summ
    assert _ws_bytes(_args(shape=shape, feature_map=1)) == phi + summ
    assert _ws_bytes(_args(shape=shape, feature_map=1, time_splits=1)) == phi
    far = FAKE + (40 << 32)
    plan = lambda a: ssm.lib().ssm_gla_plan(ctypes.byref(a))
    assert plan(_args(shape=shape, feature_map=1, workspace=far, workspace_bytes=phi + summ)) == 16
    assert plan(_args(shape=shape, feature_map=1, workspace=far, workspace_bytes=phi + summ - 1)) == 1
    assert plan(_args(shape=shape, workspace=far, workspace_bytes=summ)) == 16
    assert plan(_args(shape=shape, feature_map=1, time_splits=4, workspace=far, workspace_bytes=phi)) == -7
    assert plan(_args(shape=shape, time_splits=4)) == -7
