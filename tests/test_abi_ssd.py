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
    a.time_splits = kw.pop("time_splits", 0)
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
    (dict(time_splits=-1), -9), (dict(time_splits=65536), -9),
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


def _ws(a):
    return ssm.lib().ssm_ssd_workspace_bytes(ctypes.byref(a))


def _plan(a):
    return ssm.lib().ssm_ssd_plan(ctypes.byref(a))


FAR = FAKE + (40 << 32)  # a workspace address clear of every fake tensor


def _summary_bytes(B, S, H, N, m=1):
    """Summaries of the (S - 1) m state-only sub-segments."""
    up = lambda n: (n + 255) // 256 * 256
    return up(B * (S - 1) * m * H * 64 * N * 4) + up(B * (S - 1) * m * H * 4)


def test_time_split_plan_small_batch():
    """B*H = 64 heads leave 3/4 of 256 compute units idle: 4 segments of 128
    chunks, when the workspace holds their summaries.  The state-only pass
    fits three workgroups per compute unit, so the 3 segments before the last
    are cut in 4 sub-segments each (3 * 4 * 64 = 768 <= 768 workgroups)."""
    shape = (1, 32768, 64, 64, 1, 128)
    need = _summary_bytes(1, 4, 64, 128, m=4)
    assert _ws(_args(shape=shape)) == need
    assert _plan(_args(shape=shape)) == 1                                      # no workspace: one segment
    assert _plan(_args(shape=shape, workspace=FAR, workspace_bytes=need - 1)) == 1
    assert _plan(_args(shape=shape, workspace=FAR, workspace_bytes=need)) == 4
    assert _plan(_args(shape=shape, time_splits=1, workspace=FAR, workspace_bytes=need)) == 1
    assert _ws(_args(shape=shape, time_splits=1)) == 0


def test_time_split_plan_explicit():
    shape = (2, 640, 8, 64, 2, 64)  # 10 chunks
    # 3 segments of 4, 4, 2 chunks; 7 asked -> segments of 2 chunks -> 5; more than 10 -> 10
    for asked, got in ((3, 3), (7, 5), (10, 10), (50, 10)):
        need = _summary_bytes(2, got, 8, 64)
        assert _ws(_args(shape=shape, time_splits=asked)) == need, asked
        assert _plan(_args(shape=shape, time_splits=asked)) == -7, asked        # explicit needs the workspace
        assert _ssd(_args(shape=shape, time_splits=asked)) == -7, asked
        assert _plan(_args(shape=shape, time_splits=asked, workspace=FAR, workspace_bytes=need)) == got, asked
    # automatic: 256 // 16 = 16 segments, at least 4 chunks each -> 2
    assert _plan(_args(shape=shape, workspace=FAR, workspace_bytes=1 << 30)) == 2


def test_time_split_plan_full_device_and_empty():
    assert _ws(_args(shape=(4, 8192, 64, 64, 1, 128))) == 0        # B*H = 256: no split
    assert _plan(_args(shape=(4, 8192, 64, 64, 1, 128), workspace=FAR, workspace_bytes=1 << 30)) == 1
    assert _ws(_args(shape=(1, 0, 8, 64, 1, 128))) == 0             # no tokens
    assert _ws(_args(shape=(1, 0, 8, 64, 1, 128), time_splits=4)) == 0
    assert _ws(_args(shape=(1, 64, 8, 64, 1, 128), time_splits=4)) == 0   # one chunk


def test_workspace_checked_on_host():
    big = 1 << 30
    assert _ssd(_args(workspace=FAR + 8, workspace_bytes=big)) == -5
    assert _ssd(_args(workspace=FAR, workspace_bytes=-1)) == -5
    assert _ssd(_args(workspace=FAKE + (1 << 32), workspace_bytes=big)) == -6   # dt
    assert _ssd(_args(workspace=FAKE + (9 << 32), workspace_bytes=big)) == -6   # y


def test_state_only_sub_segments():
    """m: the largest divisor of the segment's chunks with (S - 1) m B H <= 768
    and at least 4 chunks per sub-segment."""
    # 48 chunks, 3 segments of 16: (3 - 1) m 2 <= 512 and m <= 4 -> m = 4
    assert _ws(_args(shape=(1, 64 * 48, 2, 64, 1, 64), time_splits=3)) == _summary_bytes(1, 3, 2, 64, m=4)
    # 60 chunks, 6 segments of 10: m <= 2 -> 2
    assert _ws(_args(shape=(1, 64 * 60, 2, 64, 1, 64), time_splits=6)) == _summary_bytes(1, 6, 2, 64, m=2)
    # B H = 128: 2 automatic segments of 64 chunks, 1 * m * 128 <= 768 and m | 64 -> m = 4
    assert _ws(_args(shape=(2, 8192, 64, 64, 1, 128))) == _summary_bytes(2, 2, 64, 128, m=4)
