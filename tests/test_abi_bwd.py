"""The backward entry points of the C ABI on the CPU: argument checks that
fail on the host before any HIP call, and the host-only plan and workspace
queries.  Pointers are fake, 16-byte aligned addresses that are never
dereferenced (every call here fails validation or is a query)."""
import ctypes

import pytest

import mamba_selective_scan_06_amd as ssm

FAKE = 0x7F0000000000
INPUTS = ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0", "dy", "dhT")
OUTPUTS = ("dx", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0")


def _args(**kw):
    a = ssm.ScanBwdArgs()
    a.batch, a.seqlen, a.dim, a.dstate = kw.pop("shape", (2, 64, 128, 16))
    a.dtype = kw.pop("dtype", 1)
    base = FAKE
    for name in INPUTS + OUTPUTS:
        setattr(a, name, kw.pop(name, base))
        base += 1 << 32  # disjoint 4 GiB windows
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _bwd(a):
    return ssm.lib().ssm_scan_bwd(ctypes.byref(a), None)


@pytest.mark.parametrize("mut,code", [
    (dict(shape=(-1, 8, 8, 16)), -2),
    (dict(shape=(1, 8, 8, 0)), -3),
    (dict(shape=(1, 8, 8, 65)), -3),
    (dict(dtype=5), -4),
    (dict(shape=(70000, 8, 8, 16)), -2),
    (dict(shape=(2**40, 2**20, 2**20, 16)), -2),
    (dict(x=0), -1), (dict(delta=0), -1), (dict(A=0), -1), (dict(B=0), -1), (dict(C=0), -1), (dict(dy=0), -1),
    (dict(z=0), -1),  # dz is given, so z is needed
    (dict(dx=FAKE + 4), -5), (dict(dhT=FAKE + 8), -5), (dict(workspace=FAKE + 2), -5),
    (dict(flags=4), -9), (dict(flags=8), -9),  # the carry scan is forward only; 8 is no flag (dict(time_splits=-1), -9), (dict(reserved=1), -9),
    (dict(workspace=0), -7),
    (dict(workspace_bytes=16), -7),
])
def test_invalid_arguments_rejected_on_host(mut, code):
    assert _bwd(_args(**mut)) == code


def test_null_args_struct():
    assert ssm.lib().ssm_scan_bwd(None, None) == -1
    assert ssm.lib().ssm_scan_bwd_workspace_bytes(None) == -1
    assert ssm.lib().ssm_scan_bwd_plan(None) == -1


@pytest.mark.parametrize("out", OUTPUTS)
def test_gradient_over_an_input_rejected(out):
    a = _args()
    setattr(a, out, a.x)
    assert _bwd(a) == -6
    a = _args()
    setattr(a, out, a.dy)
    assert _bwd(a) == -6


def test_gradients_overlapping_each_other_rejected():
    a = _args()
    a.ddelta = a.dx + 2 * 16  # starts inside dx
    assert _bwd(a) == -6
    a = _args()
    a.dD = a.dA  # fp32 (D,) inside (D, N)
    assert _bwd(a) == -6


def test_plan_and_workspace_queries():
    L = ssm.lib()
    q = lambda a: (L.ssm_scan_bwd_plan(ctypes.byref(a)), L.ssm_scan_bwd_workspace_bytes(ctypes.byref(a)))
    # 4 batch rows x 2048 channels: 64 (N = 16: 32 channels per wave) x 4 = 256 waves,
    # split 16 ways to reach 4096 waves; segments stay >= 64 tokens.
    S, ws = q(_args(shape=(4, 8192, 2048, 16)))
    assert S == 16 and ws > 0
    S, _ = q(_args(shape=(1, 256, 64, 16)))
    assert S == 4  # 64-token segments
    S, _ = q(_args(shape=(1, 100, 64, 16), time_splits=1))
    assert S == 1
    # requested splits round to whole 8-token chunks: ceil(100 / 3) = 34 -> 40 tokens, 3 segments
    S, _ = q(_args(shape=(1, 100, 64, 16), time_splits=3))
    assert S == 3
    S, _ = q(_args(shape=(1, 100, 64, 16), time_splits=1000))
    assert S == 13  # one 8-token chunk each
    # nothing to compute: no workspace, one segment
    for shape in [(0, 8, 8, 16), (2, 0, 8, 16), (2, 8, 0, 16)]:
        assert q(_args(shape=shape)) == (1, 0)
    # the workspace grows with the checkpoints: B * ceil(L / T) * D * N fp32 at least
    _, ws = q(_args(shape=(2, 640, 128, 16), time_splits=1))
    assert ws >= 2 * 80 * 128 * 16 * 4
    # the per-block partial dB / dC rows: B * L * ceil(D / 32) * N fp32 each (N = 16: 32 channels per wave)
    assert ws >= 2 * 80 * 128 * 16 * 4 + 2 * (2 * 640 * 4 * 16 * 4)


def test_dstate_limit_and_lane_layout():
    L = ssm.lib()
    for n in (1, 3, 4, 5, 8, 12, 16, 17, 32, 33, 64):
        assert L.ssm_scan_bwd_plan(ctypes.byref(_args(shape=(1, 64, 64, n)))) >= 1


def test_zero_order_hold_passes_host_checks():
    """SSM_FLAG_ZOH (and with GENERIC_A) is a valid backward flag: the host
    checks get as far as the workspace, and the plan and size queries accept it."""
    for flags in (2, 3):
        assert _bwd(_args(flags=flags, workspace=0)) == -7
        assert ssm.lib().ssm_scan_bwd_plan(ctypes.byref(_args(flags=flags))) >= 1
        assert ssm.lib().ssm_scan_bwd_workspace_bytes(ctypes.byref(_args(flags=flags))) > 0


def test_checkpoints_shrink_the_workspace_and_are_checked():
    """With the forward's checkpoints the backward keeps none of its own
    (nor the segment states), so it asks for less workspace; the checkpoints
    are an input for the alias checks."""
    far = FAKE + (40 << 32)
    ws = ssm.lib().ssm_scan_bwd_workspace_bytes
    plain = ws(ctypes.byref(_args()))
    with_ck = ws(ctypes.byref(_args(checkpoints=far)))
    B, L, D, N = 2, 64, 128, 16
    S = ssm.lib().ssm_scan_bwd_plan(ctypes.byref(_args()))
    up = lambda n: (n + 255) // 256 * 256
    assert plain - with_ck == up(B * (L // 8) * D * N * 4) + up(B * (L // 8) * D * 4) + up(B * S * D * N * 4)
    assert _bwd(_args(checkpoints=far + 4)) == -5
    assert _bwd(_args(checkpoints=FAKE + (11 << 32))) == -6   # under dx
