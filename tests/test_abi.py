"""The C ABI on the CPU: the library loads, exports what the header declares,
and rejects bad arguments on the host before any HIP call (no GPU needed).

Pointers below are fake, 16-byte aligned addresses: every call here either
fails validation or is a host-only query, so nothing is ever dereferenced.
"""
import ctypes
import re

import pytest

import mamba_selective_scan_06_amd as ssm

FAKE = 0x7F0000000000  # aligned, never dereferenced


def _header_functions():
    text = open(ssm.HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char \*)\s*(ssm_\w+)\s*\(", text, re.M)))


def _args(**kw):
    a = ssm.ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate = kw.pop("shape", (2, 64, 128, 16))
    a.dtype = kw.pop("dtype", 1)
    base = FAKE
    for name in ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0", "hT", "y"):
        setattr(a, name, kw.pop(name, base))
        base += 1 << 32  # disjoint 4 GiB windows
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_library_loads_and_exports_header_symbols():
    L = ssm.lib()
    declared = _header_functions()
    assert set(declared) == set(ssm.EXPORTS), declared
    for name in declared:
        assert hasattr(L, name), f"{name} not exported"
    assert L.ssm_scan_abi_version() == ssm.ABI_VERSION == 4


def test_strerror_covers_codes():
    for code in range(0, -10, -1):
        assert ssm.strerror(code) and ssm.strerror(code) != "unknown status code"
    assert ssm.strerror(-99) == "unknown status code"


def _fwd(a):
    return ssm.lib().ssm_scan_fwd(ctypes.byref(a), None)


@pytest.mark.parametrize("mut,code", [
    (dict(shape=(-1, 8, 8, 16)), -2),
    (dict(shape=(1, 8, 8, 0)), -3),
    (dict(shape=(1, 8, 8, 65)), -3),
    (dict(dtype=7), -4),
    (dict(shape=(70000, 8, 8, 16)), -2),
    (dict(shape=(2**40, 2**20, 2**20, 16)), -2),
    (dict(x=0), -1), (dict(delta=0), -1), (dict(A=0), -1), (dict(B=0), -1), (dict(C=0), -1), (dict(y=0), -1),
    (dict(x=FAKE + 2), -5), (dict(z=FAKE + 8), -5), (dict(hT=FAKE + 4), -5),
    (dict(flags=8), -9), (dict(flags=-1), -9), (dict(variant=9), -9), (dict(time_splits=-1), -9),
    (dict(variant=3), -9),  # decode needs seqlen == 1
    (dict(variant=2, time_splits=4), -9),  # splitting is NSPLIT only
    (dict(shape=(2, 64, 128, 12), variant=1), -9),  # NSPLIT needs N in {4,8,16,32,64}
])
def test_invalid_arguments_rejected_on_host(mut, code):
    assert _fwd(_args(**mut)) == code


def test_null_args_struct():
    assert ssm.lib().ssm_scan_fwd(None, None) == -1


def test_aliasing_rejected():
    a = _args()
    a.y = a.x  # y over an input
    assert _fwd(a) == -6
    a = _args()
    a.hT = a.A  # hT over A
    assert _fwd(a) == -6
    a = _args()
    a.hT = a.h0 + 16  # partial overlap with h0
    assert _fwd(a) == -6
    a = _args()
    a.y = a.hT
    assert _fwd(a) == -6


def test_time_splits_without_workspace_rejected():
    a = _args(time_splits=4)
    assert _fwd(a) == -7


def test_empty_problems_are_noops():
    # batch or dim zero: nothing is read or written, even with NULL pointers
    a = _args(shape=(0, 64, 128, 16), x=0, y=0)
    assert _fwd(a) == 0
    a = _args(shape=(2, 64, 0, 16), x=0, y=0)
    assert _fwd(a) == 0


def test_empty_problems_plan_and_workspace_queries():
    # batch or dim zero through the host-only queries: no workspace, one
    # segment, no crash (the planner's blocks-per-compute-unit division)
    lib = ssm.lib()
    for shape in ((0, 64, 128, 16), (2, 64, 0, 16), (0, 8192, 1536, 16), (1, 8192, 0, 16)):
        a = _args(shape=shape, x=0, y=0)
        assert lib.ssm_scan_workspace_bytes(ctypes.byref(a)) == 0
        assert lib.ssm_scan_plan(ctypes.byref(a)) >= 0
        assert ssm.plan(a)[1] == 1
        a.workspace, a.workspace_bytes = FAKE + (64 << 32), 1 << 30
        assert lib.ssm_scan_plan(ctypes.byref(a)) >= 0
        assert _fwd(a) == 0


def test_noalloc_rejects_oversized_explicit_split_on_host():
    # 64 x 16384 x 17 x 4 bytes of segment summaries > the 8 MiB device array:
    # rejected before any HIP call; an automatic plan of the same shape stays
    # within it (and needs no GPU to be planned)
    lib = ssm.lib()
    a = _args(shape=(1, 1 << 20, 16384, 16), time_splits=64)
    base = FAKE
    for name in ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0", "hT", "y"):
        setattr(a, name, base)
        base += 1 << 40  # disjoint 1 TiB windows
    assert lib.ssm_scan_fwd_noalloc(ctypes.byref(a), None) == -7
    assert lib.ssm_scan_fwd_noalloc(None, None) == -1
    assert lib.ssm_scan_fwd_noalloc(ctypes.byref(_args(shape=(0, 64, 128, 16), x=0, y=0)), None) == 0
    assert lib.ssm_scan_fwd_noalloc(ctypes.byref(_args(x=FAKE + 2)), None) == -5


def test_plan_and_workspace_queries():
    lib = ssm.lib()
    # the benchmark layer: 64 channel blocks x 4 batch rows = 256 blocks, one per compute unit, unsplit
    a = _args(shape=(4, 8192, 4096, 16))
    assert ssm.plan(a) == ("nsplit", 1)
    assert lib.ssm_scan_workspace_bytes(ctypes.byref(a)) == 0
    # long context with few channels splits time when a workspace is given
    a = _args(shape=(1, 8192, 1536, 16))
    nbytes = lib.ssm_scan_workspace_bytes(ctypes.byref(a))
    assert nbytes > 0
    assert ssm.plan(a) == ("nsplit", 1)  # no workspace: runs unsplit
    a.workspace, a.workspace_bytes = FAKE + (64 << 32), nbytes
    v, s = ssm.plan(a)
    assert v == "nsplit" and s == 10  # 24 blocks x 10 segments: the most that fit the 256 compute units
    # 192 blocks: a second segment would need a second round of blocks, so none
    b = _args(shape=(8, 2048, 1536, 16))
    b.workspace, b.workspace_bytes = FAKE + (64 << 32), 1 << 30
    assert ssm.plan(b) == ("nsplit", 1)
    # in-place state update never splits
    a.hT = a.h0
    assert ssm.plan(a) == ("nsplit", 1)
    # decode and the lane fallback
    assert ssm.plan(_args(shape=(256, 1, 5120, 16))) == ("decode", 1)
    assert ssm.plan(_args(shape=(2, 64, 128, 12))) == ("lane", 1)
    assert ssm.plan(_args(shape=(2, 64, 128, 16), variant=2)) == ("lane", 1)


def test_plan_long_rows_stay_on_the_main_kernel():
    """Rows past 2^31 and 2^32 bytes plan the main kernel (its descriptor
    windows move along the row); only a token wider than a window allows, or a
    row longer than 32-bit token counts allow, falls back to LANE."""
    def big(shape, dtype):
        a = _args(shape=shape, dtype=dtype)
        base = FAKE
        for name in ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0", "hT", "y"):
            setattr(a, name, base)
            base += 1 << 40  # disjoint 1 TiB windows
        return a
    assert ssm.plan(big((1, 262_152, 4104, 16), 1)) == ("nsplit", 1)   # 2.15 GB bf16 row
    assert ssm.plan(big((1, 270_008, 4104, 16), 0)) == ("nsplit", 1)   # 4.43 GB fp32 row
    assert ssm.plan(big((1, 2**31 - 1025, 64, 16), 1)) == ("nsplit", 1)
    assert ssm.plan(big((1, 2**31 - 1024, 64, 16), 1)) == ("lane", 1)
    lim = (2**31 - 1) // 320
    assert ssm.plan(big((1, 64, lim // 2, 16), 1)) == ("nsplit", 1)
    assert ssm.plan(big((1, 64, lim // 2 + 1, 16), 1)) == ("lane", 1)
    assert ssm.plan(big((1, 64, lim // 4, 16), 0)) == ("nsplit", 1)
    assert ssm.plan(big((1, 64, lim // 4 + 1, 16), 0)) == ("lane", 1)


def test_zoh_flag_accepted():
    """SSM_FLAG_ZOH (alone or with SSM_FLAG_GENERIC_A) passes the host checks;
    with batch 0 nothing is launched."""
    for f in (2, 3, 4, 7):  # SSM_FLAG_CARRY_SCAN (4) as well
        assert _fwd(_args(shape=(0, 8, 8, 16), flags=f)) == 0
        assert ssm.lib().ssm_scan_plan(ctypes.byref(_args(flags=f))) >= 0


def _ck_bytes(a):
    return ssm.lib().ssm_scan_checkpoint_bytes(ctypes.byref(a))


def test_checkpoint_bytes_query():
    """(B, ceil(L / T) - 1, 4, D, ceil(N / 4)) fp32, T = 8 tokens (16 when N <= 4)."""
    assert _ck_bytes(_args(shape=(2, 64, 128, 16))) == 2 * 7 * 128 * 16 * 4
    assert _ck_bytes(_args(shape=(2, 65, 128, 16))) == 2 * 8 * 128 * 16 * 4
    assert _ck_bytes(_args(shape=(1, 64, 8, 4))) == 1 * 3 * 8 * 4 * 4     # T = 16
    assert _ck_bytes(_args(shape=(1, 8, 8, 16))) == 0                     # one chunk: nothing to keep
    assert _ck_bytes(_args(shape=(1, 0, 8, 16))) == 0
    assert _ck_bytes(_args(shape=(1, 1, 8, 16))) == 0
    assert ssm.checkpoint_shape(2, 65, 128, 16) == (2, 8, 4, 128, 4)
    assert ssm.checkpoint_shape(1, 64, 8, 4) == (1, 3, 4, 8, 1)
    assert ssm.checkpoint_shape(1, 64, 8, 5) == (1, 7, 4, 8, 2)           # quarters of 2, three slots unused
    assert _ck_bytes(_args(shape=(1, 64, 8, 5))) == 7 * 4 * 8 * 2 * 4
    assert _ck_bytes(_args(shape=(1, 64, 8, 65))) == -3


def test_checkpoints_checked_on_host():
    far = FAKE + (40 << 32)
    assert _fwd(_args(checkpoints=far + 4)) == -5                      # misaligned
    assert _fwd(_args(checkpoints=FAKE)) == -6                         # over x
    assert _fwd(_args(checkpoints=FAKE + (10 << 32) - 64)) == -6       # runs into y
    assert _fwd(_args(checkpoints=FAKE + (9 << 32))) == -6             # over hT
