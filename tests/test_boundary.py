"""The C boundary on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments before touching a device.  No kernel is launched here."""
import math
import os
import re

import pytest

from exact_attention_90_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "page_tensor_sizes.txt")
CODES = {"f32": 0, "f16": 1, "bf16": 2}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from exact_attention_90_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_python_export_list():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libfa.so does not export {name}"


def test_status_strings_and_version(lib):
    for code in range(0, 10):
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_string(99).decode() == "unknown status"
    assert "gfx950" in lib.fa_version().decode()
    assert lib.fa_last_hip_error() == 0


def test_workspace_bytes_pinned_to_page_sizes(lib):
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        fields, cite = line.split("|")
        B, H, N, dt, printed, tol = fields.split()
        got = lib.fa_naive_workspace_bytes(int(B), int(H), int(N), CODES[dt])
        printed = float(printed)
        assert abs(got - printed) <= float(tol) * printed, (cite, got, printed)


def test_workspace_bytes_edges(lib):
    assert lib.fa_naive_workspace_bytes(1, 1, 3, 1) == 256      # 18 bytes rounded up
    assert lib.fa_naive_workspace_bytes(0, 5, 7, 0) == 0
    assert lib.fa_naive_workspace_bytes(1, 1, 1, 7) == 0        # bad dtype
    assert lib.fa_naive_workspace_bytes(-1, 1, 1, 0) == 0
    big = lib.fa_naive_workspace_bytes(2**31 - 1, 2**31 - 1, 2**31 - 1, 0)
    assert big == 2**64 - 1                                     # does not fit size_t


# fake, never-dereferenced device addresses (16-byte aligned, non-null)
A, B_, C_, O_, L_ = 0x1000, 0x2000, 0x3000, 0x4000, 0x5000


def call(lib, q=A, k=B_, v=C_, o=O_, lse=L_, B=1, H=1, N=128, d=64, scale=0.125, dtype=1):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, dtype, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dtype=3), 4), (dict(dtype=-1), 4),
    (dict(d=96), 3), (dict(d=0), 3), (dict(d=192), 3), (dict(d=512), 3),
    (dict(scale=0.0), 5), (dict(scale=-0.1), 5), (dict(scale=math.inf), 5), (dict(scale=math.nan), 5),
    (dict(B=-1), 2), (dict(H=-2), 2), (dict(N=-5), 2),
    (dict(q=None), 1), (dict(v=None), 1), (dict(lse=None), 1),
    (dict(q=A + 8), 6), (dict(o=O_ + 4), 6), (dict(lse=L_ + 2), 6),
    (dict(B=2**20, H=2**10, N=2**12), 2),                    # grid beyond 2^24 workgroups
    (dict(B=2**16, H=2**16, N=1), 2),                        # B*H beyond int
    (dict(N=2**23, d=128, dtype=1), 2),                      # one head beyond 2^31 bytes
    (dict(N=2**23 - 511, d=128, dtype=2), 2),                # one tile short of it: refused
    (dict(N=2**22, d=256, dtype=2), 2),
    (dict(N=2**21, d=256, dtype=0), 2),
])
def test_fwd_rejects_bad_arguments_before_any_device_call(lib, kwargs, code):
    assert call(lib, **kwargs) == code


@pytest.mark.parametrize("kwargs", [dict(N=0), dict(B=0), dict(H=0),
                                    dict(N=0, q=None, k=None, v=None, o=None, lse=None)])
def test_empty_problem_is_a_no_op(lib, kwargs):
    assert call(lib, **kwargs) == 0


def bwd_call(lib, dtype=1, d=64, ws=0x8000, dout=0x9000, dq=0xa000, N=128):
    return lib.fa_bwd(A, B_, C_, O_, L_, dout, dq, 0xb000, 0xc000, ws, 1, 1, N, d, 0.125, dtype,
                      None)


def test_bwd_rejects_unsupported_and_bad_arguments(lib):
    assert bwd_call(lib, dtype=0, d=256) == 3   # fp32 inputs at d = 256: no backward kernel
    assert bwd_call(lib, dtype=3) == 4
    assert bwd_call(lib, d=96) == 3
    assert bwd_call(lib, d=512) == 3
    assert bwd_call(lib, ws=0) == 7             # NULL workspace
    assert bwd_call(lib, ws=0x8010) == 7        # workspace not 256-byte aligned
    assert bwd_call(lib, dout=0) == 1
    assert bwd_call(lib, dq=0xa004) == 6
    assert bwd_call(lib, N=0, ws=0, dout=0, dq=0) == 0  # empty problem


def test_bwd_workspace_bytes(lib):
    # dO in the input type plus two floats per row, each part rounded up to 256 bytes
    assert lib.fa_bwd_workspace_bytes(8, 32, 4096, 128, 2) == 8 * 32 * 4096 * (128 * 2 + 8)
    assert lib.fa_bwd_workspace_bytes(1, 1, 3, 64, 1) == 512 + 256 + 256  # 384 B of dO -> 512
    assert lib.fa_bwd_workspace_bytes(1, 1, 3, 64, 0) == 256 + 256  # fp32: no dO copy
    assert lib.fa_bwd_workspace_bytes(1, 1, 3, 256, 0) == 0     # unsupported
    assert lib.fa_bwd_workspace_bytes(1, 1, 3, 256, 1) == 1536 + 256 + 256
    assert lib.fa_bwd_workspace_bytes(1, 1, 3, 96, 1) == 0
    assert lib.fa_bwd_workspace_bytes(-1, 1, 3, 64, 1) == 0


def test_naive_rejects_bad_workspace(lib):
    args = (A, B_, C_, O_, L_)
    assert lib.fa_naive_fwd(*args, None, 0x6000, 1, 1, 64, 64, 0.125, 1, None) == 7
    assert lib.fa_naive_fwd(*args, 0x6004, 0x7000, 1, 1, 64, 64, 0.125, 1, None) == 7
    assert lib.fa_naive_fwd(*args, 0x6000, 0x7000, 1, 1, 64, 100, 0.125, 1, None) == 3
    assert lib.fa_naive_fwd(*args, None, None, 1, 1, 0, 64, 0.125, 1, None) == 0


def split_call(lib, ws=0x8000, nsplit=4, dtype=1, d=64, N=128, B=1, H=1, q=A):
    return lib.fa_fwd_split(q, B_, C_, O_, L_, ws, nsplit, B, H, N, d, 0.125, dtype, None)


def test_split_rejects_bad_arguments(lib):
    assert split_call(lib, dtype=5) == 4
    assert split_call(lib, d=96) == 3
    assert split_call(lib, nsplit=0) == 2
    assert split_call(lib, nsplit=65) == 2      # beyond FA_MAX_SPLIT
    assert split_call(lib, ws=0) == 7           # NULL workspace
    assert split_call(lib, ws=0x8010) == 7      # workspace not 256-byte aligned
    assert split_call(lib, q=A + 8) == 6
    assert split_call(lib, B=2**20, H=2**10, N=2**12, nsplit=1) == 2   # grid limit
    assert split_call(lib, N=0, ws=0) == 0      # empty problem: nothing to launch


def test_split_noalloc_rejects_before_any_launch(lib):
    # the allocation-free key split checks like fa_fwd_split (minus the workspace) and
    # refuses problems whose partials exceed the static scratch, all before touching a
    # device (these pointers are never dereferenced)
    def call(dtype=1, d=64, nsplit=2, B=1, H=1, N=128, q=A):
        return lib.fa_fwd_split_noalloc(q, B_, C_, O_, L_, nsplit, B, H, N, d, 0.125, dtype, None)
    assert call(dtype=5) == 4
    assert call(d=96) == 3
    assert call(nsplit=0) == 2 and call(nsplit=65) == 2
    assert call(q=A + 8) == 6
    assert call(N=0) == 0
    assert _lib.FA_SCRATCH_BYTES == 64 << 20
    # 4 ranges of 8 heads x 8192 rows at d = 128 need 4 x 65536 x 129 x 4 bytes > 64 MiB
    assert lib.fa_fwd_split_workspace_bytes(1, 8, 8192, 128, 4) > _lib.FA_SCRATCH_BYTES
    assert call(H=8, N=8192, d=128, nsplit=4) == 9
    assert lib.fa_status_string(9).decode() == "problem needs more than the library's static scratch"


def test_stats_arguments_and_sizes(lib):
    # the statistics-recording forward checks like fa_fwd, plus its stats buffer
    def call(st=0x8000, dtype=1, d=64, N=128, q=A):
        return lib.fa_fwd_stats(q, B_, C_, O_, L_, st, 1, 1, N, d, 0.125, dtype, None)
    assert call(dtype=5) == 4 and call(d=96) == 3 and call(q=A + 8) == 6
    assert call(st=0) == 7 and call(st=0x8004) == 7  # NULL or misaligned stats
    assert call(N=0, st=0) == 0
    # two floats per row and 64-key block
    assert lib.fa_fwd_stats_bytes(1, 2, 333) == 2 * 333 * 6 * 2 * 4
    assert lib.fa_fwd_stats_bytes(2, 3, 64) == 6 * 64 * 1 * 8
    assert lib.fa_fwd_stats_bytes(-1, 1, 1) == 0


def test_split_workspace_bytes(lib):
    # nsplit slots of partial O (d floats per row) and of partial LSE (one float per row),
    # each part rounded up to 256 bytes
    assert lib.fa_fwd_split_workspace_bytes(1, 16, 16384, 128, 4) == 4 * 16 * 16384 * 129 * 4
    assert lib.fa_fwd_split_workspace_bytes(1, 1, 3, 64, 2) == 1536 + 256
    assert lib.fa_fwd_split_workspace_bytes(1, 1, 3, 64, 0) == 0
    assert lib.fa_fwd_split_workspace_bytes(1, 1, 3, 64, 65) == 0
    assert lib.fa_fwd_split_workspace_bytes(1, 1, 3, 96, 2) == 0
    assert lib.fa_fwd_split_workspace_bytes(-1, 1, 3, 64, 2) == 0
    assert lib.fa_fwd_split_workspace_bytes(0, 1, 3, 64, 2) == 0


def test_split_suggest(lib):
    s = lib.fa_fwd_split_suggest
    # the measured cases on 256 compute units: one head of 16384 rows has 64 Q tiles,
    # four ranges fill the device; four heads already have 256 Q tiles
    assert s(1, 1, 16384, 128, 256) == 4
    assert s(1, 4, 16384, 128, 256) == 1
    assert s(1, 16, 16384, 128, 256) == 1
    assert s(1, 8, 8192, 128, 256) == 1
    assert s(1, 1, 16384, 64, 256) == 2          # 128-row tiles at d = 64
    assert s(1, 1, 2048, 128, 256) == 4          # capped: 32 key tiles, 8 per range
    assert s(1, 1, 100, 128, 256) == 1           # two key tiles: no split
    assert s(1, 1, 2**20, 128, 100000) == 25     # ceil(100000 / 4096 Q tiles)
    assert s(1, 1, 2**20, 128, 2**30) == 64      # FA_MAX_SPLIT
    assert s(0, 1, 100, 128, 256) == 1 and s(1, 1, 100, 96, 256) == 1
    assert s(1, 1, 100, 128, 0) == 1


def test_bwd_split_arguments_and_sizes(lib):
    def call(dtype=1, d=64, ws=0x8000, nsplit=2, N=128, dout=0x9000):
        return lib.fa_bwd_split(A, B_, C_, O_, L_, dout, 0xa000, 0xb000, 0xc000, ws, nsplit,
                                1, 1, N, d, 0.125, dtype, None)
    assert call(dtype=0, d=256) == 3   # fp32 inputs at d = 256: no backward kernel
    assert call(d=96) == 3
    assert call(nsplit=0) == 2 and call(nsplit=65) == 2
    assert call(ws=0) == 7 and call(ws=0x8010) == 7
    assert call(dout=0) == 1
    assert call(N=0, ws=0, dout=0) == 0
    # fa_bwd's workspace, then 3 nsplit slots of B H N d floats rounded up to 256 bytes
    base = lib.fa_bwd_workspace_bytes(1, 2, 100, 64, 2)
    assert lib.fa_bwd_split_workspace_bytes(1, 2, 100, 64, 2, 4) == base + 3 * 4 * 2 * 100 * 64 * 4
    assert lib.fa_bwd_split_workspace_bytes(1, 1, 3, 64, 1, 1) == (
        lib.fa_bwd_workspace_bytes(1, 1, 3, 64, 1) + 2304)
    assert lib.fa_bwd_split_workspace_bytes(1, 1, 3, 64, 0, 2) == (
        lib.fa_bwd_workspace_bytes(1, 1, 3, 64, 0) + 4608)             # fp32: no dO copy
    assert lib.fa_bwd_split_workspace_bytes(1, 1, 3, 256, 0, 2) == 0
    assert lib.fa_bwd_split_workspace_bytes(1, 1, 3, 64, 1, 0) == 0
    s = lib.fa_bwd_split_suggest
    assert s(1, 1, 16384, 128, 256) == 4     # 128 workgroups of 128 rows (4: measured best)
    assert s(1, 4, 16384, 128, 256) == 1     # 512 workgroups: two per compute unit
    assert s(1, 2, 8192, 64, 256) == 4       # measured best at d = 64
    assert s(1, 1, 4096, 64, 256) == 8       # 32 workgroups; capped at 64 tiles / 8
    assert s(1, 1, 100, 64, 256) == 1


def _gpu_present():
    return os.path.exists("/dev/kfd")


@pytest.mark.skipif(_gpu_present(), reason="only meaningful on a host without a GPU")
def test_valid_call_without_a_device_reports_hip_error(lib):
    # every check passes, so the library asks HIP for a device, finds none and
    # returns FA_ERR_HIP without launching anything
    assert call(lib) == 8
    assert lib.fa_last_hip_error() != 0
    # the longest head the checks accept at d = 128 (one tile short of 2^31 bytes)
    assert call(lib, N=2**23 - 512, d=128, dtype=2) == 8
