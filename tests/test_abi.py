"""The C ABI library loads, exports every declared symbol, answers size
queries like the oracle's layout geometry, and rejects bad arguments on the
host before any HIP call (no compute calls here)."""

import ctypes
import os
import re

import pytest
import torch

from oracle import layout as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("mxfp4.h", "mxfp4_testing.h")]

import mxfp4_block_scaled_quant_amd as mx  # noqa: E402


def _declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.LIB_PATH):
        pytest.fail("libmxfp4.so is not built (python -m mxfp4_block_scaled_quant_amd.build)")
    return mx.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"mxfp4_quant_1x32", "mxfp4_preshuffle_weight", "mxfp4_gemm_a4w4",
            "a16wfp4_bmm"} <= set(names)
    raw = ctypes.CDLL(mx.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"{n} declared but not exported"
    assert set(names) <= set(mx._SIGNATURES), "binding lacks a declared function"


def _exported_functions(path):
    """Names of the defined global/weak FUNC symbols of an ELF64 shared
    library's dynamic symbol table (read directly, no external tool)."""
    import struct
    data = open(path, "rb").read()
    assert data[:4] == b"\x7fELF" and data[4] == 2, "not an ELF64 file"
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum = struct.unpack_from("<HH", data, 0x3A)
    secs = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize) for i in range(shnum)]
    dynsym = next(s for s in secs if s[1] == 11)  # SHT_DYNSYM
    strtab = secs[dynsym[6]]
    names = set()
    for off in range(dynsym[4], dynsym[4] + dynsym[5], 24):
        st_name, st_info, _other, st_shndx = struct.unpack_from("<IBBH", data, off)
        if (st_info & 0xF) == 2 and (st_info >> 4) in (1, 2) and st_shndx != 0:
            end = data.index(b"\0", strtab[4] + st_name)
            names.add(data[strtab[4] + st_name:end].decode())
    return names


def test_only_declared_functions_are_exported(lib):
    # the library is built with hidden symbols: its host functions are
    # exactly the C entry points the headers declare (kernel handles and the
    # HIP runtime's registration data are objects, not functions)
    assert _exported_functions(mx.LIB_PATH) == set(_declared_functions())


def test_status_strings_and_version(lib):
    assert lib.mxfp4_abi_version() == 103
    for s in range(8):
        assert lib.mxfp4_status_str(s)
    assert lib.mxfp4_status_str(99) == b"unknown status"


@pytest.mark.parametrize("rows,K", [(1, 32), (16, 5120), (37, 4128), (300, 256), (8192, 14336)])
def test_scale_bytes_match_oracle_geometry(lib, rows, K):
    assert lib.mxfp4_scale_bytes(rows, K, 0) == rows * K // 32
    assert lib.mxfp4_scale_bytes(rows, K, 1) == L.gemm_scale_geometry(rows, K)[3]
    assert lib.mxfp4_data_bytes(rows, K, 0) == rows * K // 2
    assert lib.mxfp4_data_bytes(rows, K, 1) == L.weight_geometry(rows, K)[2]


@pytest.mark.parametrize("B,N,K", [(1, 96, 4128), (1, 34816, 5120), (16, 512, 192), (16, 256, 512)])
def test_weight_bytes_match_oracle_geometry(lib, B, N, K):
    assert lib.mxfp4_weight_bytes(B, N, K) == B * L.weight_geometry(N, K)[2]
    assert lib.mxfp4_weight_scale_bytes(B, N, K) == B * L.gemm_scale_geometry(N, K)[3]


def test_size_queries_reject_bad_shapes(lib):
    assert lib.mxfp4_scale_bytes(4, 48, 0) == 0
    assert lib.mxfp4_scale_bytes(4, 64, 7) == 0
    assert lib.mxfp4_weight_bytes(0, 16, 64) == 0
    assert lib.mxfp4_gemm_workspace_bytes(16, 1024, 5120) == 0
    assert lib.mxfp4_gemm_workspace_bytes(128, 8192, 14336) == 0       # 64 rows per small-M launch


# Fake, suitably aligned addresses: every call below fails validation before
# anything could dereference them.
P = ctypes.c_void_p(0x100000)
P_ODD = ctypes.c_void_p(0x100004)


def test_quant_validation(lib):
    f = lib.mxfp4_quant_1x32
    assert f(P, 4, 64, 64, P, 32, P, 5, None) == 7             # bad layout
    assert f(P, 4, 48, 48, P, 24, P, 0, None) == 2             # K % 32
    assert f(P, -1, 64, 64, P, 32, P, 0, None) == 2            # M < 0
    assert f(P, 4, 64, 32, P, 32, P, 0, None) == 2             # ldx < K
    assert f(P, 4, 64, 64, P, 16, P, 0, None) == 2             # ldq < K/2
    assert f(None, 4, 64, 64, P, 32, P, 1, None) == 1          # NULL x
    assert f(P_ODD, 4, 64, 64, P, 32, P, 1, None) == 3         # x misaligned
    assert f(P, 4, 64, 68, P, 32, P, 1, None) == 3             # ldx % 8
    assert f(P, 4, 64, 64, P_ODD, 32, P, 1, None) == 3         # GEMM-layout q not 16-aligned
    assert f(None, 0, 64, 64, None, 32, None, 1, None) == 0    # M == 0: nothing to do


def test_preshuffle_validation(lib):
    f = lib.mxfp4_preshuffle_weight
    assert f(P, P, 1, 16, 40, P, P, None) == 2
    assert f(P, P, 0, 16, 64, P, P, None) == 2
    assert f(None, P, 1, 16, 64, P, P, None) == 1
    assert f(P_ODD, P, 1, 16, 64, P, P, None) == 3


def test_gemm_validation(lib):
    f = lib.mxfp4_gemm_a4w4
    ok = dict(a=P, as_=P, w=P, ws=P, bias=None, out=P, ldo=16, dt=0, M=4, N=16, K=64)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return f(d["a"], d["as_"], d["w"], d["ws"], d["bias"], d["out"], d["ldo"],
                 d["dt"], d["M"], d["N"], d["K"], None, 0, None)

    assert call(dt=3) == 7
    assert call(K=48) == 2
    assert call(N=0) == 2
    assert call(M=-1) == 2
    assert call(ldo=8) == 2         # ldo < N
    assert call(ldo=1 << 22) == 2   # 256 bf16 rows past 32-bit offsets
    assert call(ldo=1 << 21, dt=1) == 2
    assert call(w=None) == 1
    assert call(a=P_ODD) == 3
    assert call(M=0, a=None) == 0   # nothing to do


def test_linear_validation(lib):
    f = lib.mxfp4_linear
    assert lib.mxfp4_linear_workspace_bytes(4, 1024, 5120) == 0         # fused: none
    need = lib.mxfp4_linear_workspace_bytes(17, 1024, 5120)
    assert need >= L.weight_geometry(17, 5120)[2] + L.gemm_scale_geometry(17, 5120)[3]
    assert lib.mxfp4_linear_workspace_bytes(5, 1024, 5120) > 0
    assert lib.mxfp4_linear_workspace_bytes(17, 1024, 48) == 0          # K % 32

    def call(x=P, ldx=64, w=P, ws=P, bias=None, out=P, ldo=16, dt=0, M=4, N=16, K=64,
             work=None, work_bytes=0):
        return f(x, ldx, w, ws, bias, out, ldo, dt, M, N, K, work, work_bytes, None)

    assert call(dt=2) == 7
    assert call(K=48) == 2
    assert call(ldx=32) == 2          # ldx < K
    assert call(ldo=8) == 2           # ldo < N
    assert call(M=4, ldx=1 << 29) == 2    # x beyond one 32-bit buffer range
    assert call(M=17) == 4            # workspace missing
    assert call(M=17, work=P, work_bytes=need - 1, K=5120, ldx=5120) == 4
    assert call(x=None) == 1
    assert call(M=17, work=None, work_bytes=1 << 30) == 1
    assert call(x=P_ODD) == 3
    assert call(ldx=68) == 3
    assert call(M=17, work=P_ODD, work_bytes=1 << 30) == 3
    assert call(M=0, x=None) == 0


def test_mxfp4_out_validation(lib):
    f = lib.mxfp4_gemm_a4w4_mxfp4_out

    def call(a=P, as_=P, w=P, ws=P, bias=None, q=P, ldq=16, s=P, lds=1, M=4, N=32, K=64):
        return f(a, as_, w, ws, bias, q, ldq, s, lds, M, N, K, None, 0, None)

    assert call(N=48) == 2            # N % 32
    assert call(ldq=8) == 2           # ldq < N/2
    assert call(lds=0) == 2           # lds < N/32
    assert call(ldq=1 << 23) == 2
    assert call(s=None) == 1
    assert call(ldq=18) == 3          # ldq % 4
    assert call(q=P_ODD.value + 2) == 3
    assert call(M=0, a=None) == 0


def test_shuffle_scales_and_prequantized_validation(lib):
    f = lib.mxfp4_shuffle_scales
    assert f(P, 4, 8, 100, P, None) == 2        # K % 32
    assert f(P, 2, 8, 128, P, None) == 2        # lds < K/32
    assert f(None, 4, 8, 128, P, None) == 1
    assert f(P, 4, 8, 128, P_ODD.value + 1, None) == 3
    assert f(None, 4, 0, 128, None, None) == 0  # no rows
    g = lib.mxfp4_linear_prequantized
    assert lib.mxfp4_linear_prequantized_workspace_bytes(64, 96, 4128) == 0
    # up to 256 rows on few columns (ceil(M/64) * N <= 16384) the small-M
    # kernel reads the row-major operands itself, 64 rows per launch: no
    # workspace
    assert lib.mxfp4_linear_prequantized_workspace_bytes(128, 8192, 4128) == 0
    assert lib.mxfp4_linear_prequantized_workspace_bytes(256, 4096, 4128) == 0
    # ... except with many rows per launch on long K, or on many strips,
    # where the operands are permuted into the GEMM layouts first
    assert lib.mxfp4_linear_prequantized_workspace_bytes(32, 96, 14336) == 0
    assert lib.mxfp4_linear_prequantized_workspace_bytes(48, 96, 4096) == 0
    assert lib.mxfp4_linear_prequantized_workspace_bytes(16, 8192, 8192) == 0
    for M, N, K in [(64, 96, 14336), (33, 96, 8704), (100, 96, 6656), (48, 96, 5120), (16, 10240, 8192)]:
        need = lib.mxfp4_linear_prequantized_workspace_bytes(M, N, K)
        assert need >= L.weight_geometry(M, K)[2] + L.gemm_scale_geometry(M, K)[3]
    for M, N in [(257, 96), (65, 8208), (192, 6144)]:
        need = lib.mxfp4_linear_prequantized_workspace_bytes(M, N, 4128)
        assert need >= L.weight_geometry(M, 4128)[2] + L.gemm_scale_geometry(M, 4128)[3]

    def call(x=P, ldq=32, s=P, lds=2, w=P, ws=P, bias=None, out=P, ldo=16, dt=0, M=4, N=16, K=64,
             work=None, work_bytes=0):
        return g(x, ldq, s, lds, w, ws, bias, out, ldo, dt, M, N, K, work, work_bytes, None)

    assert call(dt=5) == 7
    assert call(K=48) == 2
    assert call(ldq=16) == 2          # ldq < K/2
    assert call(lds=1) == 2           # lds < K/32
    assert call(M=257) == 4           # workspace missing
    assert call(M=65, N=8208, ldo=8208) == 4
    assert call(s=None) == 1
    assert call(ldq=40) == 3          # ldq % 16
    assert call(x=P_ODD) == 3
    assert call(M=0, x=None, s=None) == 0


def test_bmm_validation(lib):
    f = lib.a16wfp4_bmm

    def call(x=P, sxb=64 * 192, sxm=192, w=P, ws=P, out=P, sob=64 * 512, som=512, dt=0,
             B=16, M=64, N=512, K=192):
        return f(x, sxb, sxm, w, ws, out, sob, som, dt, B, M, N, K, None)

    assert call(dt=2) == 7
    assert call(K=100) == 2
    assert call(B=0) == 2
    assert call(sxm=100) == 2
    assert call(x=None) == 1
    assert call(sxm=196) == 3
    assert call(som=513, sob=64 * 514) == 3                    # odd row stride
    assert call(M=0, x=None) == 0
    # output rows that would overlap are rejected before any other check
    assert call(som=510) == 2                                  # rows closer than N
    assert call(sob=512, som=512) == 2                         # heads on top of each other
    assert call(sob=63 * 512 + 510) == 2                       # head b's rows reach head b+1
    assert call(M=1, som=0, x=None) == 1                       # one row: its stride is moot
    assert call(B=1, sob=0, x=None) == 1                       # one head: its stride is moot
    assert call(sob=512, som=16 * 512, x=None) == 1            # batch-major [M, B, N]
    assert call(sob=64 * 520, som=520, x=None) == 1            # padded rows


def test_valid_call_without_gpu_reports_device(lib):
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: fake pointers must not reach a kernel")
    assert lib.mxfp4_quant_1x32(P, 4, 64, 64, P, 32, P, 1, None) == 5
    assert lib.mxfp4_quant_1x32(P, 4, 64, 64, P, 0, P, 1, None) == 5   # ldq ignored (GEMM layout)
    assert lib.mxfp4_gemm_a4w4(P, P, P, P, None, P, 16, 0, 4, 16, 64, None, 0, None) == 5
    assert lib.mxfp4_linear(P, 64, P, P, None, P, 16, 0, 4, 16, 64, None, 0, None) == 5


def test_testing_path_hook(lib):
    assert lib.mxfp4_testing_set_gemm_path(9) == 7
    assert lib.mxfp4_testing_set_gemm_path(-1) == 7
    for path in (8, 7, 6, 5, 4, 3, 2, 1, 0):
        assert lib.mxfp4_testing_set_gemm_path(path) == 0


def test_testing_path_hook_is_per_thread(lib):
    # a path forced on another thread changes neither this thread's plan
    # nor its workspace size
    import threading
    base = lib.mxfp4_gemm_workspace_bytes(2048, 34816, 5120)
    seen = {}

    def other():
        lib.mxfp4_testing_set_gemm_path(4)
        seen["other"] = lib.mxfp4_gemm_workspace_bytes(2048, 34816, 5120)
        lib.mxfp4_testing_set_gemm_path(0)

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["other"] == _split_bytes(256, 64) != base == 0
    assert lib.mxfp4_gemm_workspace_bytes(2048, 34816, 5120) == base
    assert "mxfp4_testing_set_gemm_path" not in open(HEADERS[0]).read()


# The large-M kernel's plan (256 compute units): 128-wide output tiles where
# 256-wide ones fill at most half a round and 128-wide ones fit in one; then
# the split schedule: the r tiles short of whole rounds are cut along K into
# s = 256 / r slices, one per workgroup, where the slices stay long enough to
# pay for their parts' traffic; its workspace is one fp32 256 x bn part per
# workgroup, after a give-up word, a counter per split tile and a flag per
# workgroup (those words rounded up to 256 bytes).
def _split_bytes(grid, r, bn=256):
    return grid * 256 * bn * 4 + (4 * (1 + r + grid) + 255) // 256 * 256


@pytest.mark.parametrize("M,N,K,grid,r,bn", [
    (8192, 5120, 14336, 256, 128, 256),  # 640 tiles: 128 left over, 2 slices of 14 groups
    (512, 5120, 14336, 240, 80, 128),    # 40 tiles, 128 wide: 80, 3 slices of 9-10 groups
    (1024, 5120, 14336, 0, 0, 128),      # 128 wide: 160 tiles, more than half a round
    (2048, 5120, 14336, 0, 0, 256),      # 160 tiles: more than half a round left over
    (2048, 34816, 5120, 0, 0, 256),      # 1088 tiles: slices of 2-3 groups would not pay
    (512, 14336, 5120, 0, 0, 128),       # 112 tiles; 128 wide: 224 whole tiles
    (8192, 14336, 5120, 0, 0, 256),      # 1792 tiles: whole rounds
    (37, 96, 4128, 0, 0, 128),           # one tile: slices of one group
    (64, 5120, 14336, 0, 0, 0),          # M <= 64: the small-M kernel
])
def test_split_schedule_workspace(lib, M, N, K, grid, r, bn):
    want = _split_bytes(grid, r, bn) if grid else 0
    assert lib.mxfp4_gemm_workspace_bytes(M, N, K) == want
    if M > 64:
        # the quantised activations, then the GEMM's part
        quant = L.weight_geometry(M, K)[2] + L.gemm_scale_geometry(M, K)[3]
        assert lib.mxfp4_linear_workspace_bytes(M, N, K) >= quant + want
        assert lib.mxfp4_linear_prequantized_workspace_bytes(M, N, K) >= quant + want


def test_split_schedule_forced_and_whole(lib):
    try:
        assert lib.mxfp4_testing_set_gemm_path(3) == 0
        assert lib.mxfp4_gemm_workspace_bytes(8192, 5120, 14336) == 0
        assert lib.mxfp4_testing_set_gemm_path(4) == 0
        # forced: wherever a round is left part-empty and a tile has 2+ groups
        assert lib.mxfp4_gemm_workspace_bytes(2048, 34816, 5120) == _split_bytes(256, 64)
        assert lib.mxfp4_gemm_workspace_bytes(300, 520, 1056) == _split_bytes(18, 6)
        assert lib.mxfp4_gemm_workspace_bytes(37, 96, 4128) == _split_bytes(9, 1)
        assert lib.mxfp4_gemm_workspace_bytes(300, 128, 256) == 0        # one group: nothing to split
        assert lib.mxfp4_gemm_workspace_bytes(8192, 14336, 5120) == 0    # whole rounds
        assert lib.mxfp4_gemm_workspace_bytes(2048, 5120, 14336) == 0    # 256 / 160: one slice
        assert lib.mxfp4_testing_set_gemm_path(6) == 0                      # 128 wide, split forced
        assert lib.mxfp4_gemm_workspace_bytes(2048, 5120, 14336) == _split_bytes(256, 64, 128)
        assert lib.mxfp4_testing_set_gemm_path(5) == 0                      # 128 wide, whole tiles
        assert lib.mxfp4_gemm_workspace_bytes(512, 5120, 14336) == 0
    finally:
        lib.mxfp4_testing_set_gemm_path(0)


def test_split_schedule_workspace_validation(lib):
    f = lib.mxfp4_gemm_a4w4
    need = lib.mxfp4_gemm_workspace_bytes(8192, 5120, 14336)
    assert need > 0

    def call(work=None, work_bytes=0):
        return f(P, P, P, P, None, P, 5120, 0, 8192, 5120, 14336, work, work_bytes, None)

    assert call() == 4                                  # workspace missing
    assert call(P, need - 1) == 4                       # too small
    assert call(None, need) == 1                        # NULL with a size
    assert call(P_ODD, need) == 3                       # misaligned
    g = lib.mxfp4_gemm_a4w4_mxfp4_out
    assert g(P, P, P, P, None, P, 2560, P, 160, 8192, 5120, 14336, None, 0, None) == 4
    assert g(P, P, P, P, None, P, 2560, P, 160, 8192, 5120, 14336, P_ODD, need, None) == 3
