"""The large-M tile split and the 32-bit addressing guard of the library, checked on the CPU.

csrc/mm_policy.h is plain constexpr C++ (hipcc compiles it for the GPU kernels, the host
launcher and the route kernel); here the host C++ compiler builds it with a small ctypes driver
(tests/native/policy_check.cpp).  The split's invariants are checked for every expert size below
200000 rows; the guard at the exact 4 GiB boundaries of each buffer it covers.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dispatch_fp8_grouped_topk_amd", "csrc")


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    out = tmp_path_factory.mktemp("policy") / "policy_check.so"
    subprocess.run([cxx, "-O2", "-std=c++17", "-shared", "-fPIC", "-I", CSRC,
                    os.path.join(ROOT, "tests", "native", "policy_check.cpp"), "-o", str(out)], check=True)
    L = ctypes.CDLL(str(out))
    L.pc_addressable.argtypes = [ctypes.c_int64] * 4
    L.pc_check_all.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    return L


def test_split_invariants_every_size(lib):
    what = ctypes.c_int(-1)
    bad = lib.pc_check_all(200000, ctypes.byref(what))
    assert bad == 0, f"expert of {bad} rows violates invariant {what.value}"


def _tiles(lib, c):
    n = lib.pc_large_tiles(c)
    st = [lib.pc_large_tile_start(c, i) for i in range(n)] + [c]
    return [st[i + 1] - st[i] for i in range(n)]


def test_split_hand_worked(lib):
    # 800 rows = 50 groups of 16 over 4 tiles: 25 pairs, 6 each and one more for tile 0
    # (14, 12, 12, 12 groups); no odd group
    assert _tiles(lib, 800) == [224, 192, 192, 192]
    # 801 rows = 51 groups: the odd 51st group goes to tile r = 1, the first with q pairs
    assert _tiles(lib, 801) == [224, 208, 192, 177]
    # one tile: all rows; column groups per wave = ceil(ceil(c / 16) / 2)
    assert _tiles(lib, 1) == [1] and lib.pc_large_first_ng(1) == 1
    assert _tiles(lib, 256) == [256] and lib.pc_large_first_ng(256) == 8
    assert _tiles(lib, 257) == [144, 113] and lib.pc_large_first_ng(257) == 5
    assert lib.pc_large_first_ng(81) == 3


def test_addressing_guard_boundaries(lib):
    A = lib.pc_addressable
    G = 1 << 32
    # x [T, H]: T*H = 2^32 - 128 fits, 2^32 does not
    assert A(G // 128 - 1, 128, 128, 1) == 1
    assert A(G // 128, 128, 128, 1) == 0
    # intermediate [T k, I]
    assert A(G // (128 * 64), 128, 128, 64) == 0
    assert A(G // (128 * 64) - 1, 128, 128, 64) == 1
    # pool-order scale words [H/128, T k] x 4 bytes: with k = 64 this is the binding one
    H, k, I = 16384, 64, 128
    T = G // ((H // 128) * k * 4)              # exactly 4 GiB of scale words
    assert T * H < G and T * k * I < G         # the other two buffers still fit
    assert A(T, H, I, k) == 0 and A(T - 1, H, I, k) == 1
    # the decode and prefill workloads are far inside the limits
    assert A(128, 7168, 2048, 8) == 1 and A(8192, 7168, 2048, 8) == 1
