"""The C ABI library on the CPU: it loads, exports every function include/mega_moe.h declares,
sizes workspaces and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest
import torch

import dispatch_fp8_grouped_topk_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(mega_moe_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_function():
    lib = mm.library()
    declared = _declared_functions()
    assert {"mega_moe_forward", "mega_moe_workspace_size", "mega_moe_workspace_views",
            "mega_moe_strerror", "mega_moe_abi_version"} <= declared
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_strerror():
    assert mm.mega_moe_abi_version() == mm.ABI_VERSION
    assert mm.mega_moe_strerror(0) == "ok"
    for st in range(-7, 0):
        assert mm.mega_moe_strerror(st) != "unknown status"


def test_noalloc_refuses_problems_beyond_its_scratch_before_touching_a_device():
    """mega_moe_forward_noalloc checks the problem's workspace size against its static scratch
    first: a problem that does not fit is refused (no pointer or device is looked at)."""
    lib = mm.library()
    big = _p(T=4096)                       # 0.5 GiB of workspace at the decode shape
    assert mm.mega_moe_workspace_size(big) > mm.NOALLOC_SCRATCH_BYTES
    st = lib.mega_moe_forward_noalloc(ctypes.byref(big), *([None] * 9), None)
    assert st == mm.ERR_SCRATCH_TOO_SMALL
    assert "static scratch" in mm.mega_moe_strerror(st)
    bad = _p(H=100)
    assert lib.mega_moe_forward_noalloc(ctypes.byref(bad), *([None] * 9), None) == -1
    assert lib.mega_moe_forward_noalloc(ctypes.byref(_p(T=0)), *([None] * 9), None) == 0


def _p(**kw):
    base = dict(T=128, H=7168, I=2048, E=256, k=8)
    base.update(kw)
    return mm.Problem.make(base["T"], base["H"], base["I"], base["E"], base["k"],
                           base.get("recipe", 0), base.get("clamp", 0.0), base.get("flags", 0))


def test_workspace_size_grows_with_tokens_and_covers_buffers():
    s1 = mm.mega_moe_workspace_size(_p(T=128))
    s2 = mm.mega_moe_workspace_size(_p(T=8192))
    assert s2 > s1
    P = 8192 * 8
    # at least the BF16 slot rows, the FP8 intermediate and its scales
    assert s2 >= P * 7168 * 2 + P * 2048 + P * 16 * 4
    s4 = mm.mega_moe_workspace_size(_p(T=4096, E=257, k=9, recipe=1))
    assert s4 >= 4096 * 9 * (7168 * 2 + 2048 + 2048 // 32)
    assert mm.mega_moe_workspace_size(_p(T=0)) > 0
    # the E4M3-weight per-32 recipe keeps the MXFP4 recipe's UE8M0 intermediate scales
    assert mm.mega_moe_workspace_size(_p(T=4096, E=257, k=9, recipe=2)) == s4


@pytest.mark.parametrize("kw", [dict(H=100), dict(H=0), dict(I=96), dict(E=0), dict(E=10 ** 6), dict(k=0),
                                dict(k=65), dict(recipe=3), dict(recipe=-1), dict(clamp=-1.0), dict(clamp=float("nan")),
                                dict(flags=256), dict(flags=3), dict(flags=15), dict(flags=16), dict(T=-1), dict(H=32768),
                                # the row-pair weight layout: E2M1 weights only
                                dict(flags=128), dict(flags=128, recipe=2),
                                # the fused forward runs the large-M tiles only
                                dict(flags=64 | 1),
                                # per-64 intermediate scales: the float-scale recipe only
                                dict(flags=32, recipe=1), dict(flags=32, recipe=2)])
def test_invalid_problem_rejected(kw):
    with pytest.raises(mm.MegaMoEError) as ei:
        mm.mega_moe_workspace_size(_p(**kw))
    assert ei.value.status == -1


def test_numerics_flags_accepted_with_either_tile_class():
    for flags in (4, 5, 6, 8, 12, 14):
        assert mm.mega_moe_workspace_size(_p(clamp=1.0, flags=flags)) > 0


def test_weight_sf_kmajor_flag_only_with_per32_recipes():
    # flag 16 (K-major weight scales) is rejected above for the float-scale recipe
    for recipe in (1, 2):
        for flags in (16, 17, 18, 30):
            assert mm.mega_moe_workspace_size(_p(recipe=recipe, clamp=1.0, flags=flags)) > 0


def test_weight_e2m1_paired_flag_only_with_mxfp4():
    for flags in (128, 128 | 16, 128 | 1, 128 | 64):
        assert mm.mega_moe_workspace_size(_p(recipe=1, flags=flags)) > 0


def _transform_w_raw(problem, ptrs):
    lib = mm.library()
    args = [ctypes.c_void_p(p) if p is not None else None for p in ptrs]
    return lib.mega_moe_transform_weights(ctypes.byref(problem), *args, None)


def test_transform_weights_validates_before_any_device_work():
    # E2M1 weights of one expert at H = I = 128: l1 16 KiB, l2 8 KiB, at addresses 1 MiB apart;
    # nothing is dereferenced (see the scale transform's test)
    small = dict(T=1, H=128, I=128, E=1, k=1)
    good = [1 << 20, 2 << 20, 3 << 20, 4 << 20]
    assert _transform_w_raw(_p(recipe=0, **small), good) == -1              # FP8 weights
    assert _transform_w_raw(_p(recipe=2, **small), good) == -1              # E4M3 weights
    assert _transform_w_raw(_p(recipe=1, **dict(small, H=100)), good) == -1  # invalid problem
    for i in range(4):
        bad = list(good)
        bad[i] = None
        assert _transform_w_raw(_p(recipe=1, **small), bad) == -2
    assert _transform_w_raw(_p(recipe=1, **small), [good[0] + 4] + good[1:]) == -3
    assert _transform_w_raw(_p(recipe=1, **small), [good[0], good[1], good[0] + 8192, good[3]]) == -1
    assert _transform_w_raw(_p(recipe=1, **small), [good[0], good[1], good[2], good[1] + 4096]) == -1
    if not torch.cuda.is_available():
        assert _transform_w_raw(_p(recipe=1, **small), good) in (-5, -6)   # no device to run on


def _transform_raw(problem, ptrs):
    lib = mm.library()
    args = [ctypes.c_void_p(p) if p is not None else None for p in ptrs]
    return lib.mega_moe_transform_weight_scales(ctypes.byref(problem), *args, None)


def test_transform_weight_scales_validates_before_any_device_work():
    # small tensors (l1 scales 1 KiB, l2 512 B) at addresses 1 MiB apart never overlap; no address
    # is dereferenced: every case returns before the device is touched (on a host without a GPU
    # the valid call stops at the device check)
    small = dict(T=1, H=128, I=128, E=1, k=1)
    good = [1 << 20, 2 << 20, 3 << 20, 4 << 20]
    assert _transform_raw(_p(recipe=0, **small), good) == -1              # float-scale recipe
    assert _transform_raw(_p(recipe=1, **dict(small, H=100)), good) == -1  # invalid problem
    for i in range(4):
        bad = list(good)
        bad[i] = None
        assert _transform_raw(_p(recipe=2, **small), bad) == -2
    assert _transform_raw(_p(recipe=1, **small), [good[0] + 4] + good[1:]) == -3
    # in place (output overlapping its input) is rejected, out of place gets past validation
    assert _transform_raw(_p(recipe=2, **small), [good[0], good[1], good[0] + 512, good[3]]) == -1
    assert _transform_raw(_p(recipe=2, **small), [good[0], good[1], good[1] + 256, good[3]]) == -1
    if not torch.cuda.is_available():
        assert _transform_raw(_p(recipe=2, **small), good) in (-5, -6)   # no device to run on


def _forward_raw(problem, ptrs, ws_bytes):
    lib = mm.library()
    args = [ctypes.c_void_p(p) if p is not None else None for p in ptrs]
    return lib.mega_moe_forward(ctypes.byref(problem), *args[:9], args[9], ws_bytes, None)


def test_forward_argument_errors_without_a_device():
    p = _p(T=4, H=256, I=128, E=4, k=2)
    need = mm.mega_moe_workspace_size(p)
    good = [0x10000 * (i + 1) for i in range(10)]
    assert _forward_raw(p, [None] + good[1:], need) == -2          # NULL x
    bad = list(good)
    bad[3] += 4
    assert _forward_raw(p, bad, need) == -3                        # misaligned topk_w
    assert _forward_raw(p, good, need - 1) == -4                   # workspace too small
    p0 = _p(T=0, H=256, I=128, E=4, k=2)
    assert _forward_raw(p0, [None] * 10, 0) == 0                   # T == 0: no-op
    pbad = _p(T=4, H=200, I=128, E=4, k=2)
    assert _forward_raw(pbad, good, need) == -1


def test_views_null_workspace_rejected():
    v = mm._Views()
    lib = mm.library()
    p = _p(T=4, H=256, I=128, E=4, k=2)
    assert lib.mega_moe_workspace_views(ctypes.byref(p), None, ctypes.byref(v)) == -2
