"""Python binding of libmegamoe, the MI355X (gfx950) MegaMoE expert-layer library.

Argument marshalling only: torch tensors are passed to the C ABI (include/mega_moe.h) as raw
device pointers together with the current HIP stream; every step of the layer runs in the
library's HIP kernels.  There is no fallback: if the shared library is missing or fails to
load, importing the binding's functions raises.

Functions carry the C names:

    mega_moe_workspace_size(problem) -> int
    mega_moe_forward(problem, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y,
                     workspace, stream=None)
    mega_moe_workspace_views(problem, workspace) -> dict of torch views into the workspace
    mega_moe_strerror(status) -> str
    mega_moe_abi_version() -> int
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmegamoe.so")

RECIPE_FP8_B128 = 0
RECIPE_MXFP4W_B32 = 1
RECIPE_MXFP8_B32 = 2
FLAG_TILE_AUTO = 0
FLAG_TILE_SMALL = 1
FLAG_TILE_LARGE = 2
FLAG_CLAMP_INPUTS = 4   # with swiglu_clamp > 0: clamp gate and up before SiLU
FLAG_PRECISE_SILU = 8   # SiLU with expf and IEEE division instead of the hardware exp / rcp
FLAG_WEIGHT_SF_KMAJOR = 16   # per-32 recipes: weight scales from mega_moe_transform_weight_scales
FLAG_INTER_SF64 = 32         # FP8 recipe: intermediate float scales per 64 channels (L2 in two halves)
FLAG_FUSED = 64              # the whole forward in one persistent cooperative launch
FLAG_WEIGHT_E2M1_PAIRED = 128  # MXFP4: E2M1 weights in the row-pair layout of mega_moe_transform_weights

ABI_VERSION = 1


class MegaMoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {mega_moe_strerror(status)} (status {status})")
        self.status = status


class Problem(ctypes.Structure):
    """mega_moe_problem."""
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("recipe", ctypes.c_int32),
        ("swiglu_clamp", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]

    @classmethod
    def make(cls, T, H, I, E, k, recipe=RECIPE_FP8_B128, swiglu_clamp=0.0, flags=0):
        return cls(int(T), int(H), int(I), int(E), int(k), int(recipe), float(swiglu_clamp), int(flags))


class _Views(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("expert_count", "expert_offset", "pool_src", "pair_pos", "num_invalid",
                 "inter_q", "inter_sf", "slot")]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m dispatch_fp8_grouped_topk_amd.build`")
    # torch first: its HIP runtime (soname libamdhip64.so.7) is then the one the library binds
    # to, so torch streams and the library's launches share one runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp = ctypes.c_void_p
    lib.mega_moe_abi_version.restype = ctypes.c_int
    lib.mega_moe_abi_version.argtypes = []
    lib.mega_moe_strerror.restype = ctypes.c_char_p
    lib.mega_moe_strerror.argtypes = [ctypes.c_int]
    lib.mega_moe_workspace_size.restype = ctypes.c_int
    lib.mega_moe_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.mega_moe_workspace_views.restype = ctypes.c_int
    lib.mega_moe_workspace_views.argtypes = [P, vp, ctypes.POINTER(_Views)]
    lib.mega_moe_forward.restype = ctypes.c_int
    lib.mega_moe_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.mega_moe_forward_stats.restype = ctypes.c_int
    lib.mega_moe_forward_stats.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.mega_moe_transform_weight_scales.restype = ctypes.c_int
    lib.mega_moe_transform_weight_scales.argtypes = [P, vp, vp, vp, vp, vp]
    lib.mega_moe_transform_weights.restype = ctypes.c_int
    lib.mega_moe_transform_weights.argtypes = [P, vp, vp, vp, vp, vp]
    lib.mega_moe_forward_profiled.restype = ctypes.c_int
    lib.mega_moe_forward_profiled.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp,
                                              ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    lib.mega_moe_forward_noalloc.restype = ctypes.c_int
    lib.mega_moe_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mega_moe_diag_mfma_block_sums.restype = ctypes.c_int
    lib.mega_moe_diag_mfma_block_sums.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int, vp]
    if lib.mega_moe_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI {lib.mega_moe_abi_version()}, expected {ABI_VERSION}")
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (raises if it cannot be loaded)."""
    return _load()


def mega_moe_abi_version() -> int:
    return _load().mega_moe_abi_version()


def mega_moe_strerror(status: int) -> str:
    return _load().mega_moe_strerror(int(status)).decode()


def mega_moe_workspace_size(problem: Problem) -> int:
    out = ctypes.c_size_t(0)
    st = _load().mega_moe_workspace_size(ctypes.byref(problem), ctypes.byref(out))
    if st:
        raise MegaMoEError(st, "mega_moe_workspace_size")
    return out.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensor(name, t, device, dtypes, shape):
    import torch
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def expected_shapes(problem: Problem) -> dict:
    import torch
    T, H, I, E, k = (problem.num_tokens, problem.hidden, problem.intermediate,
                     problem.num_experts, problem.topk)
    u8, f32, i32 = (torch.uint8,), (torch.float32,), (torch.int32,)
    b16 = (torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.bfloat16, torch.int16)
    if problem.recipe == RECIPE_FP8_B128:
        return dict(x=(u8, (T, H)), x_sf=(f32, (T, H // 128)), topk_idx=(i32, (T, k)), topk_w=(f32, (T, k)),
                    l1_w=(u8, (E, 2 * I, H)), l1_sf=(f32, (E, 2 * I // 128, H // 128)),
                    l2_w=(u8, (E, H, I)), l2_sf=(f32, (E, H // 128, I // 128)), y=(b16, (T, H)))
    wk = 1 if problem.recipe == RECIPE_MXFP8_B32 else 2         # K indices per weight byte
    if problem.flags & FLAG_WEIGHT_SF_KMAJOR:
        sf1, sf2 = (E, H // 128, 2 * I, 4), (E, I // 128, H, 4)
    else:
        sf1, sf2 = (E, 2 * I, H // 32), (E, H, I // 32)
    return dict(x=(u8, (T, H)), x_sf=(u8, (T, H // 32)), topk_idx=(i32, (T, k)), topk_w=(f32, (T, k)),
                l1_w=(u8, (E, 2 * I, H // wk)), l1_sf=(u8, sf1),
                l2_w=(u8, (E, H, I // wk)), l2_sf=(u8, sf2), y=(b16, (T, H)))


NUM_PHASE_EVENTS = 5


def mega_moe_transform_weight_scales(problem: Problem, l1_sf, l2_sf, stream=None):
    """The per-32 recipes' one-time weight-scale transform: returns new K-major tensors
    (l1 [E, H/128, 2I, 4], l2 [E, I/128, H, 4] uint8) for forward calls whose problem has
    FLAG_WEIGHT_SF_KMAJOR set."""
    import torch
    dev = l1_sf.device
    if dev.type != "cuda":
        raise ValueError("mega_moe_transform_weight_scales needs device tensors")
    rowmajor = Problem.make(problem.num_tokens, problem.hidden, problem.intermediate, problem.num_experts,
                            problem.topk, problem.recipe, problem.swiglu_clamp,
                            problem.flags & ~FLAG_WEIGHT_SF_KMAJOR)
    shapes = expected_shapes(rowmajor)
    for name, t in (("l1_sf", l1_sf), ("l2_sf", l2_sf)):
        _check_tensor(name, t, dev, *shapes[name])
    E, H, I = problem.num_experts, problem.hidden, problem.intermediate
    out1 = torch.empty(E, H // 128, 2 * I, 4, dtype=torch.uint8, device=dev)
    out2 = torch.empty(E, I // 128, H, 4, dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _load().mega_moe_transform_weight_scales(ctypes.byref(rowmajor), _ptr(l1_sf), _ptr(l2_sf), _ptr(out1),
                                                  _ptr(out2), ctypes.c_void_p(handle))
    if st:
        raise MegaMoEError(st, "mega_moe_transform_weight_scales")
    return out1, out2


def mega_moe_transform_weights(problem: Problem, l1_w, l2_w, stream=None):
    """The MXFP4 recipe's one-time weight transform: returns new tensors of the same shapes
    (l1 [E, 2I, H/2], l2 [E, H, I/2] uint8) holding the E2M1 weights in the row-pair layout, for
    forward calls whose problem has FLAG_WEIGHT_E2M1_PAIRED set."""
    import torch
    dev = l1_w.device
    if dev.type != "cuda":
        raise ValueError("mega_moe_transform_weights needs device tensors")
    rowmajor = Problem.make(problem.num_tokens, problem.hidden, problem.intermediate, problem.num_experts,
                            problem.topk, problem.recipe, problem.swiglu_clamp,
                            problem.flags & ~FLAG_WEIGHT_E2M1_PAIRED)
    shapes = expected_shapes(rowmajor)
    for name, t in (("l1_w", l1_w), ("l2_w", l2_w)):
        _check_tensor(name, t, dev, *shapes[name])
    out1, out2 = torch.empty_like(l1_w), torch.empty_like(l2_w)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _load().mega_moe_transform_weights(ctypes.byref(rowmajor), _ptr(l1_w), _ptr(l2_w), _ptr(out1),
                                            _ptr(out2), ctypes.c_void_p(handle))
    if st:
        raise MegaMoEError(st, "mega_moe_transform_weights")
    return out1, out2


def mega_moe_forward(problem: Problem, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y,
                     workspace, stream=None, recv_stats=None) -> None:
    """Enqueue the layer forward on ``stream`` (default: torch's current stream of x's device).
    recv_stats: optional int32 [E] device tensor to which each expert's received row count is
    added (mega_moe_forward_stats)."""
    _forward(problem, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y, workspace, stream, None,
             recv_stats)


NOALLOC_SCRATCH_BYTES = 32 << 20
ERR_SCRATCH_TOO_SMALL = -7


def mega_moe_forward_noalloc(problem: Problem, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y,
                             stream=None) -> None:
    """mega_moe_forward without a workspace: the library's static per-GPU scratch
    (NOALLOC_SCRATCH_BYTES) serves instead, so nothing is allocated.  Calls that overlap on one GPU
    race on that scratch; larger problems raise MegaMoEError with ERR_SCRATCH_TOO_SMALL."""
    import torch
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("mega_moe_forward_noalloc needs device tensors")
    shapes = expected_shapes(problem)
    tensors = dict(x=x, x_sf=x_sf, topk_idx=topk_idx, topk_w=topk_w, l1_w=l1_w, l1_sf=l1_sf,
                   l2_w=l2_w, l2_sf=l2_sf, y=y)
    for name, t in tensors.items():
        dts, shp = shapes[name]
        _check_tensor(name, t, dev, dts, shp)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _load().mega_moe_forward_noalloc(ctypes.byref(problem), _ptr(x), _ptr(x_sf), _ptr(topk_idx),
                                          _ptr(topk_w), _ptr(l1_w), _ptr(l1_sf), _ptr(l2_w), _ptr(l2_sf),
                                          _ptr(y), ctypes.c_void_p(handle))
    if st:
        raise MegaMoEError(st, "mega_moe_forward_noalloc")


def mega_moe_forward_profiled(problem: Problem, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y,
                              workspace, events, stream=None) -> None:
    """mega_moe_forward that also records the given raw hipEvent_t handles (ints) at the
    phase boundaries: before dispatch, after dispatch, after L1, after L2, after combine."""
    _forward(problem, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y, workspace, stream, events)


def _forward(problem, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y, workspace, stream, events,
             recv_stats=None):
    import torch
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("mega_moe_forward needs device tensors")
    shapes = expected_shapes(problem)
    tensors = dict(x=x, x_sf=x_sf, topk_idx=topk_idx, topk_w=topk_w, l1_w=l1_w, l1_sf=l1_sf,
                   l2_w=l2_w, l2_sf=l2_sf, y=y)
    for name, t in tensors.items():
        dts, shp = shapes[name]
        _check_tensor(name, t, dev, dts, shp)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    nbytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    args = (ctypes.byref(problem), _ptr(x), _ptr(x_sf), _ptr(topk_idx), _ptr(topk_w),
            _ptr(l1_w), _ptr(l1_sf), _ptr(l2_w), _ptr(l2_sf), _ptr(y),
            _ptr(workspace), nbytes, ctypes.c_void_p(handle))
    if recv_stats is not None:
        _check_tensor("recv_stats", recv_stats, dev, (torch.int32,), (problem.num_experts,))
        st = _load().mega_moe_forward_stats(*args[:-1], _ptr(recv_stats), args[-1])
        what = "mega_moe_forward_stats"
    elif events is None:
        st = _load().mega_moe_forward(*args)
        what = "mega_moe_forward"
    else:
        arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(int(e)) for e in events])
        st = _load().mega_moe_forward_profiled(*args, arr, len(events))
        what = "mega_moe_forward_profiled"
    if st:
        raise MegaMoEError(st, what)


def mega_moe_workspace_views(problem: Problem, workspace) -> dict:
    """Torch views (on the workspace's device) of the dispatch metadata and intermediates."""
    import torch
    v = _Views()
    st = _load().mega_moe_workspace_views(ctypes.byref(problem), _ptr(workspace), ctypes.byref(v))
    if st:
        raise MegaMoEError(st, "mega_moe_workspace_views")
    base = workspace.data_ptr()
    raw = workspace.view(torch.uint8).reshape(-1)
    T, H, I, E, k = (problem.num_tokens, problem.hidden, problem.intermediate,
                     problem.num_experts, problem.topk)
    P = T * k
    gi = 64 if problem.flags & FLAG_INTER_SF64 else 128     # channels per float intermediate scale

    def view(addr, nbytes, dtype, shape):
        off = addr - base
        return raw[off:off + nbytes].view(dtype).reshape(shape)

    return dict(
        expert_count=view(v.expert_count, 4 * E, torch.int32, (E,)),
        expert_offset=view(v.expert_offset, 4 * (E + 1), torch.int32, (E + 1,)),
        pool_src=view(v.pool_src, 4 * P, torch.int32, (P,)),
        pair_pos=view(v.pair_pos, 4 * P, torch.int32, (P,)),
        num_invalid=view(v.num_invalid, 4, torch.int32, (1,)),
        inter_q=view(v.inter_q, P * I, torch.uint8, (P, I)),
        inter_sf=(view(v.inter_sf, P * (I // gi) * 4, torch.float32, (I // gi, P)).t()
                  if problem.recipe == RECIPE_FP8_B128 else
                  view(v.inter_sf, P * (I // 32), torch.uint8, (I // 128, P, 4)).permute(1, 0, 2).reshape(P, I // 32)),
        slot=view(v.slot, P * H * 2, torch.int16, (P, H)),
    )


def mega_moe_diag_mfma_block_sums(fmt: int, a, b, a_scale=None, b_scale=None, stream=None):
    """16 x 16 block dot products over one 128-K block with the GEMMs' MFMA instruction.
    a: uint8 [n, 16, 128] (fmt 1: [n, 16, 64] packed E2M1), b: uint8 [n, 16, 128]; scales uint8
    [n, 16, 4] for fmt 1 and 2.  Returns float32 [n, 16, 16]."""
    import torch
    dev = b.device
    n = b.shape[0]
    a_cols = 64 if fmt == 1 else 128
    _check_tensor("a", a, dev, (torch.uint8,), (n, 16, a_cols))
    _check_tensor("b", b, dev, (torch.uint8,), (n, 16, 128))
    if fmt != 0:
        _check_tensor("a_scale", a_scale, dev, (torch.uint8,), (n, 16, 4))
        _check_tensor("b_scale", b_scale, dev, (torch.uint8,), (n, 16, 4))
    out = torch.empty(n, 16, 16, dtype=torch.float32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _load().mega_moe_diag_mfma_block_sums(int(fmt), _ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale),
                                               _ptr(out), int(n), ctypes.c_void_p(handle))
    if st:
        raise MegaMoEError(st, "mega_moe_diag_mfma_block_sums")
    return out


class MegaMoE:
    """Owns a workspace for repeated forwards of one problem shape on one device."""

    def __init__(self, problem: Problem, device="cuda"):
        import torch
        self.problem = problem
        self.device = torch.device(device)
        self.workspace = torch.empty(max(1, mega_moe_workspace_size(problem)), dtype=torch.uint8,
                                     device=self.device)

    def __call__(self, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y=None, stream=None):
        import torch
        if y is None:
            y = torch.empty(self.problem.num_tokens, self.problem.hidden, dtype=torch.bfloat16,
                            device=self.device)
        mega_moe_forward(self.problem, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y,
                         self.workspace, stream)
        return y

    def views(self):
        return mega_moe_workspace_views(self.problem, self.workspace)
