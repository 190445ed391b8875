"""The matrix core's 128-K block sum against the exact sum of its products (on an MI355X).

The L1 and L2 GEMMs sum each 128-long K block of FP8 (or FP4 x FP8) products in one 16x16x128
scaled MFMA.  The oracle forms the same block sums exactly (every product and every block sum of
these formats is exact in float64), so the intermediate codes of the two sides can only differ
through the hardware's summation error.  This test measures that error through the library's
diagnostic entry point (same instruction, operand layout and scale encoding as the GEMMs) on
seeded operands of several kinds and asserts the bound the intermediate tolerance is derived
from: |block_sum_hw - exact| <= EPS_MFMA * sum_k |a_k b_k| (scales included).
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import dispatch_fp8_grouped_topk_amd as mm
import oracle
from harness import EPS_MFMA

pytestmark = pytest.mark.gpu

N_TILES = 2048
_E4M3 = oracle.e4m3_decode_table()
_E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], dtype=np.float64)


def _say(msg):
    print(f"[mfma-error] {msg}", flush=True)
    sys.stdout.flush()


def _finite_e4m3_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, np.uint8(0x7E), c).astype(np.uint8)   # no NaN


def _normal_codes(rng, shape, scale=1.0):
    """E4M3 codes of N(0, 1) rows scaled so each 128-row's amax maps to 448 (the input recipe)."""
    v = rng.standard_normal(shape) * scale
    amax = np.abs(v).max(axis=-1, keepdims=True)
    t = torch.from_numpy((v / amax * 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _cancelling(rng, shape):
    """Rows whose products cancel: each K half is the other's negation (sign bit flipped), so the
    exact block sum is 0 while the magnitudes are large."""
    a = _normal_codes(rng, shape)
    a[..., 64:] = a[..., :64] ^ 0x80
    return a


def _exact(fmt, a, b, sa=None, sb=None):
    """Exact float64 block sums and magnitude sums, [n, 16, 16]."""
    if fmt == 1:
        lo, hi = a & 0xF, a >> 4
        av = np.empty(a.shape[:-1] + (128,))
        av[..., 0::2], av[..., 1::2] = _E2M1[lo], _E2M1[hi]
    else:
        av = _E4M3[a]
    bv = _E4M3[b]
    if fmt != 0:
        av = av * np.repeat(np.ldexp(1.0, sa.astype(np.int64) - 127), 32, axis=-1)
        bv = bv * np.repeat(np.ldexp(1.0, sb.astype(np.int64) - 127), 32, axis=-1)
    exact = np.einsum("tmk,tnk->tmn", av, bv)
    mag = np.einsum("tmk,tnk->tmn", np.abs(av), np.abs(bv))
    return exact, mag


def _hw(fmt, a, b, sa=None, sb=None):
    dev = torch.device("cuda")
    t = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    out = mm.mega_moe_diag_mfma_block_sums(fmt, t(a), t(b), t(sa), t(sb))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


CASES = {
    # fmt 0: the float-scale recipe's MFMA (unit scales, promoted outside)
    "fp8_all_codes": (0, "codes"),
    "fp8_normal": (0, "normal"),
    "fp8_cancelling": (0, "cancel"),
    # fmt 1: E2M1 weights x E4M3 activations with UE8M0 scales per 32
    "fp4_x_fp8_normal": (1, "normal"),
    # fmt 2: E4M3 x E4M3 with UE8M0 scales per 32
    "fp8_ue8m0_normal": (2, "normal"),
    "fp8_ue8m0_cancelling": (2, "cancel"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_block_sum_error_bound(name):
    fmt, kind = CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    shape = (N_TILES, 16, 128)
    if kind == "codes":
        a, b = _finite_e4m3_codes(rng, shape), _finite_e4m3_codes(rng, shape)
    elif kind == "cancel":
        a, b = _cancelling(rng, shape), _normal_codes(rng, shape)
    else:
        a, b = _normal_codes(rng, shape), _normal_codes(rng, shape)
    sa = sb = None
    if fmt == 1:
        a = rng.integers(0, 256, size=(N_TILES, 16, 64), dtype=np.uint8)
    if fmt != 0:
        sa = rng.integers(117, 137, size=(N_TILES, 16, 4), dtype=np.uint8)
        sb = rng.integers(117, 137, size=(N_TILES, 16, 4), dtype=np.uint8)
    exact, mag = _exact(fmt, a, b, sa, sb)
    hw = _hw(fmt, a, b, sa, sb)
    assert np.isfinite(hw).all()
    rel = np.abs(hw - exact) / np.maximum(mag, 1e-300)
    rel[mag == 0] = np.abs(hw - exact)[mag == 0]
    _say(f"{name}: max |err| / sum|products| = {rel.max():.3e} (2^{np.log2(max(rel.max(), 1e-300)):.2f}), "
         f"mean {rel.mean():.3e}, exact sums {float((hw == exact).mean()):.3f}")
    assert rel.max() <= EPS_MFMA, f"{name}: block-sum error {rel.max():.3e} above {EPS_MFMA:.3e}"


def test_exact_when_products_share_one_binade():
    """Products that are all one power of two (codes 1.0 x 1.0) sum exactly: a check that the
    instruction, the operand layout and the output placement are the ones the test assumes."""
    rng = np.random.default_rng(7)
    a = np.full((64, 16, 128), 0x38, dtype=np.uint8)            # 1.0
    b = np.where(rng.random((64, 16, 128)) < 0.5, 0x38, 0xB8).astype(np.uint8)   # +-1.0
    a[:, 3, :] = 0x40                                           # row 3: 2.0
    exact, _ = _exact(0, a, b)
    hw = _hw(0, a, b)
    assert np.array_equal(hw, exact)
