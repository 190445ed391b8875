"""Number formats of the MegaMoE expert layer, written out from their bit definitions.

TEST INFRASTRUCTURE ONLY.  This package is the CPU oracle that the GPU path is
checked against; only tests, the smoke check and the CPU-baseline leg of the
benchmark may import it.  Nothing here is shared with the HIP kernels.

Formats (all decoded to float64, which holds every one of them exactly):

* E4M3FN (OCP FP8): ``s eeee mmm``, exponent bias 7, no infinities, only
  ``0x7F``/``0xFF`` are NaN, largest finite magnitude 448.  The SM90 design page
  ("MegaMoE SM90 Implementation Design", section 1.1 decision 7 and section 10.1)
  quantises activations and the SwiGLU output to this format with a float scale
  equal to amax/448.
* E2M1 (OCP FP4): ``s ee m``, bias 1, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; the
  MXFP4 weights of the FP8 x MXFP4 pull request page (PR #411 description) and the
  SM100 FP8 x FP4 baseline of the research report (section 3.1).
* UE8M0: an unsigned power-of-two scale ``2^(code-127)``, code 255 is NaN; the
  PR #411 review (processed-MXFP4 contract) restores exactly this value per
  32-element K group.
* BF16: the top 16 bits of an IEEE binary32, round-to-nearest-even; the layer's
  output type (design page section 11.1, L2 BF16 epilogue).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def e4m3_decode_table() -> np.ndarray:
    """All 256 E4M3FN codes as float64 (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            out[code] = np.nan
        elif exp == 0:
            out[code] = sign * man * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        else:
            out[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return out


_E4M3 = e4m3_decode_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_rne(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest E4M3FN code, ties to even mantissa.

    Magnitudes above 448 saturate to 448 (the method clamps to +-448 before
    converting, so this branch only matters for direct callers).  The input is
    treated exactly (float32 inputs are exact in float64).
    """
    v = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    code = np.zeros(mag.shape, dtype=np.int64)
    sub = mag < 2.0 ** -6
    # subnormal grid: multiples of 2^-9; a result of 8 is the smallest normal, code 0x08
    code[sub] = np.rint(mag[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        m, e = np.frexp(mag[nrm])            # mag = m * 2^e with m in [0.5, 1)
        e = e - 1                            # mag = (2m) * 2^e, 2m in [1, 2)
        q = np.rint((2.0 * m - 1.0) * 8.0).astype(np.int64)   # 3-bit mantissa, RNE
        carry = q == 8
        e = e + carry
        q = np.where(carry, 0, q)
        code[nrm] = ((e + 7) << 3) | q
    code = np.minimum(code, 0x7E)            # 0x7E == 448
    sign = np.signbit(v).astype(np.int64) << 7   # a negative value that rounds to 0 keeps its sign
    return (code | sign).astype(np.uint8)


def e2m1_decode_table() -> np.ndarray:
    out = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        exp = (code >> 1) & 0x3
        man = code & 0x1
        out[code] = sign * (man * 0.5 if exp == 0 else (1.0 + man / 2.0) * 2.0 ** (exp - 1))
    return out


_E2M1 = e2m1_decode_table()


def e2m1_unpack_decode(packed: np.ndarray) -> np.ndarray:
    """Decode packed E2M1 bytes [..., K/2] into float64 [..., K].

    The low nibble of byte i holds element 2i and the high nibble element 2i+1
    (OCP MX packing; the pages fix no order, see the readings in the design notes).
    """
    p = np.asarray(packed, dtype=np.uint8)
    lo = _E2M1[p & 0xF]
    hi = _E2M1[p >> 4]
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def ue8m0_decode(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127).astype(np.float64)
    return np.where(c == 255, np.nan, out)


def ue8m0_code_for_amax(amax32: np.ndarray, fmt_max: float) -> np.ndarray:
    """Smallest power-of-two scale 2^E with amax/2^E <= fmt_max, as a UE8M0 code.

    r = float32(amax / fmt_max) by one float32 division; E = ceil(log2 r) taken
    exactly from the binary exponent of r; code = clamp(E + 127, 0, 254).  An
    all-zero group (amax == 0) gets code 0.
    """
    a = np.asarray(amax32, dtype=np.float32)
    r = (a / np.float32(fmt_max)).astype(np.float32)
    m, e = np.frexp(r.astype(np.float64))   # r = m * 2^e, m in [0.5, 1)
    ceil_log2 = np.where(m == 0.5, e - 1, e)
    code = np.clip(ceil_log2 + 127, 0, 254)
    return np.where(a > 0, code, 0).astype(np.uint8)


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16), round to nearest even; NaN stays NaN."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(f)
    r = np.where(nan, (u >> 16).astype(np.uint32) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32)
