"""NF4 (4-bit NormalFloat) codebook, quantiser and dequantiser -- oracle side.

The pages name NF4 as the four-bit format associated with QLoRA and say it cuts
the host-side frozen store to about a quarter of the bf16 size (page "Can You
Fine-Tune Llama 3.1 8B on a 4GB GPU? Soup's Layer Streaming Explained",
section "Why NF4 matters so much").  They print neither the levels nor the
block layout, so this module takes these readings:

codebook
    QLoRA's NormalFloat construction.  With delta = 1/2 (1/30 + 1/32) and
    p_hi = 1 - delta, the 8 positive levels are Phi^-1 of 9 equally spaced
    probabilities from p_hi down to 1/2 with the last (zero) dropped, the 7
    negative levels are minus Phi^-1 of 8 equally spaced probabilities from
    p_hi down to 1/2 with the last dropped, plus an exact 0.  Everything is
    divided by Phi^-1(p_hi) so the ends are exactly -1 and +1.  Derived in
    float64 with ``statistics.NormalDist`` and rounded once to float32.
blocks
    The weight [out, in] is flattened row-major; block b covers flat elements
    [64 b, 64 b + 64).  Blocks may straddle rows.
quantise
    a = max |w| over the block (float32).  a = 0 gives code 7 (the 0.0 level)
    for every element and absmax 0.  Otherwise n = w / a (float32 division) and
    the code is argmin_j |n - cb[j]| with the subtraction and the comparison in
    float32 and ties going to the lower index.  Element 2k goes to the high
    nibble of byte k, element 2k + 1 to the low nibble.
dequantise
    w32 = float32(cb[c] * a) (one float32 multiply), then bf16 round to nearest
    even.
double quantisation (the store of 112.5 MB per 8B layer)
    The pages' pinned store is 3.60 GB for 32 layers and the device buffers
    113 MB each (page "Fine tune an 8B model on a 4GB laptop GPU (Soup
    setup)", section "Step 2, train"), which is NF4 codes plus 8-bit absmax
    scales, QLoRA's double quantisation; the pages give no format, so the
    plainest one is taken: each weight's float32 absmax array is cut into
    groups of 256 consecutive entries (the last may be shorter); per group
    s = float32(max(a) / 255) and q = clamp(rint(float32(a / s)), 0, 255)
    (round half to even; s = 0 gives q = 0); the decoded absmax is
    float32(float32(q) * s).  Codes are chosen with the exact absmax first.
"""
from __future__ import annotations

from statistics import NormalDist

import numpy as np

BLOCK = 64
ZERO_CODE = 7


def codebook() -> np.ndarray:
    """The 16 NF4 levels, float32, ascending."""
    nd = NormalDist()
    delta = 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    p_hi = 1.0 - delta
    pos = [nd.inv_cdf(p_hi - i * (p_hi - 0.5) / 8.0) for i in range(8)]
    neg = [-nd.inv_cdf(p_hi - i * (p_hi - 0.5) / 7.0) for i in range(7)]
    top = nd.inv_cdf(p_hi)
    vals = sorted([v / top for v in pos] + [v / top for v in neg] + [0.0])
    return np.asarray(vals, dtype=np.float64).astype(np.float32)


def bf16_bits_rne(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even; NaN kept quiet."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x32, dtype=np.float32))
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize(w: np.ndarray, chunk_blocks: int = 1 << 16):
    """float32 weight (any shape, numel % 64 == 0) -> (codes uint8 [n/2], absmax float32 [n/64])."""
    flat = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    n = flat.size
    if n % BLOCK:
        raise ValueError("numel must be a multiple of 64")
    cb = codebook()
    nb = n // BLOCK
    blocks = flat.reshape(nb, BLOCK)
    absmax = np.max(np.abs(blocks), axis=1).astype(np.float32)
    codes = np.empty(n, dtype=np.uint8)
    for s in range(0, nb, chunk_blocks):
        e = min(nb, s + chunk_blocks)
        a = absmax[s:e]
        safe = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
        nrm = (blocks[s:e] / safe[:, None]).astype(np.float32)
        dist = np.abs(nrm[:, :, None] - cb[None, None, :])     # float32
        idx = np.argmin(dist, axis=2).astype(np.uint8)         # first minimum
        idx[a == 0] = ZERO_CODE
        codes[s * BLOCK:e * BLOCK] = idx.reshape(-1)
    packed = ((codes[0::2] << 4) | codes[1::2]).astype(np.uint8)
    return packed, absmax


def unpack(codes: np.ndarray) -> np.ndarray:
    """packed uint8 [n/2] -> code per element uint8 [n]."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.size * 2, dtype=np.uint8)
    out[0::2] = c >> 4
    out[1::2] = c & 0xF
    return out


def dequant_f32(codes: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """float32 cb[c] * absmax, flat."""
    cb = codebook()
    idx = unpack(codes)
    a = np.repeat(np.asarray(absmax, dtype=np.float32), BLOCK)
    return (cb[idx] * a).astype(np.float32)


def dequant_bits(codes: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of the dequantised weight, flat."""
    return bf16_bits_rne(dequant_f32(codes, absmax))


def dequant(codes: np.ndarray, absmax: np.ndarray, shape) -> np.ndarray:
    """bf16-valued float32 array of the dequantised weight in ``shape``."""
    return bf16_bits_to_f32(dequant_bits(codes, absmax)).reshape(shape)


# ---------------------------------------------------------------- double quantisation
DQ_GROUP = 256


def double_quant(absmax: np.ndarray):
    """Second-level quantisation of one weight's absmax array.

    Returns (q8 uint8 [nb], scales float32 [ceil(nb / 256)]).
    """
    a = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    nb = a.size
    ng = -(-nb // DQ_GROUP)
    g = np.zeros(ng * DQ_GROUP, np.float32)
    g[:nb] = a
    g = g.reshape(ng, DQ_GROUP)
    c = g.max(axis=1)
    s = (c / np.float32(255.0)).astype(np.float32)
    x = np.zeros_like(g)
    nz = s > 0
    x[nz] = (g[nz] / s[nz, None]).astype(np.float32)
    q = np.clip(np.rint(x), 0, 255).astype(np.uint8).reshape(-1)[:nb]
    return q, s


def dq_absmax(q8: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decoded absmax: float32(float32(q) * s_group)."""
    q = np.asarray(q8, dtype=np.uint8).reshape(-1).astype(np.float32)
    s = np.asarray(scales, dtype=np.float32).reshape(-1)
    return (q * s[np.arange(q.size) // DQ_GROUP]).astype(np.float32)


def dequant_dq(codes: np.ndarray, q8: np.ndarray, scales: np.ndarray, shape) -> np.ndarray:
    """Dequantise NF4 codes with double-quantised absmax (bf16 values as float32)."""
    return dequant(codes, dq_absmax(q8, scales), shape)
