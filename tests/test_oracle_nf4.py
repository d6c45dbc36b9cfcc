"""Pins for the oracle's NF4 codebook, quantiser and dequantiser (CPU only).

The pages describe NF4 only as QLoRA's four-bit format that shrinks the frozen
store to about a quarter of bf16 (page "Can You Fine-Tune Llama 3.1 8B on a 4GB
GPU? ...", section "Why NF4 matters so much"); each check below pins the
oracle to mathematics or to an independent library routine instead.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy import special

from oracle import nf4


def test_codebook_shape_and_ends():
    cb = nf4.codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert np.all(np.diff(cb) > 0)
    assert cb[0] == -1.0 and cb[15] == 1.0 and cb[7] == 0.0
    assert np.sum(cb < 0) == 7 and np.sum(cb > 0) == 8


def test_codebook_levels_are_normal_quantiles():
    """Phi(level * Phi^-1(p_hi)) must land on the equally spaced probabilities
    of the NormalFloat construction; checked with scipy's ndtr/ndtri, an
    implementation independent of statistics.NormalDist."""
    cb = nf4.codebook().astype(np.float64)
    p_hi = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    c = special.ndtri(p_hi)
    for i in range(8):                          # positive levels, ascending
        want = 0.5 + (i + 1) * (p_hi - 0.5) / 8.0
        assert abs(special.ndtr(cb[8 + i] * c) - want) < 5e-7
    for j in range(7):                          # negative levels, ascending
        want = p_hi - j * (p_hi - 0.5) / 7.0
        assert abs(special.ndtr(-cb[j] * c) - want) < 5e-7


def _bf16_by_hand(f32: np.float32) -> int:
    """Round a float32 to bf16 bits by exact rational comparison (ties to even)."""
    bits = int(np.float32(f32).view(np.uint32))
    if np.isnan(f32):
        return None
    lo = bits & 0xFFFF0000
    if bits == lo:
        return lo >> 16
    hi = lo + 0x10000
    flo = Fraction(float(np.uint32(lo).view(np.float32)))
    hi32 = np.uint32(hi & 0xFFFFFFFF).view(np.float32)
    f = Fraction(float(f32))
    if np.isinf(hi32):        # rounding up overflows: compare with the halfway point
        top = Fraction(2) ** 128
        fhi = top if f > 0 else -top
    else:
        fhi = Fraction(float(hi32))
    dlo, dhi = abs(f - flo), abs(f - fhi)
    if dlo < dhi:
        return lo >> 16
    if dhi < dlo:
        return (hi >> 16) & 0xFFFF
    return (lo >> 16) if ((lo >> 16) & 1) == 0 else ((hi >> 16) & 0xFFFF)


def test_bf16_rounding_matches_torch_and_exact():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),     # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 1.0, 3.4e38, -3.4e38], np.float32),
        # exact ties: low 16 bits == 0x8000, with even and odd kept mantissa
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00018000], np.uint32).view(np.float32),
    ])
    ours = nf4.bf16_bits_rne(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    for v in x[::37]:
        assert int(nf4.bf16_bits_rne(np.array([v]))[0]) == _bf16_by_hand(v)
    nan = nf4.bf16_bits_rne(np.array([np.nan], np.float32))
    assert np.isnan(nf4.bf16_bits_to_f32(nan))[0]


def test_dequant_exact_product_then_bf16():
    """Every code x random absmax: float32(cb*a) computed exactly in float64
    (24+24 bit mantissas fit in 53) and rounded by numpy's IEEE cast, then
    bf16-rounded by exact rational comparison."""
    cb = nf4.codebook()
    rng = np.random.default_rng(1)
    absmax = np.concatenate([
        np.abs(rng.standard_normal(300)).astype(np.float32) * np.float32(0.08),
        np.array([1.0, 0.5, 2.0 ** -20, 3.0e-39, 1e30, 0.0], np.float32),
        rng.uniform(0, 1, 100).astype(np.float32),
    ])
    codes = np.arange(16, dtype=np.uint8)
    packed = ((codes[0::2] << 4) | codes[1::2]).astype(np.uint8)
    for a in absmax:
        packed_blk = np.tile(packed, 4)                       # one 64-element block
        got = nf4.dequant_bits(packed_blk, np.array([a], np.float32))
        for i in range(64):
            c = i % 16
            exact = float(cb[c]) * float(a)                   # exact in float64
            f32 = np.float32(exact)                           # IEEE RNE cast
            assert int(got[i]) == _bf16_by_hand(f32), (c, a)


def test_nibble_order_high_first():
    w = np.zeros(64, np.float32)
    w[0], w[1] = 1.0, -1.0          # element 0 -> code 15, element 1 -> code 0
    codes, absmax = nf4.quantize(w)
    assert absmax[0] == 1.0
    assert codes[0] == (15 << 4) | 0
    assert np.all(codes[1:] == (7 << 4) | 7)


def _check_optimal(w, codes, absmax):
    cb = [Fraction(float(v)) for v in nf4.codebook()]
    idx = nf4.unpack(codes)
    for b in range(w.size // 64):
        a = float(absmax[b])
        blk = w[64 * b:64 * b + 64]
        assert a == float(np.max(np.abs(blk)))
        if a == 0.0:
            assert np.all(idx[64 * b:64 * b + 64] == 7)
            continue
        for e in range(64):
            n = Fraction(float(blk[e])) / Fraction(a)
            c = int(idx[64 * b + e])
            best = min(abs(n - q) for q in cb)
            # the float32 decision may differ from exact only within float32 rounding
            assert abs(n - cb[c]) <= best + Fraction(1, 1 << 22), (b, e)
            if abs(float(blk[e])) == a:
                assert c == (15 if blk[e] > 0 else 0)


@pytest.mark.parametrize("seed,shape,kind", [(1, (4, 64), "normal"), (2, (8, 688), "normal"),
                                             (3, (2, 96), "uniform"), (4, (2, 128), "with_zero_block")])
def test_quantize_brute_force(seed, shape, kind):
    """Blocks straddle rows for the 688- and 96-wide cases."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        w = rng.standard_normal(shape).astype(np.float32) * np.float32(0.02)
    elif kind == "uniform":
        w = rng.uniform(-1, 1, shape).astype(np.float32)
    else:
        w = rng.standard_normal(shape).astype(np.float32)
        w.reshape(-1)[64:128] = 0.0
        w.reshape(-1)[5] = -np.max(np.abs(w))               # absmax on a negative element
    if w.size % 64:
        pytest.skip("numel not a multiple of 64")
    codes, absmax = nf4.quantize(w)
    _check_optimal(w.reshape(-1), codes, absmax)


def test_quantize_ties_go_low():
    """An element exactly halfway between two levels (in float32) takes the lower index."""
    cb = nf4.codebook()
    w = np.zeros(64, np.float32)
    w[0] = 1.0
    mid = np.float32((np.float64(cb[9]) + np.float64(cb[10])) / 2)
    d_lo = abs(np.float32(mid - cb[9]))
    d_hi = abs(np.float32(mid - cb[10]))
    w[1] = mid
    codes, _ = nf4.quantize(w)
    c = nf4.unpack(codes)[1]
    assert c == (9 if d_lo <= d_hi else 10)


def test_quantize_dequant_idempotent():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((64, 192)).astype(np.float32) * np.float32(0.02)
    codes, absmax = nf4.quantize(w)
    w2 = nf4.dequant_f32(codes, absmax)
    codes2, absmax2 = nf4.quantize(w2)
    assert np.array_equal(codes, codes2) and np.array_equal(absmax, absmax2)


def test_quantize_rejects_ragged():
    with pytest.raises(ValueError):
        nf4.quantize(np.zeros(65, np.float32))


# ---------------------------------------------------------------- double quantisation
def _absmax_like(seed, nb):
    rng = np.random.default_rng(seed)
    return np.abs(rng.normal(0, 0.02, (nb, 64))).max(axis=1).astype(np.float32)


@pytest.mark.parametrize("nb", [256, 1000, 1])
def test_dq_code_is_exact_nearest_multiple(nb):
    """Each 8-bit code is an integer j in [0, 255] nearest to a / s in exact
    rational arithmetic (ties either way); the group maximum maps to 255."""
    a = _absmax_like(3, nb)
    q, s = nf4.double_quant(a)
    assert q.dtype == np.uint8 and q.shape == (nb,) and s.shape == (-(-nb // 256),)
    for i in range(0, nb, max(1, nb // 200)):
        sg = Fraction(float(s[i // 256]))
        x = Fraction(float(a[i])) / sg
        assert abs(Fraction(int(q[i])) - x) <= Fraction(1, 2) + Fraction(1, 10**6), (i, q[i], float(x))
    for gi in range(len(s)):
        grp = a[gi * 256:(gi + 1) * 256]
        assert q[gi * 256 + int(np.argmax(grp))] == 255
        assert s[gi] == np.float32(np.float32(grp.max()) / np.float32(255))


def test_dq_decoded_error_bound():
    """|a_hat - a| <= s/2 (plus float32 rounding of the product): the linear
    8-bit grid of the group max, exactly."""
    a = _absmax_like(4, 4096)
    q, s = nf4.double_quant(a)
    ah = nf4.dq_absmax(q, s)
    sg = s[np.arange(a.size) // 256].astype(np.float64)
    err = np.abs(ah.astype(np.float64) - a.astype(np.float64))
    assert np.all(err <= 0.5 * sg * (1 + 1e-6) + np.spacing(a.astype(np.float32)).astype(np.float64))
    # the decoded value is exactly the float32 product q * s
    want = np.array([Fraction(int(qi)) * Fraction(float(si)) for qi, si in zip(q[:64], sg[:64])])
    assert all(np.float32(float(w)) == h for w, h in zip(want, ah[:64]))


def test_dq_zero_group_and_short_tail():
    a = np.concatenate([np.zeros(256, np.float32), _absmax_like(5, 100)])
    q, s = nf4.double_quant(a)
    assert s[0] == 0 and not np.any(q[:256]) and not np.any(nf4.dq_absmax(q, s)[:256])
    assert s.shape == (2,) and q[256 + int(np.argmax(a[256:]))] == 255


def test_dq_store_size_matches_the_pages():
    """8B-shaped record with 8-bit absmax + one float32 scale per 256 blocks:
    codes + absmax codes + scales + two bf16 norms (256-byte aligned regions)
    must come to the pages' 3.60 GB / 32 = 112.5 MB per layer (within the
    rounding of the printed 3.60), where float32 absmax gives 122.7 MB."""
    d, I, qd, kvd = 4096, 14336, 4096, 1024
    numel = [qd * d, kvd * d, kvd * d, d * qd, I * d, I * d, d * I]
    al = lambda n: -(-n // 256) * 256
    codes = sum(al(n // 2) for n in numel)
    dq = sum(al(n // 64) for n in numel) + sum(al(4 * (-(-(n // 64) // 256))) for n in numel)
    norms = 2 * al(2 * d)
    f32 = codes + sum(al(n // 64 * 4) for n in numel) + norms
    rec = codes + dq + norms
    assert abs(rec * 32 / 3.60e9 - 1) < 0.0014, rec
    assert abs(f32 - 122_699_776) < 4096
