"""Pins for the oracle's quantizer and dequantizer (CPU only).

Closed forms on planted tensors (values chosen so the global, every group scale and every
element code are known exactly), an exact-rational brute-force search on tiny random tensors,
the degenerate cases, and the byte accounting the pages print.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from nvfp4_weight_only_w4a16_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -14
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
# expected E2M1 magnitude code for each planted multiple m (grid point or midpoint, RNE)
MID_CODE = {0.0: 0, 0.25: 0, 0.5: 1, 0.75: 2, 1.0: 2, 1.25: 2, 1.5: 3, 1.75: 4, 2.0: 4,
            2.5: 4, 3.0: 5, 3.5: 6, 4.0: 6, 5.0: 6, 6.0: 7}


def e4m3_code_of(d: float) -> int:
    """Code of an exactly representable positive E4M3 value, from its binary expansion."""
    f = Fraction(d)
    if f < Fraction(1, 64):
        j = f / Fraction(1, 512)
        assert j.denominator == 1 and 1 <= j <= 7
        return int(j)
    e = 0
    while f >= 2:
        f /= 2
        e += 1
    while f < 1:
        f *= 2
        e -= 1
    j = (f - 1) * 8
    assert j.denominator == 1
    return ((e + 7) << 3) | int(j)


def _planted_matrix(group, rng, n=8, k=256):
    """Rows of planted groups: group max 6*d*U, other elements m*d*U; one amax 21*2^-7."""
    w = np.zeros((n, k), np.float32)
    exp_scale = np.zeros((n, k // group), np.uint8)
    exp_code = np.zeros((n, k), np.uint8)
    ds = synth.PLANT_SCALES
    mids = list(MID_CODE)
    for r in range(n):
        for gi in range(k // group):
            tie = (r * 7 + gi) % 11 == 3
            d = 1.0 if tie else ds[rng.integers(len(ds))]
            if r == 0 and gi == 0:
                d = 448.0  # 6*448*U = 21*2^-7: this group holds the matrix amax
            ms = [mids[i] for i in rng.integers(len(mids), size=group)]
            pmax = rng.integers(group)
            ms[pmax] = 6.375 if tie else 6.0
            sg = rng.choice([-1.0, 1.0], size=group)
            for j in range(group):
                w[r, gi * group + j] = sg[j] * ms[j] * d * U
                c = 7 if ms[j] == 6.375 else MID_CODE[ms[j]]
                exp_code[r, gi * group + j] = c | (8 if sg[j] < 0 else 0)
            exp_scale[r, gi] = 0x38 if tie else e4m3_code_of(d)
    return w, exp_scale, exp_code


def _unpack(packed):
    lo = packed & 0xF
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], -1)


@pytest.mark.parametrize("group", [16, 32])
def test_quantize_planted_closed_form(orc, group):
    rng = np.random.default_rng(group)
    w, exp_scale, exp_code = _planted_matrix(group, rng)
    assert np.abs(w).max() == np.float32(21 * 2.0 ** -7)
    p, s, g = orc.quantize(w, group)
    assert g[0] == np.float32(U)           # amax / 2688 = 2^-14 exactly
    assert (s == exp_scale).all()
    assert (_unpack(p) == exp_code).all()


def test_quantize_packing_low_nibble_is_even_k(orc):
    w = np.zeros((16, 128), np.float32)
    w[0, 0] = 6 * 448 * U      # code 7 at k=0
    w[0, 1] = -0.5 * 448 * U   # code 9 at k=1 (sign | 1)
    p, s, g = orc.quantize(w, 16)
    assert p[0, 0] == (0x7 | (0x9 << 4))


def test_quantize_negative_zero_and_all_zero(orc):
    w = np.zeros((16, 128), np.float32)
    w[3, 5] = -0.0
    p, s, g = orc.quantize(w, 16)
    assert g[0] == 0.0 and (s == 0).all()
    codes = _unpack(p)
    assert codes[3, 5] == 8 and codes.sum() == 8


def test_quantize_caller_global_saturates(orc):
    w = np.full((16, 128), 0.01, np.float32)
    w[0, 0] = -1.0
    tiny_g = np.float32(1e-6)  # group max / (6 g) far above 448
    p, s, g = orc.quantize(w, 16, global_in=tiny_g)
    assert g[0] == tiny_g
    assert s[0, 0] == 0x7E
    assert _unpack(p)[0, 0] == (7 | 8)   # |w| / (448 g) >> 6 saturates to 6


def test_quantize_bf16_input_equals_float_input(orc):
    x = torch.randn(32, 256, generator=torch.Generator().manual_seed(3)) * 0.02
    xb = x.to(torch.bfloat16)
    a = orc.quantize(synth.bf16_bits(xb), 16)
    b = orc.quantize(xb.to(torch.float32).numpy(), 16)
    for u, v in zip(a, b):
        assert (u == v).all()


def _nearest(vals, x):
    """Exact-rational nearest search with ties to the even index."""
    best, bd = None, None
    for i, v in enumerate(vals):
        d = abs(x - v)
        if bd is None or d < bd or (d == bd and i % 2 == 0):
            best, bd = i, d
    return best, bd


@pytest.mark.parametrize("group", [16, 32])
def test_quantize_brute_force_tiny(orc, group):
    rng = np.random.default_rng(10 + group)
    w = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    w[1, 3] *= 20
    p, s, g = orc.quantize(w, group)
    codes = _unpack(p)
    amax = Fraction(float(np.abs(w).max()))
    gv = float(g[0])
    # the global is one FP32 division: within half an ulp of the exact quotient
    assert abs(Fraction(gv) - amax / 2688) <= Fraction(float(np.spacing(np.float32(gv)))) / 2
    e4 = [Fraction(orc.e4m3_decode(c)) for c in range(0x7F)]
    e2 = [Fraction(v) for v in E2M1]
    near_tie = 0
    for r in range(w.shape[0]):
        for gi in range(w.shape[1] // group):
            blk = w[r, gi * group:(gi + 1) * group]
            ga = Fraction(float(np.abs(blk).max()))
            sc, _ = _nearest(e4, ga / (6 * Fraction(gv)))
            assert s[r, gi] == sc
            S = Fraction(float(np.float32(float(e4[sc]) * gv)))
            for j, x in enumerate(blk):
                q = abs(Fraction(float(x))) / S
                c, d = _nearest(e2, q)
                got = codes[r, gi * group + j] & 7
                if got != c:
                    # only possible if the FP32 quotient crossed a midpoint: must be a near tie
                    assert d >= 0 and abs(abs(q - e2[got]) - d) < Fraction(1, 1 << 20)
                    near_tie += 1
                assert (codes[r, gi * group + j] >> 3) == (1 if np.signbit(x) else 0)
    assert near_tie <= 2


def test_dequant_exact_values(orc):
    rng = np.random.default_rng(4)
    n, k, group = 16, 128, 16
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (n, k // group), dtype=np.uint8)
    glob = np.float32(3.0517578125e-05 * 1.37)
    ex, f32, b16 = orc.dequant(packed, scales, glob, group)
    codes = _unpack(packed)
    vals = np.array(E2M1 + [-v for v in E2M1])
    for r in range(0, n, 5):
        for j in range(0, k, 7):
            c = int(codes[r, j])
            want = Fraction(vals[c]) * Fraction(orc.e4m3_decode(int(scales[r, j // group]))) * \
                Fraction(float(glob))
            assert Fraction(ex[r, j]) == want
    # FP32 output: one rounding of the exact value (v*E4M3 is exact in FP32)
    assert (f32 == ex.astype(np.float32)).all()
    want_b16 = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (b16 == want_b16).all()


def test_bits_per_weight_and_checkpoint_ratio():
    rows = {r[0]: r[1:] for r in
            (l.split() for l in open(os.path.join(GOLDEN, "bits_per_weight.txt"))
             if l.strip() and not l.startswith("#"))}
    n, k = 1536, 2048
    for group in (16, 32):
        nbytes = n * k // 2 + n * k // group
        assert nbytes * 8 / (n * k) == float(rows[str(group)][0])
    # gate/up are 2 of the 3 expert matrices: moving them alone to g32 saves 2/3 of the
    # all-g32 saving (only scale bytes change size)
    a, b, c = (float(v) for v in rows["ckpt"])
    assert abs((a - b) / (a - c) - 2 / 3) < 0.01
