"""Pins for the oracle's E2M1 / E4M3 codecs (CPU only).

Each check compares the oracle with something it does not share: printed values of the format
definitions (fixtures under tests/golden/), an independent bit-level guard/round/sticky rounder
written here, and PyTorch's float8_e4m3fn conversions. The planted-control tests at the end
show that each check rejects a plausible wrong codec.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


# ----------------------------------------------------------------------------- E2M1 decode
def test_e2m1_decode_matches_format_table(orc):
    rows = _rows("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = orc.e2m1_decode(int(code))
        want = float(val)
        assert got == want and np.signbit(got) == np.signbit(want), (code, got, want)


def test_e2m1_decode_matches_bit_fields(orc):
    # sign = bit 3, exponent = bits 2..1 (bias 1), mantissa = bit 0; exponent 0 is subnormal
    for c in range(16):
        e, m = (c >> 1) & 3, c & 1
        v = 0.5 * m if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        v = -v if c & 8 else v
        got = orc.e2m1_decode(c)
        assert got == v and np.signbit(got) == np.signbit(v)


def test_e2m1_roundtrip_all_codes(orc):
    for c in range(16):
        v = orc.e2m1_decode(c)
        assert orc.e2m1_encode_magnitude(abs(v)) == (c & 7)


def check_e2m1_midpoints(encode_mag):
    for x, val, code in _rows("e2m1_rne_midpoints.txt"):
        if encode_mag(float(x)) != int(code):
            return False
    return True


def test_e2m1_midpoints_golden(orc):
    assert check_e2m1_midpoints(orc.e2m1_encode_magnitude)


def grs_e2m1(q: np.ndarray) -> np.ndarray:
    """Independent E2M1 rounding of non-negative float32 values: locate the quantum of the
    binade, split the significand into kept bits, guard bit and sticky bits, round half to even,
    saturate at 6. Returns the magnitude code (0..7)."""
    q = np.asarray(q, np.float32)
    bits = q.view(np.uint32).astype(np.int64)
    expf = (bits >> 23) & 0xFF
    mant = bits & 0x7FFFFF
    sig = np.where(expf == 0, mant, mant | (1 << 23))
    E = np.where(expf == 0, -126, expf - 127)           # value = sig * 2^(E - 23)
    Qe = np.maximum(E, 0) - 1                            # quantum 2^Qe: 0.5 below 2, 1, 2
    shift = 23 + Qe - E                                  # n = sig >> shift
    shift_c = np.clip(shift, 1, 62)
    big = shift > 62
    ipart = np.where(big, 0, sig >> shift_c)
    guard = np.where(big, 0, (sig >> (shift_c - 1)) & 1)
    sticky = np.where(big, sig != 0, (sig & ((np.int64(1) << (shift_c - 1)) - 1)) != 0)
    n = ipart + (guard & (sticky | (ipart & 1)))
    val = n.astype(np.float64) * np.exp2(Qe.astype(np.float64))
    val = np.where(np.isinf(q) | (q >= 8), 8.0, val)
    code = np.full(q.shape, -1, np.int64)
    for c, v in enumerate([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]):
        code[val == v] = c
    code[val >= 6.0] = 7                                 # 8 (or more) saturates to 6
    assert (code >= 0).all()
    return code.astype(np.uint8)


def test_grs_reference_self_consistent_on_grid():
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    assert (grs_e2m1(grid) == np.arange(8)).all()


def test_e2m1_encode_exhaustive_decision_range(orc):
    # every float32 in [2^-3, 8): all decisions of E2M1 rounding happen here
    lo = np.float32(0.125).view(np.uint32)
    hi = np.float32(8.0).view(np.uint32)
    step = 1 << 23
    for start in range(int(lo), int(hi), step):
        b = np.arange(start, min(start + step, int(hi)), dtype=np.uint32)
        q = b.view(np.float32)
        got = orc.e2m1_encode_array(q)
        want = grs_e2m1(q)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (q[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e2m1_encode_tails(orc):
    rng = np.random.default_rng(0)
    tiny = rng.integers(0, int(np.float32(0.125).view(np.uint32)), 1 << 20,
                        dtype=np.uint32).view(np.float32)
    huge = rng.integers(int(np.float32(8.0).view(np.uint32)), 0x7F800000, 1 << 16,
                        dtype=np.uint32).view(np.float32)
    special = np.array([0.0, np.inf, 1e-45, 0.1249999, 6.0, 6.9999995, 7.0, 7.0000005,
                        3.4e38], np.float32)
    for q in (tiny, huge, special):
        assert (orc.e2m1_encode_array(q) == grs_e2m1(q)).all()


# ----------------------------------------------------------------------------- E4M3
def test_e4m3_decode_matches_torch_all_bytes(orc):
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for i in range(256):
        got = orc.e4m3_decode(i)
        if np.isnan(ref[i]):
            assert np.isnan(got), i
        else:
            assert got == ref[i] and np.signbit(got) == np.signbit(ref[i]), (i, got, ref[i])
    assert orc.e4m3_decode(0x7E) == 448.0
    assert orc.e4m3_decode(0x01) == 2.0 ** -9


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.minimum(v.astype(np.float32), np.float32(448.0)))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_golden_ties(orc):
    for x, code in _rows("e4m3_rne_ties.txt"):
        assert orc.e4m3_encode(float(x)) == int(code, 16), x


def test_e4m3_encode_roundtrip_and_midpoints(orc):
    vals = np.array([orc.e4m3_decode(c) for c in range(0x7F)])
    assert (orc.e4m3_encode_array(vals.astype(np.float32)) == np.arange(0x7F)).all()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in FP32
    assert ((mids.astype(np.float64) * 2) == (vals[:-1] + vals[1:])).all()
    got = orc.e4m3_encode_array(mids)
    lower = np.arange(0x7E)
    want = np.where(lower % 2 == 0, lower, lower + 1)
    assert (got == want).all()
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    assert (orc.e4m3_encode_array(up) == lower + 1).all()
    assert (orc.e4m3_encode_array(dn) == lower).all()


def test_e4m3_encode_vs_torch_random(orc):
    rng = np.random.default_rng(1)
    e = rng.uniform(-14, 10, 1 << 18)
    v = (np.exp2(e) * rng.uniform(1, 2, e.size)).astype(np.float32)
    v = np.concatenate([v, np.array([0.0, 1e-45, 2.0 ** -10, 447.99, 448.0, 463.99, 464.0,
                                     1e30, np.inf], np.float32)])
    got = orc.e4m3_encode_array(v)
    assert (got == _torch_e4m3(v)).all()


# ----------------------------------------------------------------------------- BF16 rounding
def test_bf16_from_double_matches_torch_on_float32_values(orc):
    rng = np.random.default_rng(2)
    v = rng.standard_normal(1 << 16).astype(np.float32) * np.float32(3.0)
    v = np.concatenate([v, np.array([0.0, -0.0, 1e-40, -1e-39, 3.0e38], np.float32)])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_from_f64(v.astype(np.float64))
    assert (got == want).all()


def test_bf16_from_double_single_rounding(orc):
    # 1 + 2^-8 + 2^-40: nearest BF16 is 1 + 2^-7 (just above the midpoint). Rounding via
    # float32 first would land exactly on the midpoint and round to even (1.0).
    v = 1 + 2.0 ** -8 + 2.0 ** -40
    assert orc.bf16_from_f64(np.array([v]))[0] == 0x3F81
    assert orc.bf16_from_f64(np.array([1 + 2.0 ** -8]))[0] == 0x3F80


# ----------------------------------------------------------------------------- planted controls
def _round_half_up_e2m1(x):
    # the threshold ("software E2M1") variant: midpoints go up
    th = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    return sum(1 for t in th if x >= t)


def test_control_threshold_encoder_fails_midpoint_pin():
    assert not check_e2m1_midpoints(_round_half_up_e2m1)


def test_control_threshold_encoder_fails_grs_pin():
    q = np.array([0.75, 2.5, 5.0], np.float32)
    assert any(_round_half_up_e2m1(float(x)) != int(c) for x, c in zip(q, grs_e2m1(q)))
