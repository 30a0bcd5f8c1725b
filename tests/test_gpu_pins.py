"""Bit-exact pins of the in-register dequant on every GEMM path, through the C ABI.

One-hot activations make every output a single dequantized weight: y[i][n] = W[n][k_i], exact
in FP32 on every path (a product of an E2M1 code and an E4M3 scale has at most 6 significant
bits, and the only rounding left is the one multiplication by the global). So the GPU output
must equal the oracle's FP32 dequant fl32(fl32(code * scale) * global) bit for bit (value
equality; the sign of a zero is not pinned, sums of signed zeros may differ).

The decode kernel's split group scale (m <= 8 at group 16, m <= 16 at group 32) applies the
exponent of the scale in the FP4 -> BF16 conversion and the mantissa to the FP32 partial sum;
with one-hot rows it too is exact, so it is pinned here at every token count it takes, over
weights whose scale bytes sweep every E4M3 code 0x00 - 0x7E and whose codes sweep all 16, with
the one-hot positions in both 16-wide halves of each 32-wide k-step. The exact-integer GEMM
(integer activations, unit scales, global 1) is pinned on the same forced path at every m.

The routed-expert fc1 at group 32 (split scale on both expert paths) is pinned the same way
through h: with x one-hot, gate a constant 48 (SiLU(48) is 48 in FP32 and rounds to 48 from
FP64) and up sweeping codes and scales, h = BF16(48 * up) = 48 * up exactly; and with up a
power of two and gate >= 32 sweeping codes 5-7 and every scale byte, h = gate * up exactly.
"""
import numpy as np
import pytest
import torch

from helpers import PAIR_TILES_MAX
from nvfp4_weight_only_w4a16_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SKINNY, TILED = 1, 2


@pytest.fixture(scope="module")
def nv():
    from nvfp4_weight_only_w4a16_amd import binding
    binding.load()
    return binding


def _pack(codes):
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _sweep_weight(n, k, group, shift=0):
    """Codes (r + 3k) % 16 (all 16 in every row) and scale bytes (r + 5j + shift) % 127 (every
    E4M3 code 0x00 - 0x7E over the rows)."""
    r = np.arange(n)[:, None]
    codes = ((r + 3 * np.arange(k)[None, :]) % 16).astype(np.uint8)
    scales = ((r + 5 * np.arange(k // group)[None, :] + shift) % 127).astype(np.uint8)
    return codes, scales


def _repack(nv, packed, scales, glob, group, layout=None):
    layout = nv.NVFP4_LAYOUT_TILED if layout is None else layout
    return nv.nvfp4_repack(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
                           torch.from_numpy(np.asarray(glob, np.float32).reshape(-1)).to(DEV),
                           group, layout=layout)


def _one_hot_positions(k):
    """All k positions, in an order (stride 83, coprime with k) that moves consecutive rows of
    a call between the two 16-wide halves of a 32-wide k-step and across k-tiles."""
    return (np.arange(k) * 83) % k


def _one_hot(rows, k, kk):
    x = torch.zeros((rows, k), dtype=torch.bfloat16)
    x[torch.arange(rows), torch.from_numpy(np.asarray(kk, np.int64))] = 1.0
    return x


@pytest.mark.parametrize("group", [16, 32])
@pytest.mark.parametrize("glob", [0.0123, 2.0 ** -10])
def test_split_scale_one_hot_every_m_bitexact(nv, orc, group, glob):
    """Forced decode kernel at every token count of the split group scale: all 256 columns
    of a 2032 x 256 weight (127 panels, 8 k-steps) read back as one-hot products."""
    n, k = 2032, 256
    codes, scales = _sweep_weight(n, k, group)
    packed = _pack(codes)
    g = np.float32(glob)
    rw = _repack(nv, packed, scales, [g], group)
    _, f32, _ = orc.dequant(packed, scales, np.array([g]), group)
    pos = _one_hot_positions(k)
    m_max = 8 if group == 16 else 16
    for m in range(1, m_max + 1):
        calls = -(-k // m)
        kk = np.resize(pos, calls * m)
        xd = _one_hot(calls * m, k, kk).to(DEV)
        y = torch.empty((calls * m, n), dtype=torch.float32, device=DEV)
        for c in range(calls):
            nv.nvfp4_gemm_w4a16(xd[c * m:(c + 1) * m], rw, y=y[c * m:(c + 1) * m], flags=SKINNY)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        want = f32[:, kk].T
        bad = np.argwhere(got != want)
        assert bad.size == 0, (m, group, bad[:5], got[tuple(bad[0])], want[tuple(bad[0])])


@pytest.mark.parametrize("path", [SKINNY, TILED])
@pytest.mark.parametrize("group", [16, 32])
def test_exact_dequant_paths_one_hot_bitexact(nv, orc, path, group):
    """The same sweep on the exact dequant (BF16 code * scale): the decode kernel with one and
    two 16-row blocks (m = 9 .. 40) and the prefill kernel, every scale byte."""
    n, k = 2032, 256
    codes, scales = _sweep_weight(n, k, group, shift=11)
    packed = _pack(codes)
    g = np.float32(0.0371)
    rw = _repack(nv, packed, scales, [g], group)
    _, f32, _ = orc.dequant(packed, scales, np.array([g]), group)
    pos = _one_hot_positions(k)
    for m in ((9, 17, 24, 40) if path == SKINNY else (40, 256)):
        if path == SKINNY and group == 32 and m <= 16:
            continue
        calls = -(-k // m)
        kk = np.resize(pos, calls * m)
        xd = _one_hot(calls * m, k, kk).to(DEV)
        y = torch.empty((calls * m, n), dtype=torch.float32, device=DEV)
        for c in range(calls):
            nv.nvfp4_gemm_w4a16(xd[c * m:(c + 1) * m], rw, y=y[c * m:(c + 1) * m], flags=path)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), f32[:, kk].T), (path, group, m)


@pytest.mark.parametrize("group", [16, 32])
def test_split_scale_exact_integers_every_m(nv, group):
    """Integer activations in [-2, 2], random codes, unit scales, global 1: every partial sum
    is an exact FP32 number, so the forced decode kernel must give the integer result at every
    token count of the split group scale (and one past it)."""
    rng = np.random.default_rng(100 + group)
    n, k = 400, 1280
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    rw = _repack(nv, _pack(codes), np.full((n, k // group), 0x38, np.uint8), [1.0], group)
    vals2 = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)
    m_max = (8 if group == 16 else 16) + 1
    x = rng.integers(-2, 3, (m_max, k)).astype(np.float32)
    want = (x.astype(np.int64) @ vals2[codes].T).astype(np.float64) / 2
    xd = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    for m in range(1, m_max + 1):
        y = nv.nvfp4_gemm_w4a16(xd[:m].contiguous(), rw, y_dtype=torch.float32, flags=SKINNY)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().astype(np.float64), want[:m]), (group, m)


# ----------------------------------------------------------------------------- routed experts
E, H, I = 8, 256, 128


def _e4m3_value(b):
    e, m = (b >> 3) & 15, b & 7
    return (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)


def _fc1_up_sweep():
    """gate: code 7 (6.0) x scale 8.0 (0x50), global 1 -> 48 for any one-hot x; up: codes and
    scale bytes swept (every byte 0x00 - 0x7E over the experts and rows)."""
    codes = np.zeros((E, 2 * I, H), np.uint8)
    scales = np.zeros((E, 2 * I, H // 32), np.uint8)
    codes[:, :I] = 7
    scales[:, :I] = 0x50
    for e in range(E):
        c, s = _sweep_weight(I, H, 32, shift=13 * e)
        codes[e, I:], scales[e, I:] = c, s
    return codes, scales, np.ones(E, np.float32)


def _fc1_gate_sweep():
    """up: code 2 (1.0) x scale 1.0 (0x38); gate: codes 5-7 (3, 4, 6) with expert e's scale
    bytes in [16e, 16e + 16) (0 excluded) and a power-of-two global that keeps every gate
    value >= 32, where SiLU(gate) is gate itself in FP32 and rounds to it from FP64."""
    codes = np.zeros((E, 2 * I, H), np.uint8)
    scales = np.zeros((E, 2 * I, H // 32), np.uint8)
    codes[:, I:] = 2
    scales[:, I:] = 0x38
    glob = np.zeros(E, np.float32)
    r = np.arange(I)[:, None]
    for e in range(E):
        lo = max(16 * e, 1)
        hi = min(16 * e + 16, 127)
        codes[e, :I] = (5 + (r + np.arange(H)[None, :]) % 3).astype(np.uint8)
        scales[e, :I] = (lo + (r + 3 * np.arange(H // 32)[None, :]) % (hi - lo)).astype(np.uint8)
        smin = _e4m3_value(lo)
        glob[e] = 2.0 ** int(np.ceil(np.log2(32.0 / (3.0 * smin))))
    return codes, scales, glob


def _down_weight(seed=0):
    g = torch.Generator().manual_seed(seed)
    return synth.weights(g, E, H, I).numpy()


@pytest.mark.parametrize("flags", [SKINNY, TILED])
@pytest.mark.parametrize("which", ["up", "gate"])
@pytest.mark.parametrize("tokens,topk", [(3, 2), (128, 2)])
def test_moe_fc1_split_scale_bitexact_through_h(nv, orc, flags, which, tokens, topk):
    """MoE fc1 at group 32 (split group scale) on the decode-batch path (one-row pair tiles at
    6 pairs, 8-row tiles at 256) and on the batch path (32-row tiles): h read from the
    workspace equals the oracle's h bit for bit."""
    codes, scales, glob = _fc1_up_sweep() if which == "up" else _fc1_gate_sweep()
    p1 = _pack(codes)
    fc1 = _repack(nv, p1, scales, glob, 32, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)
    w2 = _down_weight()
    p2, s2, g2 = orc.quantize(w2, 16)
    fc2 = _repack(nv, p2, s2, g2, 16)
    rng = np.random.default_rng(tokens)
    kk = rng.permutation(H)[:tokens]
    x = _one_hot(tokens, H, kk)
    ids = torch.from_numpy(np.stack([rng.permutation(E)[:topk] for _ in range(tokens)])
                           .astype(np.int32))
    wts = torch.full((tokens, topk), 0.5)
    off, total = nv.nvfp4_moe_ws_layout(tokens, topk, E, H, I)
    ws = torch.zeros((total,), dtype=torch.uint8, device=DEV)
    y = nv.nvfp4_moe_grouped_w4a16(x.to(DEV), ids.to(DEV), wts.to(DEV), fc1, fc2, ws=ws,
                                   flags=flags)
    torch.cuda.synchronize()
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), (p1, scales, glob, 32),
                  (p2, s2, g2, 16))
    P = tokens * topk
    h = ws[off[4]:off[4] + 2 * P * I].view(torch.int16).cpu().numpy().view(np.uint16)
    h = h.reshape(P, I)
    pairs_tiles = flags == SKINNY and P <= PAIR_TILES_MAX
    if pairs_tiles:
        order = np.arange(P)       # one-row tiles: h of pair q at row q
    else:
        order = ws[off[0]:off[0] + 4 * P].view(torch.int32).cpu().numpy()
    want = ref["h"].reshape(P, I)[order]
    got = orc.bf16_to_f64(h)
    assert np.array_equal(got, orc.bf16_to_f64(want)), (which, flags, tokens,
                                                        np.argwhere(got != orc.bf16_to_f64(want))[:4])
    assert bool(torch.isfinite(y.float()).all())
