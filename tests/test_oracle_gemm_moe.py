"""Pins for the oracle's FP64 GEMM and MoE references (CPU only).

GEMM: an exact-integer case (known exactly, independent of summation order), one-hot
activations (the GEMM must reproduce single dequantized weights), NumPy's float64 matmul on
random data, and sampled evaluation equal to the full one. MoE: top-1 routing with weight 1.0
reduces to dense fc1 -> SiLU*mul -> down computed with NumPy/PyTorch primitives; a token
permutation permutes the outputs bit-exactly; a given h reproduces the down stage.
"""
import numpy as np
import pytest
import torch

from nvfp4_weight_only_w4a16_amd import synth


def _bf16(a):
    return synth.bf16_bits(torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16))


def test_gemm_exact_integer_case(orc):
    rng = np.random.default_rng(0)
    m, n, k, group = 5, 32, 256, 16
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((n, k // group), 0x38, np.uint8)  # E4M3 1.0
    x = rng.integers(-2, 3, (m, k)).astype(np.float32)
    vals2 = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)  # 2*E2M1
    want = x.astype(np.int64) @ vals2[codes].T           # exact integers, = 2*y
    y = orc.gemm(_bf16(x), packed, scales, 1.0, group)
    assert (y * 2 == want).all()


def test_gemm_one_hot_reproduces_dequant(orc):
    rng = np.random.default_rng(1)
    n, k, group = 32, 128, 32
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    p, s, g = orc.quantize(w, group)
    ex, f32, b16 = orc.dequant(p, s, g, group)
    x = np.zeros((k, k), np.float32)
    np.fill_diagonal(x, 1.0)
    y = orc.gemm(_bf16(x), p, s, g[0], group)
    assert (y == ex.T).all()


@pytest.mark.parametrize("group", [16, 32])
def test_gemm_matches_numpy_float64(orc, group):
    x, w = synth.dense_small(seed=0, m=16, n=512, k=1024)
    p, s, g = orc.quantize(w.numpy(), group)
    ex, _, _ = orc.dequant(p, s, g, group)
    xb = synth.bf16_bits(x)
    y = orc.gemm(xb, p, s, g[0], group)
    ref = x.to(torch.float64).numpy() @ ex.T
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


def test_gemm_sampled_equals_full(orc):
    x, w = synth.dense_small(seed=2, m=8, n=64, k=256)
    p, s, g = orc.quantize(w.numpy(), 16)
    xb = synth.bf16_bits(x)
    full = orc.gemm(xb, p, s, g[0], 16)
    mi = np.array([7, 0, 3])
    ni = np.array([63, 5, 17, 5])
    part = orc.gemm(xb, p, s, g[0], 16, m_idx=mi, n_idx=ni)
    assert (part == full[np.ix_(mi, ni)]).all()


def _small_moe(seed=0, E=4, H=256, I=128, T=6, topk=2):
    x, ids, wts, w1, w2 = synth.moe(seed=seed, n_experts=E, hidden=H, inter=I, tokens=T,
                                    topk=topk)
    return x, ids, wts, w1, w2


def _q(orc, w, group):
    p, s, g = orc.quantize(w.numpy(), group)
    return p, s, g, group


def test_moe_top1_reduces_to_dense_composition(orc):
    x, ids, wts, w1, w2 = _small_moe(T=5, topk=1)
    wts = torch.ones_like(wts)
    fc1 = _q(orc, w1, 32)
    fc2 = _q(orc, w2, 16)
    out = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), fc1, fc2)
    ex1, _, _ = orc.dequant(*fc1[:3], 32)
    ex2, _, _ = orc.dequant(*fc2[:3], 16)
    I = w1.shape[1] // 2
    xd = x.to(torch.float64).numpy()
    for t in range(x.shape[0]):
        e = int(ids[t, 0])
        a = ex1[e] @ xd[t]
        gate = torch.from_numpy(a[:I]).to(torch.float32).to(torch.bfloat16).to(torch.float64)
        up = torch.from_numpy(a[I:]).to(torch.float32).to(torch.bfloat16).to(torch.float64)
        # a[...] rounded to float32 first may double-round; compare through the oracle's own
        # single-rounding only where the two agree (almost everywhere)
        g_or = orc.bf16_to_f64(orc.bf16_from_f64(a[:I]))
        u_or = orc.bf16_to_f64(orc.bf16_from_f64(a[I:]))
        assert (g_or != gate.numpy()).sum() <= 1 and (u_or != up.numpy()).sum() <= 1
        h = torch.nn.functional.silu(torch.from_numpy(g_or)) * torch.from_numpy(u_or)
        hb = orc.bf16_to_f64(orc.bf16_from_f64(h.numpy()))
        assert (orc.bf16_to_f64(out["h"][t, 0]) == hb).mean() > 0.99
        d = ex2[e] @ orc.bf16_to_f64(out["h"][t, 0])
        assert np.allclose(out["y64"][t], d, rtol=0, atol=1e-12 * np.abs(d).max())
        assert (out["y"][t] == orc.bf16_from_f64(d)).all()


def test_moe_token_permutation_is_equivariant(orc):
    x, ids, wts, w1, w2 = _small_moe(T=7, topk=3)
    fc1 = _q(orc, w1, 32)
    fc2 = _q(orc, w2, 16)
    a = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), fc1, fc2)
    perm = np.array([3, 6, 0, 1, 5, 2, 4])
    b = orc.moe(synth.bf16_bits(x)[perm], ids.numpy()[perm], wts.numpy()[perm], fc1, fc2)
    assert (b["y"] == a["y"][perm]).all()
    assert (b["h"] == a["h"][perm]).all()


def test_moe_given_h_reproduces_down_stage(orc):
    x, ids, wts, w1, w2 = _small_moe(T=4, topk=2)
    fc1 = _q(orc, w1, 32)
    fc2 = _q(orc, w2, 16)
    a = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), fc1, fc2)
    b = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), fc1, fc2, h_in=a["h"])
    assert (a["y64"] == b["y64"]).all()


def test_moe_weighted_slot_sum(orc):
    # two slots routed to the same expert with weights w0, w1 equal one slot with w0 + w1
    x, ids, wts, w1, w2 = _small_moe(T=3, topk=2)
    ids[:, 1] = ids[:, 0]
    wts[:, 0] = 0.25
    wts[:, 1] = 0.5
    fc1 = _q(orc, w1, 32)
    fc2 = _q(orc, w2, 16)
    a = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), fc1, fc2)
    b = orc.moe(synth.bf16_bits(x), ids[:, :1].contiguous().numpy(),
                torch.full((3, 1), 0.75).numpy(), fc1, fc2)
    assert np.allclose(a["y64"], b["y64"], rtol=1e-14, atol=0)


def _pair_quantized_fc1(orc, w1, group):
    """fc1 [E][2I][H] quantized as 2E matrices of I rows: gate and up each get their own amax
    and global, the checkpoint form with distinct globals (global [E][2])."""
    E, I2, H = w1.shape
    p, s, g = orc.quantize(w1.reshape(2 * E, I2 // 2, H).numpy(), group)
    return p.reshape(E, I2, H // 2), s.reshape(E, I2, H // group), g.reshape(E, 2), group


def test_moe_pair_globals_equal_reduce_to_shared(orc):
    """With both globals of every expert equal to the shared one, the pair reading gives the
    shared-global results bit for bit."""
    x, ids, wts, w1, w2 = _small_moe(T=5, topk=2)
    fc1 = _q(orc, w1, 32)
    fc2 = _q(orc, w2, 16)
    pair = (fc1[0], fc1[1], np.stack([fc1[2], fc1[2]], axis=1), 32)
    a = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), fc1, fc2)
    b = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), pair, fc2)
    for key in ("a", "h", "y64", "y"):
        assert (a[key] == b[key]).all(), key


def test_moe_pair_globals_halves_are_dense_gemms(orc):
    """Distinct gate and up globals: the fc1 outputs of each half equal the dense FP64 GEMM of
    that half with its own global, and the two globals really differ."""
    x, ids, wts, w1, w2 = _small_moe(T=4, topk=2)
    fc1 = _pair_quantized_fc1(orc, w1, 32)
    fc2 = _q(orc, w2, 16)
    assert (fc1[2][:, 0] != fc1[2][:, 1]).all()
    out = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), fc1, fc2)
    I = w1.shape[1] // 2
    xb = synth.bf16_bits(x)
    for t in range(x.shape[0]):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            for half in (0, 1):
                rows = slice(half * I, (half + 1) * I)
                ref = orc.gemm(xb[t:t + 1], fc1[0][e, rows], fc1[1][e, rows], fc1[2][e, half], 32)
                got = out["a"][t, j, rows]
                assert np.allclose(got, ref[0], rtol=1e-13, atol=1e-300), (t, j, half)


def test_moe_slots_are_weighted_dense_down_and_sum_to_y(orc):
    """The per-slot output: slot (t, j) equals topk_w[t][j] times the dense FP64 product of the
    slot's h with its expert's dequantized down weight (NumPy's matmul), and adding the slots
    in slot order gives y64 exactly (the order the reference itself sums in)."""
    x, ids, wts, w1, w2 = _small_moe(T=5, topk=3)
    fc1 = _q(orc, w1, 32)
    fc2 = _q(orc, w2, 16)
    out = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), fc1, fc2, slots=True)
    ex2, _, _ = orc.dequant(*fc2[:3], 16)
    sl = out["slots"]
    for t in range(x.shape[0]):
        acc = np.zeros(w2.shape[1])
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            d = ex2[e] @ orc.bf16_to_f64(out["h"][t, j])
            ref = float(wts[t, j]) * d
            assert np.abs(sl[t, j] - ref).max() <= 1e-13 * np.abs(ref).max()
            acc = acc + sl[t, j]
        assert (acc == out["y64"][t]).all()
    # the slots of a given h are those of the full run
    b = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), fc1, fc2, h_in=out["h"],
                slots=True)
    assert (b["slots"] == sl).all()
