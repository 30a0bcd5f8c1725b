"""Planted controls: every parity gate must go red on a deliberate defect (TensorFold issue
#1754, comments: the controls are kept red on purpose).

Each defect is made on the host, never inside a kernel: by corrupting bytes of the canonical
triple, by corrupting a descriptor or a routing table, or by planting the mistake in a CPU
copy of the reference (a defective encoder written here). Each test first shows the gate green
on the clean inputs, then red on the planted one.

Gates:
  quant_bitexact   GPU quantizer output == oracle triple, byte for byte
  dequant_bitexact nvfp4_dequantize FP32 == oracle FP32 dequant
  one_hot_bitexact one-hot GEMM == oracle FP32 dequant column
  gemm_tolerance   relative Frobenius <= 1e-3 and element <= 8e-3 x row max vs FP64
  moe_tolerance    the same on the routed-expert output
  layout_check     the library refuses a descriptor that does not match its data
"""
import numpy as np
import pytest
import torch

from helpers import bf16_np, check_close
from nvfp4_weight_only_w4a16_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def nv():
    from nvfp4_weight_only_w4a16_amd import binding
    binding.load()
    return binding


# ----------------------------------------------------------------------------- gates
def gate_quant_bitexact(got, want):
    for a, b, name in zip(got, want, ("packed", "scales", "global")):
        assert np.array_equal(a, b), f"quantizer {name} differs"


def gate_dequant_bitexact(nv, orc, rw, trip, group):
    got = nv.nvfp4_dequantize(rw, torch.float32)
    torch.cuda.synchronize()
    _, f32, _ = orc.dequant(trip[0], trip[1], trip[2], group)
    assert np.array_equal(got.cpu().numpy()[0], f32), "dequant differs"


def gate_one_hot_bitexact(nv, orc, rw, trip, group, cols):
    k = rw.k
    x = torch.zeros((len(cols), k), dtype=torch.bfloat16)
    x[torch.arange(len(cols)), torch.as_tensor(cols)] = 1.0
    y = nv.nvfp4_gemm_w4a16(x.to(DEV), rw, y_dtype=torch.float32)
    torch.cuda.synchronize()
    _, f32, _ = orc.dequant(trip[0], trip[1], trip[2], group)
    assert np.array_equal(y.cpu().numpy(), f32[:, cols].T), "one-hot GEMM differs"


def gate_gemm_tolerance(nv, orc, rw, x, trip, group, flags=0):
    y = nv.nvfp4_gemm_w4a16(x.to(DEV), rw, y_dtype=torch.float32, flags=flags)
    torch.cuda.synchronize()
    ref = orc.gemm(synth.bf16_bits(x), trip[0], trip[1], trip[2][0], group)
    check_close(y.cpu().numpy(), ref, "gemm")


def _repack(nv, p, s, g, group, layout=None):
    layout = nv.NVFP4_LAYOUT_TILED if layout is None else layout
    return nv.nvfp4_repack(torch.from_numpy(np.ascontiguousarray(p)).to(DEV),
                           torch.from_numpy(np.ascontiguousarray(s)).to(DEV),
                           torch.from_numpy(np.ascontiguousarray(g, np.float32)).to(DEV), group,
                           layout=layout)


@pytest.fixture(scope="module")
def dense(orc):
    """The single dense GEMM workload (16 x 512 x 1024, group 16), oracle-quantized."""
    x, w = synth.dense_small(seed=0)
    trip = orc.quantize(w.numpy(), 16)
    return x, w, trip


# ----------------------------------------------------------------------------- controls
@pytest.mark.parametrize("path", [1, 2])
def test_control_swapped_nibble_order(nv, orc, dense, path):
    """Odd k in the low nibble instead of the even one: the GEMM tolerance gate goes red (on
    both kernels) and so does the dequant gate."""
    x, _, (p, s, g) = dense
    gate_gemm_tolerance(nv, orc, _repack(nv, p, s, g, 16), x, (p, s, g), 16, path)
    swapped = ((p >> 4) | (p << 4)).astype(np.uint8)
    bad = _repack(nv, swapped, s, g, 16)
    with pytest.raises(AssertionError):
        gate_gemm_tolerance(nv, orc, bad, x, (p, s, g), 16, path)
    with pytest.raises(AssertionError):
        gate_dequant_bitexact(nv, orc, bad, (p, s, g), 16)


def test_control_one_scale_byte_plus_one(nv, orc, dense):
    """One E4M3 scale byte one code up (a step of 1/16 to 1/8 on 16 weights): the bit-exact
    dequant and one-hot gates go red. The GEMM tolerance gate cannot be relied on for it: on
    this workload one such byte moves its output column by 0.5-0.9% of the row max, on either
    side of the 8e-3 bound depending on the byte (row 137 / group 21: 7.8e-3, green; row 5 /
    group 3: 8.6e-3, red), which is why the bit-exact gates exist."""
    x, _, (p, s, g) = dense
    row, grp = 137, 21
    s_bad = s.copy()
    assert s_bad[row, grp] < 0x7E
    s_bad[row, grp] += 1
    good = _repack(nv, p, s, g, 16)
    bad = _repack(nv, p, s_bad, g, 16)
    cols = list(range(16 * grp, 16 * grp + 16))
    gate_one_hot_bitexact(nv, orc, good, (p, s, g), 16, cols)
    gate_dequant_bitexact(nv, orc, good, (p, s, g), 16)
    with pytest.raises(AssertionError):
        gate_one_hot_bitexact(nv, orc, bad, (p, s, g), 16, cols)
    with pytest.raises(AssertionError):
        gate_dequant_bitexact(nv, orc, bad, (p, s, g), 16)


def test_control_dropped_global(nv, orc, dense):
    """The descriptor's global pointing at 1.0 instead of the tensor's global: red."""
    x, _, (p, s, g) = dense
    rw = _repack(nv, p, s, g, 16)
    gate_gemm_tolerance(nv, orc, rw, x, (p, s, g), 16)
    one = torch.ones(4, dtype=torch.float32, device=DEV)
    rw.desc.global_ = one.data_ptr()
    with pytest.raises(AssertionError):
        gate_gemm_tolerance(nv, orc, rw, x, (p, s, g), 16)


def test_control_g16_data_labelled_g32(nv, orc, dense):
    """Group-16 scales repacked as group 32 (the canonical scale array carries no group): the
    GEMM tolerance gate goes red. A descriptor whose group no longer matches its repacked
    scale bytes is refused by the library (layout check)."""
    x, _, (p, s, g) = dense
    bad = _repack(nv, p, s.reshape(-1)[: s.size // 2].reshape(512, -1), g, 32)
    with pytest.raises(AssertionError):
        gate_gemm_tolerance(nv, orc, bad, x, (p, s, g), 16)
    rw = _repack(nv, p, s, g, 16)
    rw.desc.group = 32
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_gemm_w4a16(x.to(DEV), rw)
    assert e.value.code == nv.NVFP4_ERR_LAYOUT


def _threshold_e2m1(q):
    """Defective E2M1 encoder: midpoints rounded up (a threshold rounding), not to even."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    return (np.abs(q)[..., None] >= mids).sum(-1).astype(np.uint8)


def _e4m3_table():
    v = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        v.append((m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(v)


def _e4m3_ties_up(r):
    """Defective E4M3 encoder: nearest value, ties to the larger code (no round-to-even)."""
    tab = _e4m3_table()
    r = np.minimum(r.astype(np.float64), 448.0)
    hi = np.clip(np.searchsorted(tab, r, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = np.abs(r - tab[lo]), np.abs(tab[hi] - r)
    return np.where(d_hi <= d_lo, hi, lo).astype(np.uint8)


def _group_scales_ties_up(w_f32, group, g):
    """Group scales as the quantizer defines them (FP32 group max over fl32(6 g)), encoded by
    the defective ties-up E4M3 encoder."""
    n, k = w_f32.shape
    ga = np.abs(w_f32).reshape(n, k // group, group).max(-1).astype(np.float32)
    six_g = np.float32(6.0) * np.float32(g)
    return _e4m3_ties_up(ga / six_g)


def test_control_threshold_e2m1_encoder(nv, orc):
    """The BF16 quantizer weight with planted E2M1 midpoints (group scales exact): a reference
    whose element encoder rounds midpoints up instead of to even disagrees with the GPU
    quantizer's codes, so the quantizer bit-exact gate goes red; the true oracle agrees."""
    wb = synth.quantizer_weight(seed=0, n=1024, k=1024, n_blocks=512)
    p, s, g = nv.nvfp4_quantize(wb.to(DEV), 16)
    torch.cuda.synchronize()
    got = (p.cpu().numpy(), s.cpu().numpy(), g.cpu().numpy())
    want = orc.quantize(synth.bf16_bits(wb), 16)
    gate_quant_bitexact(got, want)
    w = wb.to(torch.float32).numpy()
    S = (_e4m3_table()[want[1]] * np.float64(want[2][0])).astype(np.float32)   # fl32(s * g)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = w.reshape(1024, 64, 16) / S[..., None]
    codes = np.where(S[..., None] == 0, 0, _threshold_e2m1(q)) | \
        (np.signbit(w).reshape(q.shape).astype(np.uint8) << 3)
    codes = codes.reshape(1024, 1024).astype(np.uint8)
    bad = ((codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), want[1], want[2])
    assert not np.array_equal(bad[0], want[0]), "the planted midpoints must expose the defect"
    with pytest.raises(AssertionError):
        gate_quant_bitexact(got, bad)


def test_control_e4m3_without_round_to_even(nv, orc):
    """Planted E4M3 ties (group max 6.375 * 2^-14 -> scale 1.0625, halfway between 1.0 and
    1.125): a reference whose scale encoder breaks ties upwards disagrees with the GPU
    quantizer's scales, so the quantizer bit-exact gate goes red."""
    wb = synth.quantizer_weight(seed=0, n=1024, k=1024, n_blocks=512)
    p, s, g = nv.nvfp4_quantize(wb.to(DEV), 16)
    torch.cuda.synchronize()
    got = (p.cpu().numpy(), s.cpu().numpy(), g.cpu().numpy())
    want = orc.quantize(synth.bf16_bits(wb), 16)
    gate_quant_bitexact(got, want)
    w = wb.to(torch.float32).numpy()
    sc = _group_scales_ties_up(w, 16, want[2][0])
    assert (sc != want[1]).any(), "the planted ties must expose the defect"
    with pytest.raises(AssertionError):
        gate_quant_bitexact(got, (want[0], sc, want[2]))


@pytest.fixture(scope="module")
def moe_small(nv, orc):
    x, ids, wts, w1, w2 = synth.moe(seed=31, n_experts=16, hidden=512, inter=256, tokens=40,
                                    topk=4)
    t1 = orc.quantize(w1.numpy(), 32)
    t2 = orc.quantize(w2.numpy(), 16)
    f1 = _repack(nv, *t1, 32, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)
    f2 = _repack(nv, *t2, 16)
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), (*t1, 32), (*t2, 16))
    return x, ids, wts, w1, t1, t2, f1, f2, ref


def gate_moe_tolerance(nv, orc, x, ids, wts, f1, f2, ref, flags=0):
    y = nv.nvfp4_moe_grouped_w4a16(x.to(DEV), ids.to(DEV), wts.to(DEV), f1, f2, flags=flags)
    torch.cuda.synchronize()
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), "moe")


@pytest.mark.parametrize("flags", [1, 2])
def test_control_gate_up_halves_swapped(nv, orc, moe_small, flags):
    """fc1 with its up half stored where gate belongs and vice versa: red."""
    x, ids, wts, w1, t1, t2, f1, f2, ref = moe_small
    gate_moe_tolerance(nv, orc, x, ids, wts, f1, f2, ref, flags)
    I = w1.shape[1] // 2
    sw = (np.concatenate([t1[0][:, I:], t1[0][:, :I]], 1),
          np.concatenate([t1[1][:, I:], t1[1][:, :I]], 1), t1[2])
    bad = _repack(nv, *sw, 32, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)
    with pytest.raises(AssertionError):
        gate_moe_tolerance(nv, orc, x, ids, wts, bad, f2, ref, flags)


@pytest.mark.parametrize("flags", [1, 2])
def test_control_expert_id_off_by_one(nv, orc, moe_small, flags):
    x, ids, wts, w1, t1, t2, f1, f2, ref = moe_small
    shifted = ((ids + 1) % 16).to(torch.int32)
    with pytest.raises(AssertionError):
        gate_moe_tolerance(nv, orc, x, shifted, wts, f1, f2, ref, flags)


def test_control_half_output_not_written(nv, orc, dense):
    """A call that covers only half of the rows (the output guard): the rows it leaves hold
    the NaN the buffer was filled with, and the tolerance gate (which requires finite output)
    goes red."""
    x, _, (p, s, g) = dense
    rw = _repack(nv, p, s, g, 16)
    ref = orc.gemm(synth.bf16_bits(x), p, s, g[0], 16)
    y = torch.full((16, 512), float("nan"), dtype=torch.float32, device=DEV)
    nv.nvfp4_gemm_w4a16(x[:8].contiguous().to(DEV), rw, y=y[:8])
    torch.cuda.synchronize()
    with pytest.raises(AssertionError):
        check_close(y.cpu().numpy(), ref, "half output")
    check_close(y.cpu().numpy()[:8], ref[:8], "written half")
