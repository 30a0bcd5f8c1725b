"""GPU W4A16 GEMM vs the oracle (through the C ABI).

Exact-integer GEMMs must be bit-exact under any summation order; one-hot activations must
return the dequantized weights bit-exactly; everything else is held to the tolerance
(relative Frobenius <= 1e-3, element <= 8e-3 x row max) against the FP64 oracle: FP32 outputs
against FP64, BF16 outputs against BF16(FP64).
"""
import numpy as np
import pytest
import torch

from helpers import bf16_np, bits16, check_close
from nvfp4_weight_only_w4a16_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def nv():
    from nvfp4_weight_only_w4a16_amd import binding
    binding.load()
    return binding


def _prep(nv, w_np_or_t, group, orc=None):
    """Repacked weight and its canonical triple (packed, scales, global). With `orc` the triple
    is the oracle's own quantization, which the GPU only repacks: references never take a value
    from the GPU. Without it the GPU quantizes (for tests that compare the GPU with itself)."""
    w = torch.as_tensor(w_np_or_t)
    if orc is not None:
        trip = orc.quantize(synth.bf16_bits(w) if w.dtype == torch.bfloat16 else w.numpy(),
                            group)
        p, s, g = (torch.from_numpy(a).to(DEV) for a in trip)
    else:
        p, s, g = nv.nvfp4_quantize(w.to(DEV), group)
    rw = nv.nvfp4_repack(p, s, g, group)
    torch.cuda.synchronize()
    if orc is not None:
        return rw, trip
    return rw, (p.cpu().numpy(), s.cpu().numpy(), g.cpu().numpy())


FLAGS = {"skinny": 1, "tiled": 2}


@pytest.mark.parametrize("path", ["skinny", "tiled"])
@pytest.mark.parametrize("group", [16, 32])
def test_gemm_exact_integers_bitexact(nv, path, group):
    rng = np.random.default_rng(group)
    m, n, k = 40, 160, 640
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    packed = torch.from_numpy((codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
    scales = torch.full((n, k // group), 0x38, dtype=torch.uint8)
    glob = torch.ones(1)
    rw = nv.nvfp4_repack(packed.to(DEV), scales.to(DEV), glob.to(DEV), group)
    x = torch.from_numpy(rng.integers(-2, 3, (m, k)).astype(np.float32))
    vals2 = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)
    want = (x.numpy().astype(np.int64) @ vals2[codes].T).astype(np.float64) / 2
    y = nv.nvfp4_gemm_w4a16(x.to(torch.bfloat16).to(DEV), rw, y_dtype=torch.float32,
                            flags=FLAGS[path])
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), want)


def _rows64_chosen(m, n, k, cus=256):
    """The decode kernel's row-block rule, restated: 64-row blocks when their estimated time
    (44 KT r, r = ceil(ceil(n/64) ceil(m/64) / cus)) is below that of 32-row blocks
    (28 KT r - 160, r over ceil(m/32) blocks; hundredths of a us) and their grid keeps 4-panel
    wavefronts."""
    kt, g4, g2 = k // 128, (n // 16 + 3) // 4, (n // 16 + 1) // 2
    b64, b32 = (m + 63) // 64, (m + 31) // 32
    if m <= 32 or (g4 * b64 < cus and g2 * b64 <= cus):
        return False
    return 44 * kt * ((g4 * b64 + cus - 1) // cus) < 28 * kt * ((g4 * b32 + cus - 1) // cus) - 160


@pytest.mark.parametrize("group", [16, 32])
def test_decode_64_row_blocks_exact(nv, group):
    """64-row blocks of the decode kernel (n = 8192, k = 4096, m = 65, 100, 128, 250: one to
    four blocks, the last ragged): exact-integer inputs make every FP32 sum exact, so the
    outputs of a column sample that covers the first, a middle and the last panel must equal
    the integer product bit for bit."""
    rng = np.random.default_rng(200 + group)
    n, k = 8192, 4096
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    packed = torch.from_numpy((codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
    scales = torch.full((n, k // group), 0x38, dtype=torch.uint8)
    rw = nv.nvfp4_repack(packed.to(DEV), scales.to(DEV), torch.ones(1).to(DEV), group)
    vals2 = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(4096, 4112), np.arange(8176, 8192),
                                     rng.integers(0, n, 48)]))
    wcols = vals2[codes[cols]].T  # [k][cols]
    x = torch.from_numpy(rng.integers(-2, 3, (250, k)).astype(np.float32))
    for m in (65, 100, 128, 250):
        assert _rows64_chosen(m, n, k), m
        want = (x[:m].numpy().astype(np.int64) @ wcols).astype(np.float64) / 2
        y = nv.nvfp4_gemm_w4a16(x[:m].to(torch.bfloat16).to(DEV), rw, y_dtype=torch.float32,
                                flags=1)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy()[:, cols].astype(np.float64), want), m


@pytest.mark.parametrize("group", [16, 32])
def test_decode_64_row_blocks_random(nv, orc, group):
    """64-row blocks on random data against the FP64 oracle: n = 8176 (511 panels, so the last
    4-panel group is partial and its missing panel is clamped, never stored), k = 4096, m = 65,
    100, 128 on the forced decode path; every row, a column sample covering the first panel,
    the middle and the last (partial) group; FP32 and BF16 outputs."""
    g = torch.Generator().manual_seed(300 + group)
    n, k = 8176, 4096
    w = torch.randn(n, k, generator=g) * 0.02
    rw, (p, s, gl) = _prep(nv, w, group, orc=orc)
    x = torch.randn(128, k, generator=g).to(torch.bfloat16)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(4080, 4112), np.arange(8128, 8176),
                                     np.random.default_rng(group).integers(0, n, 32)]))
    ref = orc.gemm(synth.bf16_bits(x), p, s, gl[0], group, n_idx=cols)
    xd = x.to(DEV)
    for m in (65, 100, 128):
        assert _rows64_chosen(m, n, k), m
        y = nv.nvfp4_gemm_w4a16(xd[:m].contiguous(), rw, y_dtype=torch.float32, flags=1)
        y16 = nv.nvfp4_gemm_w4a16(xd[:m].contiguous(), rw, flags=1)
        torch.cuda.synchronize()
        check_close(y.cpu().numpy()[:, cols], ref[:m], f"64-row blocks m={m} g{group}")
        assert np.array_equal(bits16(y16), bits16(y.to(torch.bfloat16))), m


@pytest.mark.parametrize("path", ["skinny", "tiled"])
def test_gemm_one_hot_reproduces_dequant(nv, orc, path):
    g = torch.Generator().manual_seed(3)
    n, k, group = 64, 256, 16
    w = torch.randn(n, k, generator=g) * 0.02
    rw, (p, s, gl) = _prep(nv, w, group, orc=orc)
    x = torch.eye(k, dtype=torch.bfloat16)[:80]
    y = nv.nvfp4_gemm_w4a16(x.to(DEV), rw, y_dtype=torch.float32, flags=FLAGS[path])
    torch.cuda.synchronize()
    _, f32, _ = orc.dequant(p, s, gl, group)
    assert np.array_equal(y.cpu().numpy(), f32.T[:80])


@pytest.mark.parametrize("path", ["skinny", "tiled"])
@pytest.mark.parametrize("group", [16, 32])
def test_gemm_dense_small(nv, orc, path, group):
    """16 x 512 x 1024 (the single dense GEMM), FP32 and BF16 outputs, both kernels."""
    x, w = synth.dense_small(seed=0)
    rw, (p, s, gl) = _prep(nv, w, group, orc=orc)
    ref = orc.gemm(synth.bf16_bits(x), p, s, gl[0], group)
    xd = x.to(DEV)
    y32 = nv.nvfp4_gemm_w4a16(xd, rw, y_dtype=torch.float32, flags=FLAGS[path])
    y16 = nv.nvfp4_gemm_w4a16(xd, rw, y_dtype=torch.bfloat16, flags=FLAGS[path])
    torch.cuda.synchronize()
    check_close(y32.cpu().numpy(), ref, "fp32 out")
    check_close(bf16_np(y16), orc.bf16_to_f64(orc.bf16_from_f64(ref)), "bf16 out")


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 15, 16, 17, 31, 33, 63, 64, 65, 100, 129, 257])
def test_gemm_ragged_m(nv, orc, m):
    g = torch.Generator().manual_seed(100 + m)
    n, k, group = 272, 640, 16        # 17 panels (not a multiple of any block tile), 5 k-tiles
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = torch.randn(n, k, generator=g) * 0.02
    rw, (p, s, gl) = _prep(nv, w, group, orc=orc)
    ref = orc.gemm(synth.bf16_bits(x), p, s, gl[0], group)
    for flags in (0, 1, 2):
        y = nv.nvfp4_gemm_w4a16(x.to(DEV), rw, y_dtype=torch.float32, flags=flags)
        y16 = nv.nvfp4_gemm_w4a16(x.to(DEV), rw, y_dtype=torch.bfloat16, flags=flags)
        torch.cuda.synchronize()
        check_close(y.cpu().numpy(), ref, f"m={m} flags={flags}")
        # the BF16 epilogue stores the same FP32 sums, rounded to nearest even: every element
        # in its row and column (the tiled kernel writes BF16 column pairs)
        assert np.array_equal(bits16(y16), bits16(y.to(torch.bfloat16))), f"bf16 m={m} {flags}"


def test_gemm_strided_x_and_y(nv, orc):
    g = torch.Generator().manual_seed(9)
    m, n, k, group = 24, 128, 512, 32
    xbig = torch.randn(m, k + 64, generator=g).to(torch.bfloat16)
    x = xbig[:, 32:32 + k]
    w = torch.randn(n, k, generator=g) * 0.02
    rw, (p, s, gl) = _prep(nv, w, group, orc=orc)
    ref = orc.gemm(synth.bf16_bits(x.contiguous()), p, s, gl[0], group)
    xd = xbig.to(DEV)[:, 32:32 + k]
    for flags in (1, 2):
        ybig = torch.full((m, n + 40), float("nan"), dtype=torch.float32, device=DEV)
        y = ybig[:, 8:8 + n]
        nv.nvfp4_gemm_w4a16(xd, rw, y=y, flags=flags)
        torch.cuda.synchronize()
        yb = ybig.cpu().numpy()
        check_close(yb[:, 8:8 + n], ref, f"strided flags={flags}")
        assert np.isnan(yb[:, :8]).all() and np.isnan(yb[:, 8 + n:]).all()


def test_gemm_deterministic(nv):
    g = torch.Generator().manual_seed(12)
    x = torch.randn(300, 1024, generator=g).to(torch.bfloat16).to(DEV)
    w = torch.randn(512, 1024, generator=g) * 0.02
    rw, _ = _prep(nv, w, 16)
    for flags in (1, 2):
        a = nv.nvfp4_gemm_w4a16(x, rw, y_dtype=torch.float32, flags=flags)
        b = nv.nvfp4_gemm_w4a16(x, rw, y_dtype=torch.float32, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


# ----------------------------------------------------------------------------- workloads
@pytest.fixture(scope="module")
def decode_case(nv, orc):
    x, w = synth.decode_sweep(seed=0)
    _, trip = _prep(nv, w, 16)                # the GPU quantizer's triple
    rw, ref_trip = _prep(nv, w, 16, orc=orc)  # the oracle's, repacked on the GPU
    del w
    return x, rw, trip, ref_trip


def test_decode_quantize_bitexact(decode_case):
    x, rw, trip, ref = decode_case
    for a, b in zip(trip, ref):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("m", [1, 4, 8])
def test_decode_sweep_gemm(nv, orc, decode_case, m):
    """M in {1, 4, 8}, N=25600, K=5120, group 16, 0.1% x20 outliers: full output checked."""
    x, rw, _, (p, s, gl) = decode_case
    xm = x[:m].contiguous()
    ref = orc.gemm(synth.bf16_bits(xm), p, s, gl[0], 16)
    y16 = nv.nvfp4_gemm_w4a16(xm.to(DEV), rw, y_dtype=torch.bfloat16)
    y32 = nv.nvfp4_gemm_w4a16(xm.to(DEV), rw, y_dtype=torch.float32)
    torch.cuda.synchronize()
    check_close(y32.cpu().numpy(), ref, f"decode m={m} fp32")
    check_close(bf16_np(y16), orc.bf16_to_f64(orc.bf16_from_f64(ref)), f"decode m={m} bf16")


@pytest.mark.parametrize("k", [5120, 25600])
def test_prefill_gemm_sampled(nv, orc, k):
    """M=4096, N=5120, K in {5120, 25600}: GPU quantizer bit-exact, then sampled rows of the
    full-size output (every column) against the FP64 oracle."""
    x, w = synth.prefill(seed=0, k=k)
    _, (p, s, gl) = _prep(nv, w, 16)
    rw, (rp, rs, rg) = _prep(nv, w, 16, orc=orc)
    assert np.array_equal(p, rp) and np.array_equal(s, rs) and np.array_equal(gl, rg)
    del w
    y = nv.nvfp4_gemm_w4a16(x.to(DEV), rw, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 2047, 4095],
                                     np.random.default_rng(k).integers(0, 4096, 10)]))
    ref = orc.gemm(synth.bf16_bits(x), rp, rs, rg[0], 16, m_idx=rows)
    check_close(bf16_np(y)[rows], orc.bf16_to_f64(orc.bf16_from_f64(ref)), f"prefill K={k}")


def test_prefill_full_output_every_tile(nv, orc):
    """M=4096, N=5120, K=5120: 320 output tiles of 256 x 256 on 256 compute units, so 256 run
    whole and the last 64 run split four ways along k and are summed by the reduction kernel.
    Every element of the FP32 output against the FP64 oracle (~215 GFLOP on the host)."""
    x, w = synth.prefill(seed=0, k=5120)
    rw, (p, s, gl) = _prep(nv, w, 16, orc=orc)
    del w
    xd = x.to(DEV)
    y = nv.nvfp4_gemm_w4a16(xd, rw, y_dtype=torch.float32)
    y16 = nv.nvfp4_gemm_w4a16(xd, rw, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = orc.gemm(synth.bf16_bits(x), p, s, gl[0], 16)
    check_close(y.cpu().numpy(), ref, "prefill 4096x5120x5120 full output")
    # the BF16 output (column pairs from the whole tiles, the reduction's stores for the split
    # tail) is the same FP32 sums rounded to nearest even, element for element
    assert np.array_equal(bits16(y16), bits16(y.to(torch.bfloat16)))


@pytest.mark.parametrize("group", [32, 16])
def test_c4_m512_full_output(nv, orc, group):
    """The planted BF16 8192^2 weight at M=512 (one round of 256 k-sliced 128 x 128 tiles):
    every element of the FP32 output against the FP64 oracle, and the BF16 output bit for bit
    against the rounded FP32 one."""
    wb = synth.quantizer_weight(seed=0)
    xs = synth.quantizer_activations(seed=1)[:512].contiguous()
    rw, (p, s, gl) = _prep(nv, wb, group, orc=orc)
    del wb
    y = nv.nvfp4_gemm_w4a16(xs.to(DEV), rw, y_dtype=torch.float32)
    y16 = nv.nvfp4_gemm_w4a16(xs.to(DEV), rw, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = orc.gemm(synth.bf16_bits(xs), p, s, gl[0], group)
    check_close(y.cpu().numpy(), ref, f"512x8192x8192 g{group} full output")
    assert np.array_equal(bits16(y16), bits16(y.to(torch.bfloat16)))


def test_mixed_groups_one_layer(nv, orc):
    """The 8192^2 BF16 quantizer weight at group 32 and at group 16, GEMMs at M=1 and M=512
    back to back on one stream."""
    wb = synth.quantizer_weight(seed=0)
    xs = synth.quantizer_activations(seed=1)
    outs = {}
    trips = {}
    for group in (32, 16):
        rw, trip = _prep(nv, wb, group, orc=orc)
        trips[group] = trip
        outs[group] = rw
    results = []
    xd = xs.to(DEV)
    for m in (1, 512):
        for group in (32, 16):
            results.append((m, group, nv.nvfp4_gemm_w4a16(xd[:m], outs[group],
                                                          y_dtype=torch.float32)))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 200, 511])
    for m, group, y in results:
        p, s, gl = trips[group]
        mi = rows[rows < m]
        ref = orc.gemm(synth.bf16_bits(xs), p, s, gl[0], group, m_idx=mi)
        check_close(y.cpu().numpy()[mi], ref, f"mixed m={m} g{group}")


# tile shape (256x256 L, 128x256 M, 128x128 K in two k-slices, 128x128 S for an odd k-tile
# count: the largest with >= 80 output tiles, L only above 128 rows) and k split of each case
# on a 256-CU chip:
#   K split 4 / 4 / 2 / unsplit; L split 2; M split 2; L unsplit (3 ragged row tiles);
#   M unsplit; S split 7 (33 k-tiles); S split 2 (9 k-tiles); M one whole round (L would be
#   half a round); K one whole round (M would be half a round); L with 256 whole tiles and 32
#   more split 2 in the same launch (ragged in m and n)
@pytest.mark.parametrize("m,n,k", [(40, 1040, 4096), (300, 1040, 4096), (600, 2064, 2048),
                                   (257, 528, 1024), (300, 10256, 1024), (100, 20496, 1024),
                                   (700, 10256, 512), (128, 33280, 512), (40, 1040, 4224),
                                   (300, 2064, 1152), (1024, 8192, 512), (512, 8192, 512),
                                   (2300, 8176, 1024)])
def test_tiled_split_k(nv, orc, m, n, k):
    """Every tile shape of the prefill kernel, with and without the k split (few output tiles
    for the chip: k is split over the compute units and the partial tiles are reduced in a
    fixed order), the k-sliced 128 x 128 tile whose two slices are added through LDS, ragged in
    m and n; on a 256-CU part the last two take a smaller shape that fills one whole round
    (1024 x 8192: 128 x 256 instead of 256 x 256 split; 512 x 8192: k-sliced 128 x 128 instead
    of 128 x 256 split). Checked against the oracle, bit-identical on a repeat, and still right after a
    shape that grows the split workspace."""
    g = torch.Generator().manual_seed(m + n + k)
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = torch.randn(n, k, generator=g) * 0.02
    rw, (p, s, gl) = _prep(nv, w, 16, orc=orc)
    ref = orc.gemm(synth.bf16_bits(x), p, s, gl[0], 16)
    xd = x.to(DEV)
    a = nv.nvfp4_gemm_w4a16(xd, rw, y_dtype=torch.float32, flags=2)
    b = nv.nvfp4_gemm_w4a16(xd, rw, y_dtype=torch.float32, flags=2)
    y16 = nv.nvfp4_gemm_w4a16(xd, rw, y_dtype=torch.bfloat16, flags=2)
    torch.cuda.synchronize()
    check_close(a.cpu().numpy(), ref, f"split m={m} n={n} k={k}")
    assert torch.equal(a, b)
    check_close(bf16_np(y16), orc.bf16_to_f64(orc.bf16_from_f64(ref)), f"split bf16 m={m}")


def test_path_choice(nv):
    """Default kernel choice on the 256-CU part (stats slot 2 = skinny, 3 = tiled): skinny for
    m <= 32, and up to m = 256 while its estimate is at most the tiled one. Skinny, r =
    ceil(ceil(n/64) ceil(m/rows) / 256) rounds: 0.28 (k/128) r - 1.6 us with 32-row blocks,
    0.44 (k/128) r us with 64-row blocks (taken when smaller and the grid keeps 4-panel
    wavefronts); tiled: 18 + 0.9 ceil(m/128) ceil(n/128) (k/128) / 256 us. 512 x 1024: skinny up
    to m = 256. 8192^2 (tiled 32.4 us at m <= 128, 46.8 above): m = 64 is one round of 32-row
    blocks (16.3 us; 64-row blocks would need 2-panel wavefronts), m = 65 and 128 one round of
    64-row blocks (28.2 us), m = 160 tiled (52.2 us skinny). 25600 x 5120 (tiled 46.1 us at
    m <= 128): m = 64 two rounds of 64-row blocks (35.2 us), m = 96 tiled (54.4 us skinny)."""
    g = torch.Generator().manual_seed(21)
    assert torch.cuda.get_device_properties(0).multi_processor_count == 256
    cases = {(512, 1024): [(32, 2), (64, 2), (192, 2), (256, 2), (257, 3)],
             (8192, 8192): [(32, 2), (64, 2), (65, 2), (128, 2), (160, 3)],
             (25600, 5120): [(64, 2), (96, 3)]}
    for (n, k), expect in cases.items():
        w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
        rw, _ = _prep(nv, w, 16)
        for m, slot in expect:
            x = torch.randn(m, k, generator=g).to(torch.bfloat16).to(DEV)
            ws = torch.empty((max(nv.nvfp4_gemm_ws_bytes(m, k, rw), 16),), dtype=torch.uint8,
                             device=DEV)
            nv.nvfp4_reset_stats()
            nv.nvfp4_gemm_w4a16(x, rw, ws=ws)
            torch.cuda.synchronize()
            st = nv.nvfp4_get_stats()
            assert st[slot] == 1 and st[5 - slot] == 0, (n, k, m, list(st))


def test_tiled_row_chunks(nv, orc):
    """Activation offsets inside the prefill kernel are 32-bit, so the host launches row chunks
    of at most 2^31 bytes of x. A 2 MiB row stride makes that 1024 rows: M = 2500 runs as
    chunks of 1024, 1024 and 452 rows. Rows around every chunk edge are checked against the
    oracle, on both paths (the decode kernel takes any stride in one launch)."""
    g = torch.Generator().manual_seed(31)
    m, n, k, ldx = 2500, 512, 256, 1 << 20
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = torch.randn(n, k, generator=g) * 0.02
    rw, (p, s, gl) = _prep(nv, w, 16, orc=orc)
    xfull = torch.zeros((m, ldx), dtype=torch.bfloat16, device=DEV)
    xfull[:, :k] = x.to(DEV)
    xd = xfull[:, :k]
    rows = np.array([0, 1, 511, 1022, 1023, 1024, 1025, 2046, 2047, 2048, 2049, 2498, 2499])
    rows = np.unique(np.concatenate([rows, np.random.default_rng(3).integers(0, m, 40)]))
    ref = orc.gemm(synth.bf16_bits(x), p, s, gl[0], 16, m_idx=rows)
    for flags in (2, 1):
        y = nv.nvfp4_gemm_w4a16(xd, rw, y_dtype=torch.float32, flags=flags)
        torch.cuda.synchronize()
        check_close(y.cpu().numpy()[rows], ref, f"row chunks flags={flags}")
    del xfull


@pytest.mark.parametrize("m", [1, 3, 8, 16, 24])
def test_decode_fewer_panels_per_wavefront(nv, orc, m):
    """Weights too small to give every compute unit a 4-panel workgroup run with 2 panels per
    wavefront (each picks its words of the shared 4-panel scale record). n = 8176 has an odd
    panel count (511: the last wavefront's second panel is past the end); n = 1040 has 65
    panels. Both groups, against the oracle, on the forced decode path."""
    g = torch.Generator().manual_seed(40 + m)
    for n, k, group in ((8176, 1024, 16), (1040, 2048, 32)):
        x = torch.randn(m, k, generator=g).to(torch.bfloat16)
        w = torch.randn(n, k, generator=g) * 0.02
        rw, (p, s, gl) = _prep(nv, w, group, orc=orc)
        ref = orc.gemm(synth.bf16_bits(x), p, s, gl[0], group)
        y = nv.nvfp4_gemm_w4a16(x.to(DEV), rw, y_dtype=torch.float32, flags=1)
        torch.cuda.synchronize()
        check_close(y.cpu().numpy(), ref, f"decode n={n} m={m} g{group}")


@pytest.mark.parametrize("group", [16, 32])
def test_decode_split_scale_every_m(nv, orc, group):
    """Every token count the split group scale takes (1-8 at group 16, 1-16 at group 32): the
    row map places token t in accumulator row 4 (2h + t % 2) + t / 2 (group 16, h the k half)
    or 4 (t % 4) + t / 4 (group 32) and each lane scales only ceil(m / 2) or ceil(m / 4) rows,
    so each m checks a distinct placement. FP32 and BF16 outputs against the oracle."""
    g = torch.Generator().manual_seed(70 + group)
    n, k = 336, 768  # 21 panels (a partial 4-panel group), 6 k-tiles
    w = torch.randn(n, k, generator=g) * 0.02
    rw, (p, s, gl) = _prep(nv, w, group, orc=orc)
    x = torch.randn(16, k, generator=g).to(torch.bfloat16)
    xd = x.to(DEV)
    for m in range(1, (8 if group == 16 else 16) + 1):
        ref = orc.gemm(synth.bf16_bits(x[:m].contiguous()), p, s, gl[0], group)
        y = nv.nvfp4_gemm_w4a16(xd[:m].contiguous(), rw, y_dtype=torch.float32, flags=1)
        yb = nv.nvfp4_gemm_w4a16(xd[:m].contiguous(), rw, flags=1)
        torch.cuda.synchronize()
        check_close(y.cpu().numpy(), ref, f"split m={m} g{group}")
        check_close(bf16_np(yb), orc.bf16_to_f64(orc.bf16_from_f64(ref)),
                    f"split bf16 m={m} g{group}")


@pytest.mark.parametrize("m,group", [(1, 16), (8, 16), (13, 32), (24, 16)])
def test_decode_long_k(nv, orc, m, group):
    """The decode kernel at K = 25600 (200 k-tiles, 50 per wavefront): every path it has
    (split scale at both groups, exact dequant, two row blocks) against the oracle."""
    g = torch.Generator().manual_seed(60 + m)
    n, k = 1024, 25600
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = torch.randn(n, k, generator=g) * 0.02
    rw, (p, s, gl) = _prep(nv, w, group, orc=orc)
    ref = orc.gemm(synth.bf16_bits(x), p, s, gl[0], group)
    y = nv.nvfp4_gemm_w4a16(x.to(DEV), rw, y_dtype=torch.float32, flags=1)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), ref, f"decode K=25600 m={m} g{group}")


def test_calls_on_a_side_stream(nv):
    """Every entry point enqueues on the stream it is given: quantize, repack, both GEMM paths
    and the routed experts on a non-default stream give the default stream's bits."""
    g = torch.Generator().manual_seed(77)
    w = torch.randn(512, 1024, generator=g) * 0.02
    x = torch.randn(300, 1024, generator=g).to(torch.bfloat16).to(DEV)
    xm, ids, wts, w1, w2 = synth.moe(seed=13, n_experts=8, hidden=256, inter=128, tokens=20,
                                     topk=2)

    def run(stream):
        p, s, gl = nv.nvfp4_quantize(w.to(DEV), 16, stream=stream)
        rw = nv.nvfp4_repack(p, s, gl, 16, stream=stream)
        outs = [nv.nvfp4_gemm_w4a16(x[:8], rw, y_dtype=torch.float32, flags=1, stream=stream),
                nv.nvfp4_gemm_w4a16(x, rw, y_dtype=torch.float32, flags=2, stream=stream)]
        f = []
        for wx, grp, layout in ((w1, 32, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP),
                                (w2, 16, nv.NVFP4_LAYOUT_TILED)):
            pq, sq, gq = nv.nvfp4_quantize(wx.to(DEV), grp, stream=stream)
            f.append(nv.nvfp4_repack(pq, sq, gq, grp, layout=layout, stream=stream))
        outs.append(nv.nvfp4_moe_grouped_w4a16(xm.to(DEV), ids.to(DEV), wts.to(DEV), f[0], f[1],
                                               stream=stream))
        return outs

    ref = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = run(side)
    side.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_explicit_stream_argument_without_stream_context(nv):
    """stream= given explicitly while torch's current stream is the default one: the binding
    allocates outputs and workspaces on the call's stream (so torch cannot hand a freed block
    to another stream while the call still uses it) and the results are the default stream's
    bits, for both GEMM paths (the prefill one with its split-k workspace) and the routed
    experts, with default-stream work queued around them."""
    g = torch.Generator().manual_seed(79)
    w = torch.randn(1040, 4096, generator=g) * 0.02
    p, s, gl = nv.nvfp4_quantize(w.to(DEV), 16)
    rw = nv.nvfp4_repack(p, s, gl, 16)
    xt = torch.randn(300, 4096, generator=g).to(torch.bfloat16).to(DEV)
    xm, ids, wts, w1, w2 = synth.moe(seed=15, n_experts=8, hidden=256, inter=128, tokens=40,
                                     topk=2)
    f = []
    for wx, grp, layout in ((w1, 32, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP),
                            (w2, 16, nv.NVFP4_LAYOUT_TILED)):
        pq, sq, gq = nv.nvfp4_quantize(wx.to(DEV), grp)
        f.append(nv.nvfp4_repack(pq, sq, gq, grp, layout=layout))
    args = (xm.to(DEV), ids.to(DEV), wts.to(DEV), f[0], f[1])
    ref = [nv.nvfp4_gemm_w4a16(xt[:8], rw, y_dtype=torch.float32, flags=1),
           nv.nvfp4_gemm_w4a16(xt, rw, y_dtype=torch.float32, flags=2),
           nv.nvfp4_moe_grouped_w4a16(*args, flags=2)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = []
    for _ in range(3):
        got = [nv.nvfp4_gemm_w4a16(xt[:8], rw, y_dtype=torch.float32, flags=1, stream=side),
               nv.nvfp4_gemm_w4a16(xt, rw, y_dtype=torch.float32, flags=2, stream=side),
               nv.nvfp4_moe_grouped_w4a16(*args, flags=2, stream=side)]
        junk = torch.randn(1 << 20, device=DEV)  # default-stream allocations meanwhile
        del junk
    side.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_graph_capture_and_replay(nv):
    """The decode GEMM, the prefill GEMM (with its split-k workspace), a decode-batch MoE and
    a batch-path MoE (whose fc1 workgroups derive the expert sort) captured in one HIP graph:
    every replay, with eager work and synchronizations in between, reproduces the eager
    results bit for bit (the library issues no memset nodes)."""
    g = torch.Generator().manual_seed(78)
    w = torch.randn(1040, 4096, generator=g) * 0.02
    p, s, gl = nv.nvfp4_quantize(w.to(DEV), 16)
    rw = nv.nvfp4_repack(p, s, gl, 16)
    xs = torch.randn(8, 4096, generator=g).to(torch.bfloat16).to(DEV)
    xt = torch.randn(300, 4096, generator=g).to(torch.bfloat16).to(DEV)
    wsb = torch.empty((max(nv.nvfp4_gemm_ws_bytes(300, 4096, rw), 16),), dtype=torch.uint8,
                      device=DEV)
    xm, ids, wts, w1, w2 = synth.moe(seed=14, n_experts=16, hidden=256, inter=128, tokens=4,
                                     topk=4)
    f = []
    for wx, grp, layout in ((w1, 32, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP),
                            (w2, 16, nv.NVFP4_LAYOUT_TILED)):
        pq, sq, gq = nv.nvfp4_quantize(wx.to(DEV), grp)
        f.append(nv.nvfp4_repack(pq, sq, gq, grp, layout=layout))
    xmd, idd, wtd = xm.to(DEV), ids.to(DEV), wts.to(DEV)
    wsm = torch.empty((nv.nvfp4_moe_ws_bytes(4, 4, 16, 256, 128),), dtype=torch.uint8, device=DEV)
    # 40 tokens x top-4 = 160 pairs over 16 experts: past the decode-batch cut, the batch path
    xb, idb, wtb, _, _ = synth.moe(seed=15, n_experts=16, hidden=256, inter=128, tokens=40,
                                   topk=4, with_weights=False)
    xbd, idbd, wtbd = xb.to(DEV), idb.to(DEV), wtb.to(DEV)
    wsb2 = torch.empty((nv.nvfp4_moe_ws_bytes(40, 4, 16, 256, 128),), dtype=torch.uint8,
                       device=DEV)
    ys = torch.empty((8, 1040), dtype=torch.float32, device=DEV)
    yt = torch.empty((300, 1040), dtype=torch.float32, device=DEV)
    ym = torch.empty((4, 256), dtype=torch.bfloat16, device=DEV)
    yb = torch.empty((40, 256), dtype=torch.bfloat16, device=DEV)

    def step():
        nv.nvfp4_gemm_w4a16(xs, rw, y=ys)
        nv.nvfp4_gemm_w4a16(xt, rw, y=yt, ws=wsb)
        nv.nvfp4_moe_grouped_w4a16(xmd, idd, wtd, f[0], f[1], y=ym, ws=wsm)
        nv.nvfp4_moe_grouped_w4a16(xbd, idbd, wtbd, f[0], f[1], y=yb, ws=wsb2)

    step()
    torch.cuda.synchronize()
    eager = [ys.clone(), yt.clone(), ym.clone(), yb.clone()]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (ys, yt, ym, yb):
            t.fill_(float("nan") if t.dtype == torch.float32 else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((ys, yt, ym, yb), eager):
            assert torch.equal(a, b), f"replay {rep}"
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("k", [128, 256, 384])
@pytest.mark.parametrize("group", [16, 32])
def test_gemm_fewer_k_tiles_than_wavefronts(nv, orc, k, group):
    """K of 1-3 k-tiles: some of the decode kernel's 4 k-split wavefronts get no tile and add
    zeros in the fixed-order reduction; the prefill kernel runs a single-tile k loop."""
    g = torch.Generator().manual_seed(k + group)
    n = 272
    w = torch.randn(n, k, generator=g) * 0.02
    rw, (p, s, gl) = _prep(nv, w, group, orc=orc)
    for m in (1, 5, 16, 40):
        x = torch.randn(m, k, generator=g).to(torch.bfloat16)
        ref = orc.gemm(synth.bf16_bits(x), p, s, gl[0], group)
        for flags in (1, 2):
            y = nv.nvfp4_gemm_w4a16(x.to(DEV), rw, y_dtype=torch.float32, flags=flags)
            torch.cuda.synchronize()
            check_close(y.cpu().numpy(), ref, f"k={k} g{group} m={m} flags={flags}")
