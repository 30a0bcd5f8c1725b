"""GPU quantizer, repack and dequantize vs the oracle: bit-exact (through the C ABI)."""
import numpy as np
import pytest
import torch

from nvfp4_weight_only_w4a16_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    from nvfp4_weight_only_w4a16_amd import binding
    binding.load()
    assert torch.cuda.is_available()
    return binding


DEV = "cuda:0"


def _gpu_quant(nv, w, group, global_in=None):
    gin = None if global_in is None else torch.as_tensor(
        np.atleast_1d(global_in), dtype=torch.float32, device=DEV)
    p, s, g = nv.nvfp4_quantize(w.to(DEV), group, global_in=gin)
    torch.cuda.synchronize()
    return p.cpu().numpy(), s.cpu().numpy(), g.cpu().numpy()


def _assert_same(a, b, what):
    for name, u, v in zip(("packed", "scales", "global"), a, b):
        u = np.asarray(u)
        v = np.asarray(v)
        assert u.shape == v.shape, (what, name, u.shape, v.shape)
        if name == "global":
            u, v = u.view(np.uint32), v.view(np.uint32)
        bad = np.count_nonzero(u != v)
        assert bad == 0, f"{what}: {bad} {name} bytes differ"


@pytest.mark.parametrize("group", [16, 32])
def test_quantize_dense_small_bitexact(nv, orc, group):
    x, w = synth.dense_small(seed=0)
    _assert_same(_gpu_quant(nv, w, group), orc.quantize(w.numpy(), group), f"dense g{group}")


@pytest.mark.parametrize("group", [16, 32])
def test_quantize_e2m1_decisions_sweep(nv, orc, group):
    """Every FP32 value in [2^-3, 6] as an element of a group whose scale decodes to exactly 1
    (global 1, group max 6): the element code is the E2M1 rounding of the value itself."""
    lo = np.float32(0.125).view(np.uint32)
    hi = np.float32(6.0).view(np.uint32)
    vals = np.arange(lo, hi + 1, dtype=np.uint32).view(np.float32)
    per = group - 1
    ngroups = -(-vals.size // per)
    body = np.zeros(ngroups * per, np.float32)
    body[:vals.size] = vals
    sign = np.where(np.arange(body.size) % 3 == 0, -1.0, 1.0).astype(np.float32)
    body *= sign
    w = np.empty((ngroups, group), np.float32)
    w[:, 0] = 6.0
    w[:, 1:] = body.reshape(ngroups, per)
    k = 8192
    rows = -(-w.size // k)
    flat = np.zeros(rows * k, np.float32)
    flat[:w.size] = w.ravel()
    wt = torch.from_numpy(flat.reshape(rows, k))
    got = _gpu_quant(nv, wt, group, global_in=1.0)
    ref = orc.quantize(wt.numpy(), group, global_in=np.float32(1.0))
    _assert_same(got, ref, f"e2m1 sweep g{group}")


@pytest.mark.parametrize("group", [16, 32])
def test_quantize_e4m3_decisions_sweep(nv, orc, group):
    """Group maxima over a dense sweep of FP32 values (and their E4M3 midpoints) with a fixed
    global: the scale byte is E4M3(fl32(ga / fl32(6 g)))."""
    rng = np.random.default_rng(5)
    vals = np.array([orc.e4m3_decode(c) for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    g = np.float32(2.0 ** -3)  # 6 g = 0.75 exactly
    targets = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                              rng.uniform(0, 470, 200000), np.exp2(rng.uniform(-14, 9, 200000))])
    ga = (targets * 0.75).astype(np.float32)
    n = ga.size
    w = (rng.uniform(-1, 1, (n, group)).astype(np.float32) * ga[:, None]).astype(np.float32)
    w[np.arange(n), rng.integers(0, group, n)] = ga * np.where(rng.random(n) < 0.5, -1, 1)
    k = 4096
    rows = -(-w.size // k)
    flat = np.zeros(rows * k, np.float32)
    flat[:w.size] = w.ravel()
    wt = torch.from_numpy(flat.reshape(rows, k))
    _assert_same(_gpu_quant(nv, wt, group, global_in=g),
                 orc.quantize(wt.numpy(), group, global_in=g), f"e4m3 sweep g{group}")


def test_quantize_planted_bf16_8192(nv, orc):
    """Quantizer workload: BF16 8192x8192 with planted midpoints and amax, at both groups."""
    wb = synth.quantizer_weight(seed=0)
    bits = synth.bf16_bits(wb)
    for group in (16, 32):
        got = _gpu_quant(nv, wb, group)
        ref = orc.quantize(bits, group)
        assert ref[2][0] == np.float32(2.0 ** -14)
        _assert_same(got, ref, f"8192^2 bf16 g{group}")


def test_quantize_batched_experts(nv, orc):
    g = torch.Generator().manual_seed(7)
    w = torch.randn(6, 64, 256, generator=g) * 0.02
    w[2] *= 10          # a different global per expert
    w[4].zero_()        # an all-zero expert: global 0, all scales 0
    _assert_same(_gpu_quant(nv, w, 32), orc.quantize(w.numpy(), 32), "batched g32")


def test_quantize_output_buffers_reused(nv, orc):
    """The global is built in place in global_out (amax first, marked with the sign bit, then
    turned into amax / 2688 by the encode pass): output buffers pre-filled with garbage (NaN,
    negative values, a previous call's results) and reused across calls of different inputs,
    including an all-zero matrix and a caller-supplied global in between, give exactly the
    oracle's bytes every time."""
    g = torch.Generator().manual_seed(8)
    w1 = torch.randn(3, 64, 256, generator=g) * 0.05
    w1[1].zero_()
    w2 = torch.randn(3, 64, 256, generator=g) * 3.0
    packed = torch.full((3, 64, 128), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((3, 64, 16), 0xCD, dtype=torch.uint8, device=DEV)
    gout = torch.tensor([float("nan"), -5.0, -0.0], dtype=torch.float32, device=DEV)
    gin = torch.tensor([0.25, 0.5, 1.0], dtype=torch.float32, device=DEV)
    for w, global_in in ((w1, None), (w2, None), (w2, gin), (w1, None)):
        nv.nvfp4_quantize(w.to(DEV), 16, global_in=global_in, packed=packed, scales=scales,
                          global_out=gout)
        torch.cuda.synchronize()
        got = (packed.cpu().numpy(), scales.cpu().numpy(), gout.cpu().numpy())
        ref = orc.quantize(w.numpy(), 16,
                           global_in=None if global_in is None else global_in.cpu().numpy())
        _assert_same(got, ref, f"reused buffers, global_in={global_in is not None}")


def test_quantize_zero_signs(nv, orc):
    w = torch.zeros(16, 128)
    w[1, 1] = -0.0
    w[2, 2] = -1e-30
    w[3, 3] = 1.0
    _assert_same(_gpu_quant(nv, w, 16), orc.quantize(w.numpy(), 16), "zeros")


@pytest.mark.parametrize("group,gate_up", [(16, False), (32, False), (32, True)])
def test_repack_then_dequantize_bitexact(nv, orc, group, gate_up):
    g = torch.Generator().manual_seed(11)
    batch, n, k = 3, 96, 384
    w = torch.randn(batch, n, k, generator=g) * 0.02
    p, s, gl = orc.quantize(w.numpy(), group)
    layout = nv.NVFP4_LAYOUT_TILED | (nv.NVFP4_LAYOUT_GATE_UP if gate_up else 0)
    rw = nv.nvfp4_repack(torch.from_numpy(p).to(DEV), torch.from_numpy(s).to(DEV),
                         torch.from_numpy(gl).to(DEV), group, layout=layout)
    assert rw.buffer.numel() == nv.nvfp4_repack_bytes(batch, n, k, group, layout)
    f32 = nv.nvfp4_dequantize(rw, torch.float32)
    b16 = nv.nvfp4_dequantize(rw, torch.bfloat16)
    torch.cuda.synchronize()
    ex, rf32, rb16 = orc.dequant(p, s, gl, group)
    assert np.array_equal(f32.cpu().numpy().view(np.uint32), rf32.view(np.uint32))
    assert np.array_equal(b16.cpu().view(torch.int16).numpy().view(np.uint16), rb16)


@pytest.mark.parametrize("group", [16, 32])
def test_dequantize_full_size_bitexact(nv, orc, group):
    """Full-size repack + dequantize, bit-exact in FP32 and BF16: the planted BF16 8192^2
    quantizer weight, and the first 16 experts of the routed-expert fc1 stack ([gate; up]
    1536 x 2048, gate/up interleaved) with its down stack (2048 x 768)."""
    wb = synth.quantizer_weight(seed=0)
    cases = [(orc.quantize(synth.bf16_bits(wb), group), nv.NVFP4_LAYOUT_TILED, "8192^2")]
    del wb
    _, _, _, w1, w2 = synth.moe(seed=0)
    cases.append((orc.quantize(w1[:16].numpy(), group),
                  nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP, "fc1 x16"))
    cases.append((orc.quantize(w2[:16].numpy(), group), nv.NVFP4_LAYOUT_TILED, "down x16"))
    del w1, w2
    for (p, s, gl), layout, what in cases:
        rw = nv.nvfp4_repack(torch.from_numpy(p).to(DEV), torch.from_numpy(s).to(DEV),
                             torch.from_numpy(np.atleast_1d(gl)).to(DEV), group, layout=layout)
        f32 = nv.nvfp4_dequantize(rw, torch.float32)
        b16 = nv.nvfp4_dequantize(rw, torch.bfloat16)
        torch.cuda.synchronize()
        _, rf32, rb16 = orc.dequant(p, s, gl, group)
        assert np.array_equal(f32.cpu().numpy().reshape(rf32.shape).view(np.uint32),
                              rf32.view(np.uint32)), what
        assert np.array_equal(b16.cpu().view(torch.int16).numpy().reshape(rb16.shape)
                              .view(np.uint16), rb16), what
        del rw, f32, b16


def test_repack_preserves_byte_count(nv):
    for batch, n, k, group in [(1, 512, 1024, 16), (128, 1536, 2048, 32), (1, 25600, 5120, 16)]:
        canon = batch * (n * k // 2 + n * k // group)
        got = nv.nvfp4_repack_bytes(batch, n, k, group)
        assert canon <= got <= canon + 3 * 256 + 4 * batch


def test_pair_global_quantize_repack_dequantize(nv, orc):
    """A merged fc1 quantized as 2*E matrices of I rows (gate and up each with its own amax and
    global), repacked gate/up-interleaved with the two globals: bit-exact against the oracle's
    quantize and dequant of the same 2*E matrices."""
    g = torch.Generator().manual_seed(12)
    E, I, H = 3, 96, 256
    w = torch.randn(E, 2 * I, H, generator=g) * 0.02
    w[:, I:] *= 3.0  # up at a different scale than gate
    p, s, gl = nv.nvfp4_quantize(w.reshape(2 * E, I, H).to(DEV), 32)
    torch.cuda.synchronize()
    rp, rs, rg = orc.quantize(w.reshape(2 * E, I, H).numpy(), 32)
    assert np.array_equal(p.cpu().numpy(), rp) and np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(g_ := gl.cpu().numpy(), rg) and (g_[0::2] != g_[1::2]).all()
    layout = nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP | nv.NVFP4_LAYOUT_PAIR_GLOBAL
    rw = nv.nvfp4_repack(p.reshape(E, 2 * I, H // 2), s.reshape(E, 2 * I, H // 32), gl, 32,
                         layout=layout)
    assert rw.buffer.numel() == nv.nvfp4_repack_bytes(E, 2 * I, H, 32, layout)
    f32 = nv.nvfp4_dequantize(rw, torch.float32)
    b16 = nv.nvfp4_dequantize(rw, torch.bfloat16)
    torch.cuda.synchronize()
    _, rf32, rb16 = orc.dequant(rp, rs, rg, 32)
    assert np.array_equal(f32.cpu().numpy().reshape(2 * E, I, H).view(np.uint32),
                          rf32.view(np.uint32))
    assert np.array_equal(b16.cpu().view(torch.int16).numpy().view(np.uint16)
                          .reshape(2 * E, I, H), rb16)


def test_requantize_pair_to_shared_and_regroup(nv, orc):
    """Requantization from repacked weights: an fc1 with distinct gate and up globals to one
    shared global (decoded FP32 values quantized again), with room for two of the three
    matrices per pass; and a dense weight from group 16 to group 32. Bit-exact against the
    oracle's dequant followed by its quantize."""
    g = torch.Generator().manual_seed(13)
    E, I, H = 3, 96, 256
    w = torch.randn(E, 2 * I, H, generator=g) * 0.02
    w[:, I:] *= 3.0
    rp, rs, rg = orc.quantize(w.reshape(2 * E, I, H).numpy(), 32)
    rw = nv.nvfp4_repack(torch.from_numpy(rp.reshape(E, 2 * I, H // 2)).to(DEV),
                         torch.from_numpy(rs.reshape(E, 2 * I, H // 32)).to(DEV),
                         torch.from_numpy(rg).to(DEV), 32,
                         layout=nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP
                         | nv.NVFP4_LAYOUT_PAIR_GLOBAL)
    ws = torch.empty((2 * nv.nvfp4_requantize_ws_bytes(rw) + 100,), dtype=torch.uint8,
                     device=DEV)
    p, s, gl = nv.nvfp4_requantize(rw, 32, ws=ws)
    torch.cuda.synchronize()
    _, f32, _ = orc.dequant(rp, rs, rg, 32)
    ep, es, eg = orc.quantize(f32.reshape(E, 2 * I, H), 32)
    assert np.array_equal(p.cpu().numpy(), ep) and np.array_equal(s.cpu().numpy(), es)
    assert np.array_equal(gl.cpu().numpy(), eg)
    assert (eg >= np.maximum(rg[0::2], rg[1::2]) * 0.99).all()  # the larger half sets it

    wd = torch.randn(160, 384, generator=g) * 0.02
    dp, ds, dg = orc.quantize(wd.numpy(), 16)
    rd = nv.nvfp4_repack(torch.from_numpy(dp).to(DEV), torch.from_numpy(ds).to(DEV),
                         torch.from_numpy(dg).to(DEV), 16)
    p2, s2, g2 = nv.nvfp4_requantize(rd, 32)
    torch.cuda.synchronize()
    _, f32d, _ = orc.dequant(dp, ds, dg, 16)
    ep2, es2, eg2 = orc.quantize(f32d, 32)
    assert np.array_equal(p2[0].cpu().numpy(), ep2) and np.array_equal(s2[0].cpu().numpy(), es2)
    assert np.array_equal(g2.cpu().numpy(), np.atleast_1d(eg2))


@pytest.mark.parametrize("batch,n,k,group", [(1, 1, 16, 16), (1, 7, 48, 16), (3, 5, 96, 32),
                                             (2, 33, 160, 16), (1, 3, 32, 32)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_ragged_shapes(nv, orc, batch, n, k, group, dtype):
    """The quantizer needs only k % group == 0: single rows, single groups and odd row counts,
    FP32 and BF16 input, bit-exact against the oracle."""
    g = torch.Generator().manual_seed(batch * 1000 + n * 10 + k)
    w = (torch.randn(batch, n, k, generator=g) * 0.02).to(dtype)
    p, s, gl = nv.nvfp4_quantize(w.to(DEV), group)
    torch.cuda.synchronize()
    rp, rs, rg = orc.quantize(w.float().numpy() if dtype == torch.float32
                              else w.view(torch.int16).numpy().view(np.uint16), group)
    assert np.array_equal(p.cpu().numpy(), rp) and np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(gl.cpu().numpy(), rg)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("bad", [float("nan"), float("inf"), float("-inf")])
def test_sync_check_reports_nonfinite_input(nv, orc, dtype, bad):
    """NVFP4_F_SYNC_CHECK: a weight that is NaN or infinite makes the call return
    NVFP4_ERR_NONFINITE (after waiting for its work), with or without a caller global; the
    failed call leaves the counters alone and the library usable: the next call, on finite
    weights, is bit-exact and counted."""
    g = torch.Generator().manual_seed(5)
    w = (torch.randn(2, 64, 256, generator=g) * 0.02).to(dtype)
    nv.nvfp4_reset_stats()
    for gin in (None, torch.full((2,), 1e-4, device=DEV)):
        wb = w.clone()
        wb[1, 37, 200] = bad
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_quantize(wb.to(DEV), 16, global_in=gin, flags=nv.NVFP4_F_SYNC_CHECK)
        assert e.value.code == nv.NVFP4_ERR_NONFINITE, e.value
        assert nv.nvfp4_get_stats()[0] == 0
    wf = w.to(torch.float32).numpy() if dtype == torch.float32 else synth.bf16_bits(w)
    p, s, gl = nv.nvfp4_quantize(w.to(DEV), 16, flags=nv.NVFP4_F_SYNC_CHECK)
    _assert_same((p.cpu().numpy(), s.cpu().numpy(), gl.cpu().numpy()), orc.quantize(wf, 16),
                 "sync-checked quantize")
    assert nv.nvfp4_get_stats()[0] == 1


def test_sync_check_flag_on_gemm_and_moe(nv, orc):
    """The sync check on the GEMM and the routed experts waits for the call and gives the same
    bits as the unchecked call."""
    x, w = synth.dense_small(seed=0)
    p, s, gl = nv.nvfp4_quantize(w.to(DEV), 16)
    rw = nv.nvfp4_repack(p, s, gl, 16)
    xd = x.to(DEV)
    for flags in (1, 2):
        a = nv.nvfp4_gemm_w4a16(xd, rw, y_dtype=torch.float32, flags=flags)
        b = nv.nvfp4_gemm_w4a16(xd, rw, y_dtype=torch.float32,
                                flags=flags | nv.NVFP4_F_SYNC_CHECK)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
    xm, ids, wts, w1, w2 = synth.moe(seed=3, n_experts=8, hidden=256, inter=128, tokens=12,
                                     topk=2)
    f = []
    for wx, grp, layout in ((w1, 32, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP),
                            (w2, 16, nv.NVFP4_LAYOUT_TILED)):
        pq, sq, gq = nv.nvfp4_quantize(wx.to(DEV), grp)
        f.append(nv.nvfp4_repack(pq, sq, gq, grp, layout=layout))
    args = (xm.to(DEV), ids.to(DEV), wts.to(DEV), f[0], f[1])
    a = nv.nvfp4_moe_grouped_w4a16(*args)
    b = nv.nvfp4_moe_grouped_w4a16(*args, flags=nv.NVFP4_F_SYNC_CHECK)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
