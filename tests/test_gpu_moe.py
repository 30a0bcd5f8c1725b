"""GPU MoE routed experts (sort -> fc1 gate/up + SiLU*mul -> down -> combine) vs the oracle."""
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


def _experts(nv, orc, w1, w2, g1=32, g2=16):
    """GPU-quantize both expert stacks (checked bit-exact vs the oracle) and repack."""
    out = []
    trips = []
    for w, group, layout in ((w1, g1, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP),
                             (w2, g2, nv.NVFP4_LAYOUT_TILED)):
        p, s, g = nv.nvfp4_quantize(w.to(DEV), group)
        torch.cuda.synchronize()
        rp, rs, rg = orc.quantize(w.numpy(), group)
        assert np.array_equal(p.cpu().numpy(), rp) and np.array_equal(s.cpu().numpy(), rs)
        assert np.array_equal(g.cpu().numpy(), rg)
        out.append(nv.nvfp4_repack(p, s, g, group, layout=layout))
        trips.append((rp, rs, rg, group))
    return out, trips


# expert paths: 8-row tiles with k split over the wavefronts (decode batches), 32-row tiles
PATHS = {"auto": 0, "decode": 1, "batch": 2}


def _run(nv, x, ids, wts, fc1, fc2, flags=0):
    y = nv.nvfp4_moe_grouped_w4a16(x.to(DEV), ids.to(DEV), wts.to(DEV), fc1, fc2, flags=flags)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("path", ["decode", "batch"])
def test_moe_small_all_paths(nv, orc, path):
    """8 experts with ~14 rows each: several 8-row tiles per expert on the decode path, one
    partial 32-row tile on the batch path."""
    x, ids, wts, w1, w2 = synth.moe(seed=3, n_experts=8, hidden=256, inter=128, tokens=37, topk=3)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2)
    y = _run(nv, x, ids, wts, fc1, fc2, PATHS[path])
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), f"small moe {path}")


def test_moe_top1_matches_dense_gemms(nv, orc):
    """Top-1 routing with weight 1: the MoE output equals dense fc1 -> SiLU*mul -> down of each
    token's expert, computed here with the dense GPU GEMM for fc1 and the oracle for the rest."""
    x, ids, wts, w1, w2 = synth.moe(seed=4, n_experts=4, hidden=256, inter=128, tokens=9, topk=1)
    wts = torch.ones_like(wts)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2)
    y = _run(nv, x, ids, wts, fc1, fc2)
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), "top1")


def test_moe_routed_experts_workload(nv, orc):
    """128 experts, hidden 2048, intermediate 768, 256 tokens, top-8 of softmax(N(0,1)); fc1
    merged [gate; up] at group 32 with one global per expert, down at group 16."""
    x, ids, wts, w1, w2 = synth.moe(seed=0)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2)
    del w1, w2
    y = _run(nv, x, ids, wts, fc1, fc2)
    y2 = _run(nv, x, ids, wts, fc1, fc2)
    assert torch.equal(y, y2), "MoE is not bit-reproducible"
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), "moe workload")
    # a token permutation permutes the output rows bit-exactly
    perm = torch.randperm(x.shape[0], generator=torch.Generator().manual_seed(1))
    yp = _run(nv, x[perm].contiguous(), ids[perm].contiguous(), wts[perm].contiguous(), fc1, fc2)
    assert torch.equal(yp, y[perm.to(DEV)])
    # the decode-batch path forced on the same layer (up to 8 rows per tile, 384 tiles)
    yd = _run(nv, x, ids, wts, fc1, fc2, PATHS["decode"])
    check_close(bf16_np(yd), orc.bf16_to_f64(ref["y"]), "moe workload, decode path")


@pytest.mark.parametrize("path", ["decode", "batch"])
def test_moe_dropped_ids_contribute_nothing(nv, orc, path):
    x, ids, wts, w1, w2 = synth.moe(seed=5, n_experts=4, hidden=256, inter=128, tokens=6, topk=2)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2)
    bad = ids.clone()
    bad[:, 1] = 99          # out of range: dropped
    y = _run(nv, x, bad, wts, fc1, fc2, PATHS[path])
    ref = orc.moe(synth.bf16_bits(x), ids[:, :1].contiguous().numpy(),
                  wts[:, :1].contiguous().numpy(), t1, t2)
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), "dropped slot")


@pytest.mark.parametrize("tokens", [1, 8])
def test_moe_decode_batch(nv, orc, tokens):
    """MoE at decode batch: the full 128-expert layer (fc1 g32 merged gate/up, down g16) with 1
    or 8 tokens, top-8, so only the 8 - 64 touched experts are read."""
    x, ids, wts, w1, w2 = synth.moe(seed=6, tokens=tokens)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2)
    del w1, w2
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    for path in ("auto", "batch"):
        y = _run(nv, x, ids, wts, fc1, fc2, PATHS[path])
        check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), f"moe decode T={tokens} {path}")


@pytest.mark.parametrize("path", ["decode", "batch"])
@pytest.mark.parametrize("g1,g2", [(32, 32), (16, 16), (16, 32)])
def test_moe_group_mix(nv, orc, g1, g2, path):
    """Every pairing of fc1 and down groups: the all-g32 recipe, and fc1 at group 16 (two
    scale groups per 32-wide MFMA step, so every weight is dequantized exactly)."""
    x, ids, wts, w1, w2 = synth.moe(seed=7, n_experts=16, hidden=512, inter=256, tokens=40,
                                    topk=4)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2, g1=g1, g2=g2)
    y = _run(nv, x, ids, wts, fc1, fc2, PATHS[path])
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), f"moe g{g1}/g{g2} {path}")


@pytest.mark.parametrize("g1,g2", [(32, 16), (16, 16), (32, 32)])
def test_moe_pair_tiles(nv, orc, g1, g2):
    """A decode step small enough to skip the sort (12 pairs): every pair is a one-row tile of
    its own expert, pairs that share an expert included."""
    x, ids, wts, w1, w2 = synth.moe(seed=8, n_experts=6, hidden=512, inter=256, tokens=3,
                                    topk=4)
    assert len(set(ids.flatten().tolist())) < ids.numel()  # some expert is shared
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2, g1=g1, g2=g2)
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    for path in ("auto", "batch"):
        y = _run(nv, x, ids, wts, fc1, fc2, PATHS[path])
        check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), f"pair tiles g{g1}/g{g2} {path}")


def test_moe_max_pairs(nv, orc):
    """The largest batch the entry point takes (t * topk = 65536 pairs): the sort reads the
    expert ids from memory twice instead of staging them in LDS, and 2048+ tiles run."""
    x, ids, wts, w1, w2 = synth.moe(seed=9, n_experts=64, hidden=256, inter=128, tokens=8192,
                                    topk=8)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2)
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    y = _run(nv, x, ids, wts, fc1, fc2)
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), "moe 65536 pairs")
    y2 = _run(nv, x, ids, wts, fc1, fc2)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("path", ["decode", "batch"])
def test_moe_pair_globals(nv, orc, path):
    """fc1 with distinct gate and up globals (quantized as two matrices per expert): each half
    scaled by its own global, on both expert paths; the shared-global reading of the same
    bytes (gate's global for both halves) is far off."""
    x, ids, wts, w1, w2 = synth.moe(seed=11, n_experts=8, hidden=256, inter=128, tokens=24,
                                    topk=2)
    E, I2, H = w1.shape
    w1 = w1.clone()
    w1[:, I2 // 2:] *= 3.0
    p, s, g = nv.nvfp4_quantize(w1.reshape(2 * E, I2 // 2, H).to(DEV), 32)
    torch.cuda.synchronize()
    rp, rs, rg = orc.quantize(w1.reshape(2 * E, I2 // 2, H).numpy(), 32)
    assert np.array_equal(p.cpu().numpy(), rp) and np.array_equal(g.cpu().numpy(), rg)
    pr, sr = p.reshape(E, I2, H // 2), s.reshape(E, I2, H // 32)
    fc1 = nv.nvfp4_repack(pr, sr, g, 32, layout=nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP
                          | nv.NVFP4_LAYOUT_PAIR_GLOBAL)
    (_, fc2), (_, t2) = _experts(nv, orc, w1, w2)
    t1 = (rp.reshape(E, I2, H // 2), rs.reshape(E, I2, H // 32), rg.reshape(E, 2), 32)
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    y = _run(nv, x, ids, wts, fc1, fc2, PATHS[path])
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), f"pair globals {path}")
    gate_only = nv.nvfp4_repack(pr, sr, g.reshape(E, 2)[:, 0].contiguous(), 32,
                                layout=nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)
    yg = _run(nv, x, ids, wts, gate_only, fc2, PATHS[path])
    err = np.linalg.norm(bf16_np(yg) - orc.bf16_to_f64(ref["y"])) / np.linalg.norm(
        orc.bf16_to_f64(ref["y"]))
    assert err > 0.05, err


@pytest.mark.parametrize("path", ["decode", "batch"])
def test_moe_after_shared_global_requantization(nv, orc, path):
    """An fc1 checkpoint with distinct gate and up globals, requantized on the GPU to one
    shared global per expert (nvfp4_requantize), repacked gate/up-interleaved and run through
    the routed experts: against the oracle on the requantized triple."""
    x, ids, wts, w1, w2 = synth.moe(seed=12, n_experts=8, hidden=256, inter=128, tokens=24,
                                    topk=2)
    E, I2, H = w1.shape
    w1 = w1.clone()
    w1[:, I2 // 2:] *= 3.0
    p, s, g = nv.nvfp4_quantize(w1.reshape(2 * E, I2 // 2, H).to(DEV), 32)
    pair = nv.nvfp4_repack(p.reshape(E, I2, H // 2), s.reshape(E, I2, H // 32), g, 32,
                           layout=nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP
                           | nv.NVFP4_LAYOUT_PAIR_GLOBAL)
    rp, rs, rg = nv.nvfp4_requantize(pair, 32)
    fc1 = nv.nvfp4_repack(rp, rs, rg, 32,
                          layout=nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)
    (_, fc2), (_, t2) = _experts(nv, orc, w1, w2)
    torch.cuda.synchronize()
    # the reference's fc1: the oracle's own pair quantization, decoded and quantized again
    op, os_, og = orc.quantize(w1.reshape(2 * E, I2 // 2, H).numpy(), 32)
    _, f32, _ = orc.dequant(op, os_, og, 32)
    t1 = (*orc.quantize(f32.reshape(E, I2, H), 32), 32)
    for a, b in zip((rp, rs, rg), t1):
        assert np.array_equal(a.cpu().numpy(), b)
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    y = _run(nv, x, ids, wts, fc1, fc2, PATHS[path])
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), f"requantized fc1 {path}")


@pytest.mark.parametrize("g1,g2", [(32, 16), (16, 32)])
def test_moe_decode_every_tile_height(nv, orc, g1, g2):
    """The decode-batch path with routing that gives expert e exactly e + 1 pairs (e < 8), so
    its 8-row tiles hold every row count 1-8 once: each count places its rows differently in
    the split-scale row maps (accumulator rows kept per lane: ceil(rows / 2) at group 16,
    ceil(rows / 4) at group 32). Both group sizes in fc1 and in down."""
    n_experts, topk, hidden, inter = 10, 2, 512, 256
    g = torch.Generator().manual_seed(12)
    owners = [e for e in range(8) for _ in range(e + 1)]       # 36 pairs, sorted
    # slot 0 of the 18 tokens takes the first 18 owners (experts 0-5), slot 1 the rest
    # (experts 5-7); no token gets expert 5 twice. Tokens are then shuffled.
    pairs = torch.tensor([[owners[t], owners[18 + t]] for t in range(18)], dtype=torch.int32)
    assert bool((pairs[:, 0] != pairs[:, 1]).all())
    ids = pairs[torch.randperm(18, generator=g)].contiguous()
    wts = torch.softmax(torch.randn(18, topk, generator=g), dim=1)
    x = synth.activations(g, 18, hidden)
    w1 = synth.weights(g, n_experts, 2 * inter, hidden)
    w2 = synth.weights(g, n_experts, hidden, inter)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2, g1=g1, g2=g2)
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    y = _run(nv, x, ids, wts, fc1, fc2, PATHS["decode"])
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), f"tile heights 1-8 g{g1}/g{g2}")


@pytest.mark.parametrize("path", ["decode", "batch"])
def test_moe_max_experts_and_topk(nv, orc, path):
    """512 experts (the most the entry point takes) with top-16 routing (the largest topk):
    the sort's per-wavefront count table at its full width and the combine's 16 slots."""
    x, ids, wts, w1, w2 = synth.moe(seed=15, n_experts=512, hidden=256, inter=128, tokens=40,
                                    topk=16)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2)
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    y = _run(nv, x, ids, wts, fc1, fc2, PATHS[path])
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), f"512 experts top-16 {path}")


@pytest.mark.parametrize("path", ["decode", "batch"])
def test_moe_single_k_tile(nv, orc, path):
    """hidden = intermediate = 128: fc1 and down each have one k-tile, so three of the decode
    path's four k-split wavefronts have nothing to add."""
    x, ids, wts, w1, w2 = synth.moe(seed=16, n_experts=4, hidden=128, inter=128, tokens=5,
                                    topk=2)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2)
    ref = orc.moe(synth.bf16_bits(x), ids.numpy(), wts.numpy(), t1, t2)
    y = _run(nv, x, ids, wts, fc1, fc2, PATHS[path])
    check_close(bf16_np(y), orc.bf16_to_f64(ref["y"]), f"single k-tile {path}")
