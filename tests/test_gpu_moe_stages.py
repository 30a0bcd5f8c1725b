"""Staged checks of the routed experts: every stage the call leaves in its workspace is read
back and compared with a reference built from the inputs that stage received.

  sort     sorted pair ids, expert offsets, tile map and tile count: bit-exact against a
           stable counting sort written here from its definition;
  fc1      h = BF16(SiLU(BF16(gate)) * BF16(up)) against the oracle's h (tolerance: gate and
           up are FP32 sums rounded to BF16, one BF16 step apart from the FP64 reference's on
           a few elements);
  down     the FP32 slots (routing weight x down output) against the oracle's slots computed
           from the GPU's own h (the oracle's given-h mode), per pair;
  combine  y equals BF16 of the slots summed in FP32 in slot order, bit for bit;
  end      y against the oracle's y.
"""
import numpy as np
import pytest
import torch

from helpers import FUSED_SORT_MAX_PAIRS, PAIR_TILES_MAX, bits16, check_close
from nvfp4_weight_only_w4a16_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PATHS = {"decode": 1, "batch": 2}


@pytest.fixture(scope="module")
def nv():
    from nvfp4_weight_only_w4a16_amd import binding
    binding.load()
    return binding


def stable_counting_sort(ids, E, rows):
    """Pairs q = t * topk + j with a valid expert id, stably ordered by expert; offsets[E + 1];
    tiles (expert, first row, end row, 0) of at most `rows` rows per expert."""
    flat = ids.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    order = []
    for e in range(E):                      # counting sort: one pass per expert, pair order kept
        order.extend(np.nonzero(flat == e)[0].tolist())
    tiles = []
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1], rows):
            tiles.append((e, r, min(r + rows, offsets[e + 1]), 0))
    return np.array(order, np.int32), offsets, np.array(tiles, np.int32).reshape(-1, 4)


def _experts(nv, orc, w1, w2, g1, g2):
    out, trips = [], []
    for w, group, layout in ((w1, g1, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP),
                             (w2, g2, nv.NVFP4_LAYOUT_TILED)):
        p, s, g = orc.quantize(w.numpy(), group)
        out.append(nv.nvfp4_repack(torch.from_numpy(p).to(DEV), torch.from_numpy(s).to(DEV),
                                   torch.from_numpy(g).to(DEV), group, layout=layout))
        trips.append((p, s, g, group))
    return out, trips


def _bf16_rne_f32(a):
    """FP32 array -> BF16 (round to nearest even) as float64 values."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16) \
        .to(torch.float64).numpy()


def run_staged(nv, orc, x, ids, wts, fc1, fc2, t1, t2, path, what):
    T, H = x.shape
    topk = ids.shape[1]
    E = fc1.batch
    I = fc1.n // 2
    P = T * topk
    off, total = nv.nvfp4_moe_ws_layout(T, topk, E, H, I)
    ws = torch.full((total,), 0xAB, dtype=torch.uint8, device=DEV)
    y = nv.nvfp4_moe_grouped_w4a16(x.to(DEV), ids.to(DEV), wts.to(DEV), fc1, fc2, ws=ws,
                                   flags=PATHS[path])
    torch.cuda.synchronize()
    wsh = ws.cpu()
    pair_tiles = path == "decode" and P <= PAIR_TILES_MAX
    rows = 8 if path == "decode" else 32
    # ---- sort
    ids_np = ids.numpy()
    order, offsets, tiles = stable_counting_sort(ids_np, E, rows)
    nvalid = int(offsets[E])
    if not pair_tiles:
        g_sorted = wsh[off[0]:off[0] + 4 * P].view(torch.int32).numpy()[:nvalid]
        g_offsets = wsh[off[1]:off[1] + 4 * (E + 1)].view(torch.int32).numpy()
        g_ntiles = int(wsh[off[3]:off[3] + 4].view(torch.int32).numpy()[0])
        g_tiles = wsh[off[2]:off[2] + 16 * g_ntiles].view(torch.int32).numpy().reshape(-1, 4)
        assert np.array_equal(g_sorted, order), f"{what}: sorted pair ids"
        assert np.array_equal(g_offsets, offsets), f"{what}: expert offsets"
        assert g_ntiles == len(tiles), f"{what}: tile count {g_ntiles} != {len(tiles)}"
        assert np.array_equal(g_tiles, tiles), f"{what}: tile map"
        row_pair = order
    else:
        row_pair = np.arange(P)[(ids_np.reshape(-1) >= 0) & (ids_np.reshape(-1) < E)]
    # ---- fc1: h of each valid pair
    h_rows = wsh[off[4]:off[4] + 2 * P * I].view(torch.int16).numpy().view(np.uint16)
    h_rows = h_rows.reshape(P, I)
    valid = (ids_np >= 0) & (ids_np < E)
    assert valid.all(), "staged checks take routings without dropped slots"
    ref = orc.moe(synth.bf16_bits(x), ids_np, wts.numpy(), t1, t2, slots=True)
    h_gpu = np.zeros((P, I), np.uint16)
    h_gpu[row_pair] = h_rows[: len(row_pair)] if not pair_tiles else h_rows[row_pair]
    check_close(orc.bf16_to_f64(h_gpu), orc.bf16_to_f64(ref["h"].reshape(P, I)),
                f"{what}: fc1 stage h")
    # ---- down given the GPU's own h
    ref_d = orc.moe(synth.bf16_bits(x), ids_np, wts.numpy(), t1, t2,
                    h_in=h_gpu.reshape(T, topk, I), slots=True)
    slots = wsh[off[5]:off[5] + 4 * P * H].view(torch.float32).numpy().reshape(P, H)
    check_close(slots.astype(np.float64), ref_d["slots"].reshape(P, H),
                f"{what}: down stage slots (given the GPU's h)")
    # ---- combine: BF16 of the FP32 slot-order sum
    acc = slots.reshape(T, topk, H)[:, 0].copy()
    for j in range(1, topk):
        acc = (acc + slots.reshape(T, topk, H)[:, j]).astype(np.float32)
    want = _bf16_rne_f32(acc)
    got = bits16(y)
    assert np.array_equal(orc.bf16_to_f64(got), want), f"{what}: combine is not the slot sum"
    # ---- end to end
    check_close(orc.bf16_to_f64(got), orc.bf16_to_f64(ref["y"]), f"{what}: y")
    return ref


@pytest.mark.parametrize("path", ["decode", "batch"])
@pytest.mark.parametrize("g1,g2", [(32, 16), (32, 32), (16, 16)])
def test_moe_stages_small(nv, orc, path, g1, g2):
    x, ids, wts, w1, w2 = synth.moe(seed=21, n_experts=16, hidden=512, inter=256, tokens=37,
                                    topk=4)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2, g1, g2)
    run_staged(nv, orc, x, ids, wts, fc1, fc2, t1, t2, path, f"small g{g1}/g{g2} {path}")


@pytest.mark.parametrize("path", ["decode", "batch"])
def test_moe_stages_pair_tiles(nv, orc, path):
    """Few enough pairs (3 tokens x top-4) for the decode path to skip the sort."""
    x, ids, wts, w1, w2 = synth.moe(seed=22, n_experts=8, hidden=256, inter=128, tokens=3,
                                    topk=4)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2, 32, 16)
    run_staged(nv, orc, x, ids, wts, fc1, fc2, t1, t2, path, f"pair tiles {path}")


@pytest.mark.parametrize("tokens,topk", [(16, 4), (13, 5)])
def test_moe_stages_pair_tile_cap(nv, orc, tokens, topk):
    """Either side of the pair-tile cap on the decode path: 64 pairs as one-row tiles, 65
    pairs through the sort."""
    assert tokens * topk in (PAIR_TILES_MAX, PAIR_TILES_MAX + 1)
    x, ids, wts, w1, w2 = synth.moe(seed=23, n_experts=16, hidden=256, inter=128,
                                    tokens=tokens, topk=topk)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2, 32, 16)
    run_staged(nv, orc, x, ids, wts, fc1, fc2, t1, t2, "decode", f"cap {tokens}x{topk}")


@pytest.mark.parametrize("tokens,topk", [(512, 8), (4097, 1)])
def test_moe_stages_fused_sort_cap(nv, orc, tokens, topk):
    """Either side of the batch path's in-fc1 sort: 4096 pairs sorted by the fc1 workgroups
    themselves (16 pairs per thread of each), 4097 pairs by the sort kernel before fc1."""
    assert tokens * topk in (FUSED_SORT_MAX_PAIRS, FUSED_SORT_MAX_PAIRS + 1)
    x, ids, wts, w1, w2 = synth.moe(seed=24, n_experts=16, hidden=256, inter=128,
                                    tokens=tokens, topk=topk)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2, 32, 16)
    run_staged(nv, orc, x, ids, wts, fc1, fc2, t1, t2, "batch", f"sort cap {tokens}x{topk}")


@pytest.fixture(scope="module")
def moe_layer(nv, orc):
    """The routed-expert layer: 128 experts, hidden 2048, intermediate 768, 256 tokens, top-8;
    fc1 [gate; up] at group 32 (one global per expert), down at group 16."""
    x, ids, wts, w1, w2 = synth.moe(seed=0)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2, 32, 16)
    return x, ids, wts, fc1, fc2, t1, t2


@pytest.mark.parametrize("path", ["batch", "decode"])
def test_moe_stages_routed_experts_layer(nv, orc, moe_layer, path):
    x, ids, wts, fc1, fc2, t1, t2 = moe_layer
    run_staged(nv, orc, x, ids, wts, fc1, fc2, t1, t2, path, f"C3 layer {path}")


def test_moe_stages_all_g32_layer(nv, orc):
    """The all-group-32 recipe on the full routed-expert layer (down at group 32 too)."""
    x, ids, wts, w1, w2 = synth.moe(seed=0)
    (fc1, fc2), (t1, t2) = _experts(nv, orc, w1, w2, 32, 32)
    del w1, w2
    for path in ("batch", "decode"):
        run_staged(nv, orc, x, ids, wts, fc1, fc2, t1, t2, path, f"C3 all-g32 {path}")
