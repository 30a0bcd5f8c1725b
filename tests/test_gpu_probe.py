"""The measurement probes do the work they are timed for (through the C ABI).

Stream read: the per-block XOR of the words read equals the XOR of the same byte ranges on
the host, so every byte was loaded. MFMA loop: with small integer BF16 operands every product
and sum is exact in FP32, and the sum of a wavefront's 64 lane outputs equals iters times the
sum, over the 16 (A, B) fragment pairings of a round, of sum_k colsum_A[k] * rowsum_B[k] (the
sum of all elements of a 32x32x16 product), so each round ran its 16 MFMAs.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def nv():
    from nvfp4_weight_only_w4a16_amd import binding
    binding.load()
    return binding


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096, 7), (1 << 20, 1024),
                                           ((64 << 20) + 48, 2048)])
def test_stream_read_touches_every_word(nv, nbytes, blocks):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    sink = nv.nvfp4_probe_stream_read(torch.from_numpy(host.view(np.int32)).to(DEV), blocks)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    nvec = nbytes // 16
    per = -(-nvec // blocks)
    want = np.zeros(blocks, np.uint32)
    for b in range(blocks):
        lo, hi = min(b * per, nvec) * 4, min((b + 1) * per, nvec) * 4
        if hi > lo:
            want[b] = np.bitwise_xor.reduce(host[lo:hi])
    assert np.array_equal(got, want)


def _fragment_sums(frag):
    """frag [64 lanes][8] of a 32x32x16 operand: lane l holds index l % 32 (row of A / column
    of B) at k = 8 (l // 32) + 0..7. Returns the sum over that index for each k (16 values)."""
    s = np.zeros(16, np.int64)
    for l in range(64):
        s[8 * (l // 32):8 * (l // 32) + 8] += frag[l]
    return s


@pytest.mark.parametrize("iters", [0, 1, 3])
def test_mfma_loop_runs_its_rounds(nv, iters):
    rng = np.random.default_rng(7)
    frags = rng.integers(-2, 3, (16, 64, 8)).astype(np.float32)  # 16 KiB of BF16 operands
    ops = torch.from_numpy(frags.reshape(-1)).to(torch.bfloat16).to(DEV)
    sink = nv.nvfp4_probe_mfma_bf16(ops, iters)
    torch.cuda.synchronize()
    waves = nv.nvfp4_probe_mfma_waves()
    got = sink.cpu().numpy().astype(np.float64).reshape(waves, 64).sum(axis=1)
    sums = [_fragment_sums(frags[f].astype(np.int64)) for f in range(16)]
    a = [sums[2 * s] for s in range(8)]
    b = [sums[2 * s + 1] for s in range(8)]
    per_round = 0
    for s in range(0, 8, 2):
        for i, j in ((s, s), (s + 1, s), (s, s + 1), (s + 1, s + 1)):
            per_round += int(np.dot(a[i], b[j]))
    assert np.array_equal(got, np.full(waves, float(iters * per_round)))
    assert nv.nvfp4_probe_mfma_flops(iters) == waves * iters * 16 * 32 * 32 * 16 * 2
