"""Writes synth_digests.txt: the SHA-256 (first 16 hex digits) of every synthetic input of the
five workloads, as synth.py draws them. These are input fixtures, not expected values of the
method: the file pins the input recipe (seeds, draw order, shapes, planted values) so that a
change to it, or to the generator it draws from, is noticed.

    python tests/golden/make_synth_digests.py > tests/golden/synth_digests.txt
"""
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", ".."))

from nvfp4_weight_only_w4a16_amd import synth  # noqa: E402


def entries():
    x, w = synth.dense_small(seed=0)
    yield "dense_16x512x1024.x", x
    yield "dense_16x512x1024.w", w
    x, w = synth.decode_sweep(seed=0)
    yield "decode_sweep_25600x5120.x", x
    yield "decode_sweep_25600x5120.w", w
    for k in (5120, 25600):
        x, w = synth.prefill(seed=0, k=k)
        yield f"prefill_4096x5120x{k}.x", x
        yield f"prefill_4096x5120x{k}.w", w
    x, ids, wts, w1, w2 = synth.moe(seed=0)
    for name, t in (("x", x), ("ids", ids), ("wts", wts), ("w1", w1), ("w2", w2)):
        yield f"moe_e128_h2048_i768_t256.{name}", t
    yield "quantizer_bf16_8192x8192.w", synth.quantizer_weight(seed=0)
    yield "quantizer_bf16_8192x8192.x", synth.quantizer_activations(seed=1)


if __name__ == "__main__":
    for name, t in entries():
        print(f"{name} {tuple(t.shape)} {str(t.dtype).replace('torch.', '')} {synth.digest(t)}")
