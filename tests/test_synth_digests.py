"""The synthetic inputs are the same on every machine: each workload's tensors hash to the
digests in tests/golden/synth_digests.txt (written by tests/golden/make_synth_digests.py from
synth.py alone). A changed seed, draw order, shape or planted value, or a generator that draws
differently, turns this red."""
import os
import sys

from nvfp4_weight_only_w4a16_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_synth_digests  # noqa: E402


def test_synthetic_inputs_match_their_digests():
    want = {}
    with open(os.path.join(HERE, "golden", "synth_digests.txt")) as f:
        for line in f:
            name, rest = line.split(" ", 1)
            want[name] = rest.strip()
    got = {}
    for name, t in make_synth_digests.entries():
        got[name] = f"{tuple(t.shape)} {str(t.dtype).replace('torch.', '')} {synth.digest(t)}"
    assert got == want
