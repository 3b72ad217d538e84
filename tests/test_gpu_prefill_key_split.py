"""Full-layer prefill with the key range of each row tile split between two wave streams
whose partial softmaxes merge in LDS, against the fp64 oracle, and against the same call
with whole key ranges.

The library picks the split from the grid size; BEAMATTN_PREFILL_KEY_SPLIT=1 / 0 forces
it either way, so both paths run on the same inputs here. The batch holds the cases where
the two streams' tile counts differ: one key tile (the first stream gets none), two tiles
with a tail (one each, the second masked), odd and even counts, a sequence ending inside
its first row tile, and a row tile that is not full. The result is unique ("Reflection
Beam 1.0 on vLLM", section "Attention: sliding-window layers plus NoPE full-attention
layers": every token attends to all earlier positions), whichever stream saw which key."""

import pytest
import torch

import oracle.beam_oracle as O
import synth
from tests.gpu_util import assert_close_to_oracle, bits16, run_layer, say

pytestmark = pytest.mark.gpu

CASES = [
    ((6, 1), [1, 64, 65, 300, 7, 129], [1, 64, 1100, 2100, 70, 4000]),
    ((48, 8), [3, 40, 1, 200], [3, 1500, 64, 2113]),
]


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


@pytest.mark.parametrize("case", CASES, ids=["hq6-hkv1", "hq48-hkv8"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_key_split_prefill_matches_oracle_and_whole_ranges(case, kv_dtype, monkeypatch):
    heads, q_lens, kv_lens = case
    say(f"case prefill key split heads={heads} dtype={kv_dtype}")
    call = synth.make_call(q_lens, kv_lens, "full", kv_dtype, [71, heads[0], len(q_lens)], heads=heads)
    ref = O.layer_call(call.oracle_inputs())["y"]
    outs = {}
    for mode in ("1", "0"):
        monkeypatch.setenv("BEAMATTN_PREFILL_KEY_SPLIT", mode)
        d = run_layer(call, "prefill")
        outs[mode] = d["out"].clone()
        assert_close_to_oracle(bits16(d["out"]), ref, kv_dtype,
                               f"prefill split={mode} {heads} {kv_dtype}")
    # the two paths add the same terms in different orders, so some bf16 outputs differ:
    # evidence that the forced split really took the other path
    differ = int((outs["1"].view(torch.int16) != outs["0"].view(torch.int16)).sum())
    say(f"  outputs differing between the paths: {differ} of {outs['1'].numel()}")
    assert differ > 0, "split and whole-range prefill gave identical bits everywhere"
