"""A seeded sweep of random call shapes through the C ABI against the fp64 oracle.

Each case draws, from its own seed: the number of sequences, the new-token count and the
key count of each sequence (cached keys before the new ones, from none to a few thousand,
with page boundaries and the 512-key window edge hit often), the layer kind, the cache
dtype and the entry point (prefill for any new-token count, decode for 1..16). Every
output row is compared with the oracle at the cache dtype's tolerance. The sweep covers
combinations the named cases do not: empty sequences next to long ones, blocks that end
exactly on a page or window boundary, and mixed block lengths in one decode call."""

import numpy as np
import pytest

import oracle.beam_oracle as O
import synth
from tests.gpu_util import assert_close_to_oracle, bits16, run_layer, say

pytestmark = pytest.mark.gpu

NUM_CASES = 24
EDGES = [0, 1, 63, 64, 65, 127, 128, 511, 512, 513, 575, 576]


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


def draw_case(i: int):
    rng = np.random.default_rng([71, i])
    mode = "decode" if i % 2 else "prefill"
    kind = ("swa", "full")[(i // 2) % 2]
    kv_dtype = ("bf16", "fp8")[(i // 4) % 2]
    B = int(rng.integers(1, 6))
    q_lens, kv_lens = [], []
    for _ in range(B):
        if mode == "decode":
            n = int(rng.integers(1, 17))
        else:
            n = int(rng.choice([0, 1, int(rng.integers(2, 64)), int(rng.integers(64, 400))]))
        cached = int(rng.choice([int(rng.choice(EDGES)), int(rng.integers(0, 3000))]))
        q_lens.append(n)
        kv_lens.append(n + cached)
    if mode == "decode" and max(q_lens) == 0:
        q_lens[0] = 1
        kv_lens[0] += 1
    return mode, kind, kv_dtype, q_lens, kv_lens


@pytest.mark.parametrize("i", range(NUM_CASES))
def test_random_shape_matches_oracle(i):
    mode, kind, kv_dtype, q_lens, kv_lens = draw_case(i)
    say(f"case random #{i}: {mode} {kind} {kv_dtype} q_lens={q_lens} kv_lens={kv_lens}")
    if sum(q_lens) == 0:
        pytest.skip("no new tokens drawn")
    call = synth.make_call(q_lens, kv_lens, kind, kv_dtype, [72, i])
    ref = O.layer_call(call.oracle_inputs())
    d = run_layer(call, mode=mode)
    assert_close_to_oracle(bits16(d["out"]), ref["y"], kv_dtype, f"random #{i}")
