"""The attention path at other head counts: the share of one GPU when the heads are
split across GPUs (tensor parallelism over the independent KV heads), and the extreme
grouping ratios the kernels accept.

With the 8 KV heads split over 8 GPUs, each holds one KV head and its 6 query heads
(Hq = 6, Hkv = 1), its own pages and its 768 gate columns ("SGLang natively supports
Reflection's Beam": the attention projections, the gate included, are sharded under
tensor parallelism; "Reflection Beam 1.0 on vLLM", architecture section: 48 query heads
over 8 KV heads). Over 4 GPUs each holds Hq = 12, Hkv = 2. The kernels take the head
counts as parameters; these cases run the whole path (fused store, prefill, decode)
through the C ABI at those shapes and compare every output row with the fp64 oracle,
which reads the head counts off the tensor shapes."""

import pytest

import oracle.beam_oracle as O
import synth
from tests.gpu_util import assert_close_to_oracle, bits16, run_layer, say

pytestmark = pytest.mark.gpu

HEADS = [(6, 1), (12, 2), (16, 1), (8, 8)]


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


@pytest.mark.parametrize("heads", HEADS, ids=[f"hq{a}-hkv{b}" for a, b in HEADS])
@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_prefill_at_head_share(heads, kind, kv_dtype):
    say(f"case prefill heads={heads} kind={kind} dtype={kv_dtype}")
    call = synth.make_call([300, 77, 5], [1500, 77, 700], kind, kv_dtype, [61, heads[0], heads[1]],
                           heads=heads)
    ref = O.layer_call(call.oracle_inputs())["y"]
    d = run_layer(call, "prefill")
    assert_close_to_oracle(bits16(d["out"]), ref, kv_dtype, f"prefill {heads} {kind} {kv_dtype}")


# Many (sequence, KV head) pairs of short ragged sequences over several row tiles, as in
# a batched full-layer prefill: 200 new tokens x 6 heads = 1,200 rows = 5 row tiles for
# each of 64 pairs (320 workgroups, more than one round on 256 CUs); shorter sequences end
# inside their first or a middle tile.
MANY_PAIR_CASES = [((48, 8), [200, 150, 200, 37, 200, 180, 1, 200], [900, 150, 1300, 500, 200, 2000, 64, 777]),
               ((6, 1), [200] * 60 + [171, 1, 200, 90], [200 + 13 * i for i in range(64)])]


@pytest.mark.parametrize("case", MANY_PAIR_CASES, ids=["hq48-hkv8-8seq", "hq6-hkv1-64seq"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_prefill_many_pairs(case, kv_dtype):
    heads, q_lens, kv_lens = case
    say(f"case prefill many pairs heads={heads} seqs={len(q_lens)} dtype={kv_dtype}")
    call = synth.make_call(q_lens, kv_lens, "full", kv_dtype, [63, heads[0], len(q_lens)], heads=heads)
    ref = O.layer_call(call.oracle_inputs())["y"]
    d = run_layer(call, "prefill")
    assert_close_to_oracle(bits16(d["out"]), ref, kv_dtype, f"prefill many pairs {heads} {kv_dtype}")


@pytest.mark.parametrize("heads", HEADS, ids=[f"hq{a}-hkv{b}" for a, b in HEADS])
@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_decode_at_head_share(heads, kind, kv_dtype):
    say(f"case decode heads={heads} kind={kind} dtype={kv_dtype}")
    call = synth.make_call([1, 3, 8, 16], [5000, 700, 64, 2100], kind, kv_dtype,
                           [62, heads[0], heads[1]], heads=heads)
    ref = O.layer_call(call.oracle_inputs())["y"]
    d = run_layer(call, "decode")
    assert_close_to_oracle(bits16(d["out"]), ref, kv_dtype, f"decode {heads} {kind} {kv_dtype}")
