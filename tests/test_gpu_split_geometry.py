"""Decode results do not depend on how the keys are split.

The host bounds of a decode call (max_q_len, max_kv_len) choose its split geometry:
keys per split, 16/32/48-row chunks, 4- or 12-wave workgroups, and whether the
log-sum-exp merge kernel runs at all. The result is the same softmax-weighted sum
whatever the split ("Reflection Beam 1.0 on vLLM", section "Attention: sliding-window
layers plus NoPE full-attention layers", defines it; splitting only reorders fp32
sums), so one batch run under several bounds must agree with itself far more tightly
than with the fp64 oracle: at most one bf16 step apart, almost always bit-equal, and
bit-equal run to run under one geometry. Prefill over the same tokens (another entry
point, another kernel) must meet the oracle's tolerance too.
"""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from nope_gqa_attention_amd import beamattn as ba
from tests.gpu_util import (assert_close_to_oracle, bits16, ordered16, run_attend, run_kvwrite,
                            say, stage)

pytestmark = pytest.mark.gpu

# (name, kind, q_lens, kv_lens, host bounds [(max_q_len or None, max_kv_len or None), ...])
CASES = [
    ("full-multi", "full", [1, 3, 2], [9000, 2500, 700],
     [(None, None), (8, None), (16, None), (None, 50_000), (16, 300_000)]),
    ("full-short", "full", [1, 2, 1], [700, 300, 650],
     [(None, None), (None, 50_000), (16, None), (16, 120_000)]),
    ("swa", "swa", [1, 4, 2], [9000, 2500, 700],
     [(None, None), (16, None), (None, 1_000_000)]),
    ("full-one-seq", "full", [8], [40_000], [(None, None), (16, None), (None, 1_048_584)]),
]


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


def _with_bounds(call, max_q_len, max_kv_len):
    pages = -(-(max_kv_len or call.max_kv_len) // 64)
    bt = np.zeros((call.num_seqs, max(pages, call.block_table.shape[1])), dtype=np.int32)
    bt[:, :call.block_table.shape[1]] = call.block_table    # columns past a sequence are never read
    b = ba.DeviceBatch(call.q_start, call.kv_len, bt, "cuda")
    if max_q_len:
        b.max_q_len = max_q_len
        b.num_tokens = call.num_tokens     # rows stay the real tokens (no padding rows)
    if max_kv_len:
        b.max_kv_len = max_kv_len
    return b


def _agreement(a_bits, b_bits, what, check=True):
    """Agreement of two bf16 outputs of the same call. Splitting changes the fp32 order of
    the sums and the running maxima against which each softmax weight is rounded to bf16
    for the P.V product, so two geometries differ by rounding only: at most one bf16 step
    at the larger of the two magnitudes, or at 2^-4 where the output is smaller (sums that
    cancel), and a mean difference far inside the oracle's mean tolerance."""
    a, b = O.bf16_bits_to_f64(a_bits), O.bf16_bits_to_f64(b_bits)
    steps = np.abs(ordered16(a_bits) - ordered16(b_bits))
    mag = np.maximum(np.maximum(np.abs(a), np.abs(b)), 2.0 ** -4)
    step = np.exp2(np.floor(np.log2(mag)) - 7)
    d = np.abs(a - b)
    say(f"  {what}: bit-equal {np.mean(steps == 0):.5f}, max diff in bf16 steps at max(|y|, 2^-4) "
        f"{(d / step).max():.3f}, max-abs diff {d.max():.3e}, mean-abs {d.mean():.3e}")
    if check:
        assert np.all(d <= step)
        assert d.mean() <= 1e-4


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("name,kind,q_lens,kv_lens,bounds", CASES, ids=[c[0] for c in CASES])
def test_decode_agrees_across_split_geometries(name, kind, q_lens, kv_lens, bounds, kv_dtype):
    say(f"case split geometry {name} kind={kind} kv={kv_dtype}")
    call = synth.make_call(q_lens, kv_lens, kind, kv_dtype, [71, len(q_lens)])
    ref = O.layer_call(call.oracle_inputs())
    d = stage(call)
    run_kvwrite(d)
    outs = []
    for mq, mk in bounds:
        d["batch"] = _with_bounds(call, mq, mk)
        ws = d["layer"].workspace(d["batch"])
        say(f"  bounds max_q_len={d['batch'].max_q_len} max_kv_len={d['batch'].max_kv_len}: "
            f"workspace {0 if ws is None else ws.numel()} bytes")
        run_attend(d, "decode")
        torch.cuda.synchronize()
        outs.append(bits16(d["out"]))
        assert_close_to_oracle(outs[-1], ref["y"], kv_dtype, f"{name} bounds {mq},{mk}")
        run_attend(d, "decode")
        torch.cuda.synchronize()
        assert np.array_equal(bits16(d["out"]), outs[-1]), "not reproducible under one geometry"
    for i, o in enumerate(outs[1:], 1):
        _agreement(o, outs[0], f"geometry {i} vs 0")
    # prefill over the same tokens: another kernel, the same definition
    d["batch"] = _with_bounds(call, None, None)
    run_attend(d, "prefill")
    torch.cuda.synchronize()
    pf = bits16(d["out"])
    assert_close_to_oracle(pf, ref["y"], kv_dtype, f"{name} prefill")
    _agreement(pf, outs[0], "prefill vs decode", check=False)
