"""Layers at other constants than the model's: sliding windows other than 512 keys,
other RoPE, RMSNorm, SSMax and softmax-scale constants, and per-head norm weights.

The layer descriptor carries the window as a parameter; the pages fix it at 512 keys for
this model ("Reflection Beam 1.0 on vLLM", section "Attention: sliding-window layers plus
NoPE full-attention layers"), and the kernels take it at run time (masks at the window
start, the first key tile a row tile visits, the decode split range). These cases run
prefill and decode at windows of 1 (each token sees only itself), 64 (one page), 200 (not
a page multiple), 1,000 and 2^20 (wider than any context: causal attention with RoPE)
against the oracle at the same window, whose visibility rule is pinned at these lengths
against the transformers library's sliding-window mask."""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from tests.gpu_util import assert_close_to_oracle, bits16, ordered16, run_attend, run_kvwrite, say, stage

pytestmark = pytest.mark.gpu

WINDOWS = [1, 64, 200, 1000, 1 << 20]


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_sliding_layer_at_window(window, mode):
    from nope_gqa_attention_amd.layer import HybridAttention

    kv_dtype = "fp8" if window == 200 else "bf16"
    q_lens = [300, 77, 5] if mode == "prefill" else [1, 7, 16]
    kv_lens = [1500, 77, 700] if mode == "prefill" else [2000, 77, 700]
    say(f"case sliding window={window} mode={mode} dtype={kv_dtype}")
    call = synth.make_call(q_lens, kv_lens, "swa", kv_dtype, [95, window, len(mode)], window=window)
    inp = call.oracle_inputs()
    inp["window"] = window
    ref = O.layer_call(inp)["y"]
    d = stage(call)
    d["layer"] = HybridAttention("swa", window=window)
    run_kvwrite(d)
    run_attend(d, mode)
    torch.cuda.synchronize()
    assert_close_to_oracle(bits16(d["out"]), ref, kv_dtype, f"window {window} {mode}")


# Other layer constants than the model's: the descriptor carries them all, and the kernels
# read them at run time (RoPE frequencies, the RMS epsilon, the SSMax base and exponent,
# the softmax scale).
CONSTS = {"rope_theta": 5.0e5, "rms_eps": 1.0e-3, "ssmax_base": 4096.0, "ssmax_exponent": 0.25,
          "sm_scale": 0.0625}


@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_layer_at_other_constants(kind, mode):
    from nope_gqa_attention_amd.layer import HybridAttention

    q_lens = [300, 77, 5] if mode == "prefill" else [1, 7, 16]
    kv_lens = [1500, 77, 700] if mode == "prefill" else [2000, 77, 700]
    say(f"case constants kind={kind} mode={mode} {CONSTS}")
    call = synth.make_call(q_lens, kv_lens, kind, "bf16", [96, len(kind), len(mode)])
    inp = call.oracle_inputs()
    inp.update(CONSTS)
    res = O.layer_call(inp)
    d = stage(call)
    d["layer"] = HybridAttention(kind, **CONSTS)
    run_kvwrite(d)
    run_attend(d, mode)
    torch.cuda.synchronize()
    # q' within one bf16 step of the oracle's, then the layer output within tolerance
    _assert_within_one_step(bits16(d["q_out"]), res["q_out"])
    assert_close_to_oracle(bits16(d["out"]), res["y"], "bf16", f"constants {kind} {mode}")


# One norm weight vector per head ([heads][128] with a head stride, here padded to 136
# elements) instead of one shared [128] vector: the fused store reads head h's weights
# at h * norm_w_head_stride.
@pytest.mark.parametrize("kind", ["swa", "full"])
def test_kvwrite_with_per_head_norm_weights(kind):
    from nope_gqa_attention_amd import beamattn as ba

    say(f"case per-head norm weights kind={kind}")
    call = synth.make_call([5, 64, 130], [5, 100, 700], kind, "bf16", [97, len(kind)])
    gen = torch.Generator().manual_seed(970 + len(kind))
    qw = (1.0 + 0.1 * torch.randn(synth.HQ, 136, generator=gen)).bfloat16()
    kw = (1.0 + 0.1 * torch.randn(synth.HKV, 136, generator=gen)).bfloat16()
    inp = call.oracle_inputs()
    inp["q_norm_w"] = bits16(qw[:, :128])
    inp["k_norm_w"] = bits16(kw[:, :128])
    ref = O.layer_call(inp, rows=[])
    d = stage(call)
    ba.beam_qknorm_rope_ssmax_kvwrite(d["layer"].desc, d["batch"], d["cache"], d["q"], d["k"], d["v"],
                                      qw.cuda(), kw.cuda(), d["q_out"], norm_w_head_stride=136)
    torch.cuda.synchronize()
    seq, pos = ref["seq"], ref["pos"]
    page, slot = O.physical_slot(inp["block_table"], seq, pos)
    kc = d["cache"].k.cpu().view(torch.int16).numpy().view(np.uint16)
    _assert_within_one_step(bits16(d["q_out"]), ref["q_out"])
    _assert_within_one_step(kc[page, :, slot, :], ref["k_cache"][page, :, slot, :])


def _assert_within_one_step(got_bits, exp_bits):
    """One bf16 ulp of the fp64 value, or 2^-16 absolute where two RoPE terms cancel;
    at least 99% bit-equal."""
    gv, ev = O.bf16_bits_to_f64(got_bits), O.bf16_bits_to_f64(exp_bits)
    spacing = np.exp2(np.floor(np.log2(np.maximum(np.abs(ev), 2.0 ** -126))) - 7)
    assert np.all(np.abs(gv - ev) <= spacing + 2.0 ** -16)
    assert np.mean(ordered16(got_bits) == ordered16(exp_bits)) > 0.99
