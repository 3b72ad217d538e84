"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on seeded synthetic
inputs small enough for the oracle to finish in seconds but spanning several tiles,
ragged tails, many sequences, both layer kinds and both cache dtypes."""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from tests.gpu_util import (assert_close_to_oracle, bits16, ordered8, ordered16, run_attend,
                            run_kvwrite, run_layer, say, stage)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


# ------------------------------------------------------------------ fused Q/K prepare + KV store

@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_kvwrite_matches_oracle_and_touches_only_new_slots(kind, kv_dtype):
    say(f"case kvwrite kind={kind} dtype={kv_dtype}")
    call = synth.make_call([5, 64, 130, 1, 0], [5, 100, 700, 3000, 64], kind, kv_dtype, [21, 3])
    inp = call.oracle_inputs()
    ref = O.layer_call(inp, rows=[])
    d = stage(call)
    run_kvwrite(d)
    torch.cuda.synchronize()
    # q' within one bf16 ulp of the fp64 value (fp32 vs fp64 arithmetic before the single
    # rounding), or 2^-16 absolute where the two RoPE terms cancel and fp32's relative
    # error on the small result exceeds an ulp
    got_q, exp_q = bits16(d["q_out"]), ref["q_out"]
    dq = np.abs(ordered16(got_q) - ordered16(exp_q))
    gv, ev = O.bf16_bits_to_f64(got_q), O.bf16_bits_to_f64(exp_q)
    spacing = np.exp2(np.floor(np.log2(np.maximum(np.abs(ev), 2.0 ** -126))) - 7)
    worst = np.argmax(np.abs(gv - ev) / spacing)
    say(f"  q' ulp diff max {dq.max()}, exact {np.mean(dq == 0):.5f}, worst oracle value "
        f"{ev.flat[worst]:.4e} vs {gv.flat[worst]:.4e}")
    assert np.all(np.abs(gv - ev) <= spacing + 2.0 ** -16)
    assert np.mean(dq == 0) > 0.999
    seq, pos = ref["seq"], ref["pos"]
    page, slot = O.physical_slot(inp["block_table"], seq, pos)
    for name, before in (("k_cache", inp["k_cache"]), ("v_cache", inp["v_cache"])):
        after = d["cache"].k if name == "k_cache" else d["cache"].v
        after = after.cpu()
        after = (after.view(torch.int16).numpy().view(np.uint16) if kv_dtype == "bf16"
                 else after.numpy())
        written = np.zeros(after.shape[0:1] + after.shape[2:3], dtype=bool)
        written[page, slot] = True
        untouched = ~written[:, None, :, None].repeat(after.shape[1], 1).repeat(after.shape[3], 3)
        assert np.array_equal(after[untouched], before[untouched]), f"{name}: bytes outside new slots changed"
        got, exp = after[page, :, slot, :], ref[name][page, :, slot, :]
        if kv_dtype == "bf16":
            diff = np.abs(ordered16(got) - ordered16(exp))
        else:
            diff = np.abs(ordered8(got) - ordered8(exp))
        say(f"  {name}: new-slot diff max {diff.max()}, exact {np.mean(diff == 0):.5f}")
        if kv_dtype == "bf16" and name == "k_cache":
            gk, ek = O.bf16_bits_to_f64(got), O.bf16_bits_to_f64(exp)
            sk = np.exp2(np.floor(np.log2(np.maximum(np.abs(ek), 2.0 ** -126))) - 7)
            assert np.all(np.abs(gk - ek) <= sk + 2.0 ** -16)
        elif name == "v_cache":
            assert diff.max() == 0            # V: unchanged bits, or the code of the exact quotient
        else:
            assert diff.max() <= 1            # K: q/k' may differ by one bf16 ulp
        assert np.mean(diff == 0) > 0.99


def test_kvwrite_in_place_equals_out_of_place():
    say("case kvwrite in place")
    call = synth.make_call([40, 3], [40, 300], "swa", "bf16", [22, 0])
    d = stage(call)
    run_kvwrite(d)
    ref = d["q_out"].clone()
    d2 = stage(call)
    d2["q_out"] = d2["q"]
    run_kvwrite(d2)
    torch.cuda.synchronize()
    assert torch.equal(d2["q"].view(torch.int16), ref.view(torch.int16))


# ------------------------------------------------------------------ standalone gate

def test_head_gate_matches_oracle_and_switches_heads():
    from nope_gqa_attention_amd import beamattn as ba
    say("case head_gate")
    g = torch.Generator().manual_seed(5)
    N = 333
    attn = torch.randn(N, 48, 128, generator=g).bfloat16()
    gate = torch.randn(N, 6144, generator=g).bfloat16()
    bias = torch.randn(48, generator=g).bfloat16()
    bias[5] = -1e4
    bias[9] = 1e4
    layer = ba.layer_desc("full")
    out = torch.empty(N, 48, 128, dtype=torch.bfloat16, device="cuda")
    ba.beam_head_gate(layer, attn.cuda(), gate.cuda(), bias.cuda(), out)
    torch.cuda.synchronize()
    y = O.head_gate(O.bf16_bits_to_f64(bits16(attn)), bits16(gate), bits16(bias))
    got = O.bf16_bits_to_f64(bits16(out))
    # one bf16 rounding of an fp32 result
    assert np.all(np.abs(got - y) <= np.abs(y) * 2.0 ** -8 + 1e-30)
    assert np.all(got[:, 5, :] == 0.0)
    assert np.array_equal(bits16(out)[:, 9, :], bits16(attn)[:, 9, :])
    # in place
    a2 = attn.cuda()
    ba.beam_head_gate(layer, a2, gate.cuda(), bias.cuda(), a2)
    torch.cuda.synchronize()
    assert torch.equal(a2.view(torch.int16), out.view(torch.int16))


# ------------------------------------------------------------------ attention

PREFILL_CASES = [
    ("ragged", [1, 70, 300, 0, 17], [1, 200, 900, 50, 1500]),
    ("one-long", [777], [777]),
]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("name,q_lens,kv_lens", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_matches_oracle(kind, name, q_lens, kv_lens, kv_dtype):
    say(f"case prefill {name} kind={kind} kv={kv_dtype}")
    call = synth.make_call(q_lens, kv_lens, kind, kv_dtype, [23, len(q_lens)])
    ref = O.layer_call(call.oracle_inputs())
    d = run_layer(call, mode="prefill")
    assert_close_to_oracle(bits16(d["out"]), ref["y"], kv_dtype, f"prefill {name} {kind} {kv_dtype}")


@pytest.mark.parametrize("kind", ["swa", "full"])
def test_prefill_tiny_config_full_size(kind):
    """The tiny prefill workload at its real size: 1 x 1024 new tokens, no cache."""
    say(f"case config0 kind={kind}")
    call = synth.make_config(0, kind)
    ref = O.layer_call(call.oracle_inputs())
    d = run_layer(call, mode="prefill")
    assert_close_to_oracle(bits16(d["out"]), ref["y"], "bf16", f"config0 {kind}")


DECODE_CASES = [
    ("q1-short", [1, 1, 1], [1, 37, 700]),
    ("q1-split", [1, 1], [9000, 5003]),
    ("q3", [3, 3, 2], [3, 2000, 6000]),
    ("q8-split", [8], [20000]),
    ("q16", [16, 5], [16, 4100]),
    ("finished-seqs", [0, 2, 0, 1], [700, 3000, 64, 9000]),   # sequences with no new token
]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("name,q_lens,kv_lens", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_matches_oracle(kind, kv_dtype, name, q_lens, kv_lens):
    say(f"case decode {name} kind={kind} dtype={kv_dtype}")
    call = synth.make_call(q_lens, kv_lens, kind, kv_dtype, [24, len(q_lens), max(q_lens)])
    ref = O.layer_call(call.oracle_inputs())
    d = run_layer(call, mode="decode")
    assert_close_to_oracle(bits16(d["out"]), ref["y"], kv_dtype, f"decode {name} {kind} {kv_dtype}")


@pytest.mark.parametrize("kind", ["swa", "full"])
def test_decode_and_prefill_agree(kind):
    say(f"case decode-vs-prefill kind={kind}")
    call = synth.make_call([8, 1, 16], [3000, 800, 16], kind, "bf16", [25, 1])
    dp = run_layer(call, mode="prefill")
    dd = run_layer(call, mode="decode")
    a = O.bf16_bits_to_f64(bits16(dp["out"]))
    b = O.bf16_bits_to_f64(bits16(dd["out"]))
    say(f"  max diff {np.abs(a - b).max():.3e}")
    assert np.abs(a - b).max() <= 1.6e-2


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_physical_page_order_does_not_change_bits(mode):
    """Outputs depend only on the logical contents: permuting physical pages (and the
    block table with them) gives bit-identical results."""
    say(f"case page permutation mode={mode}")
    call = synth.make_call([4, 9], [3000, 700], "full", "bf16", [26, 2])
    d1 = run_layer(call, mode=mode)
    P = call.k_cache.shape[0]
    perm = np.random.default_rng(3).permutation(P)
    inv = np.argsort(perm)
    call.k_cache = call.k_cache[torch.from_numpy(inv)].contiguous()
    call.v_cache = call.v_cache[torch.from_numpy(inv)].contiguous()
    call.block_table = perm[call.block_table].astype(np.int32)
    d2 = run_layer(call, mode=mode)
    assert torch.equal(d1["out"].view(torch.int16), d2["out"].view(torch.int16))


def test_ungated_attention_then_standalone_gate_equals_fused():
    from nope_gqa_attention_amd import beamattn as ba
    say("case unfused gate")
    call = synth.make_call([50, 3], [50, 2000], "full", "bf16", [27, 1])
    d = stage(call)
    run_kvwrite(d)
    run_attend(d, mode="prefill", gate=False)
    ungated = d["out"].clone()
    run_attend(d, mode="prefill", gate=True)
    fused = d["out"].clone()
    sep = torch.empty_like(fused)
    ba.beam_head_gate(d["layer"].desc, ungated, d["gate"], d["gate_bias"], sep)
    torch.cuda.synchronize()
    a = O.bf16_bits_to_f64(bits16(fused))
    b = O.bf16_bits_to_f64(bits16(sep))
    # the unfused path rounds the attention output to bf16 once more
    assert np.abs(a - b).max() <= 2e-2


@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_ungated_attention_matches_oracle(kind, mode, kv_dtype):
    """gate = NULL: the attention output itself, o[t,h] of the oracle (no sigmoid)."""
    say(f"case ungated kind={kind} mode={mode} dtype={kv_dtype}")
    q_lens = [300, 77, 5] if mode == "prefill" else [1, 7, 16]
    call = synth.make_call(q_lens, [1500, 77, 700], kind, kv_dtype, [28, len(kind), len(mode)])
    ref = O.layer_call(call.oracle_inputs())["o"]
    d = stage(call)
    run_kvwrite(d)
    run_attend(d, mode=mode, gate=False)
    torch.cuda.synchronize()
    assert_close_to_oracle(bits16(d["out"]), ref, kv_dtype, f"ungated {kind} {mode} {kv_dtype}")


# ------------------------------------------------------------------ ABI errors launch nothing

def test_invalid_arguments_return_status_and_launch_nothing():
    from nope_gqa_attention_amd import beamattn as ba
    say("case abi errors")
    call = synth.make_call([4], [100], "full", "bf16", [28, 0])
    d = stage(call)
    sentinel = torch.full_like(d["out"], 7.0)
    d["out"].copy_(sentinel)
    bad = ba.layer_desc("full")
    bad.head_dim = 64
    with pytest.raises(ba.BeamError) as e:
        ba.beam_attn_prefill(bad, d["batch"], d["cache"], d["q"], d["gate"], d["gate_bias"], d["out"])
    assert e.value.status == ba.BEAM_ERR_INVALID_ARG and "head_dim" in str(e.value)
    fp8 = ba.DeviceCache(torch.zeros_like(d["cache"].k, dtype=torch.uint8), torch.zeros_like(d["cache"].v, dtype=torch.uint8), 0.1, 0.0)
    with pytest.raises(ba.BeamError) as e:
        ba.beam_attn_prefill(d["layer"].desc, d["batch"], fp8, d["q"], d["gate"], d["gate_bias"], d["out"])
    assert e.value.status == ba.BEAM_ERR_INVALID_ARG and "scale" in str(e.value)
    big = synth.make_call([20], [100], "full", "bf16", [28, 1])
    db = stage(big)
    with pytest.raises(ba.BeamError) as e:
        ba.beam_attn_decode(db["layer"].desc, db["batch"], db["cache"], db["q"], db["gate"], db["gate_bias"], db["out"], None)
    assert e.value.status == ba.BEAM_ERR_INVALID_ARG
    long = synth.make_call([1], [50000], "full", "bf16", [28, 2])
    dl = stage(long)
    dl["out"].fill_(7.0)
    need = ba.beam_attn_decode_workspace_bytes(dl["layer"].desc, 1, 1, 50000)
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ba.BeamError) as e:
        ba.beam_attn_decode(dl["layer"].desc, dl["batch"], dl["cache"], dl["q"], dl["gate"], dl["gate_bias"], dl["out"], small)
    assert e.value.status == ba.BEAM_ERR_WORKSPACE
    # q_out overlapping q without being the same buffer
    buf = torch.zeros(5 * 6144, dtype=torch.bfloat16, device="cuda")
    q_in = buf[:4 * 6144].view(4, 48, 128)
    q_out = buf[8:8 + 4 * 6144].view(4, 48, 128)
    with pytest.raises(ba.BeamError) as e:
        ba.beam_qknorm_rope_ssmax_kvwrite(d["layer"].desc, d["batch"], d["cache"], q_in, d["k"], d["v"],
                                          d["q_norm_w"], d["k_norm_w"], q_out)
    assert e.value.status == ba.BEAM_ERR_INVALID_ARG and "overlaps" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(d["out"], sentinel)
    assert bool((dl["out"] == 7.0).all())
    assert not bool(buf.any())
