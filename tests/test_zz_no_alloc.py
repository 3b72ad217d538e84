"""The allocation-free decode entry point (beam_attn_decode_noalloc) against the
workspace one (beam_attn_decode), through the C ABI.

Both run the same kernels on the same split geometry, so their outputs must be equal bit
for bit; the first case is also checked against the fp64 oracle. Two calls in a row on
the shared per-device scratch, the second over a smaller batch (so stale partials of the
first call sit in the scratch), then bounds that need more scratch than the array holds,
which must be refused before anything is launched."""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from nope_gqa_attention_amd import beamattn as ba
from tests.gpu_util import assert_close_to_oracle, bits16, run_attend, run_kvwrite, say, stage

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


def _noalloc(d, out):
    ba.beam_attn_decode_noalloc(d["layer"].desc, d["batch"], d["cache"], d["q_out"], d["gate"],
                                d["gate_bias"], out)


CALLS = [  # (name, kind, kv dtype, q_lens, kv_lens)
    ("large", "full", "fp8", [1, 3, 8, 2], [30000, 9000, 120000, 700]),
    ("smaller", "full", "fp8", [2, 1], [5000, 800]),
    ("bf16", "full", "bf16", [1], [100000]),
    ("swa", "swa", "bf16", [4, 1], [3000, 600]),
]


def test_noalloc_decode_equals_workspace_decode_on_consecutive_calls():
    for i, (name, kind, kv_dtype, q_lens, kv_lens) in enumerate(CALLS):
        say(f"case noalloc decode {name} kind={kind} kv={kv_dtype} q_lens={q_lens} kv_lens={kv_lens}")
        call = synth.make_call(q_lens, kv_lens, kind, kv_dtype, [91, i])
        d = stage(call)
        run_kvwrite(d)
        run_attend(d, "decode")               # the workspace entry point
        ref = d["out"].clone()
        out = torch.full_like(d["out"], float("nan"))
        _noalloc(d, out)
        torch.cuda.synchronize()
        need = ba.beam_attn_decode_workspace_bytes(d["layer"].desc, d["batch"].num_seqs,
                                                   d["batch"].max_q_len, d["batch"].max_kv_len)
        say(f"  workspace need {need} bytes; outputs bit-equal: "
            f"{torch.equal(out.view(torch.int16), ref.view(torch.int16))}")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        if i == 0:
            assert need > 0
            y = O.layer_call(call.oracle_inputs())["y"]
            assert_close_to_oracle(bits16(out), y, kv_dtype, "noalloc large")


def test_noalloc_decode_refuses_bounds_beyond_its_scratch():
    say("case noalloc decode beyond scratch")
    call = synth.make_call([1, 1], [700, 600], "full", "bf16", [92, 0])
    d = stage(call)
    run_kvwrite(d)
    pages = -(-1_048_584 // 64)
    need = ba.beam_attn_decode_workspace_bytes(d["layer"].desc, 64, 16, 1_048_584)
    assert need > ba.BEAM_DECODE_NOALLOC_SCRATCH_BYTES
    # 64 sequences' worth of bounds: pad the batch to 64 sequences with empty ones
    qs = np.zeros(65, dtype=np.int32)
    qs[1:3] = call.q_start[1:3]
    qs[3:] = call.q_start[2]
    kl = np.zeros(64, dtype=np.int32)
    kl[:2] = call.kv_len
    big = ba.DeviceBatch(qs, kl, np.zeros((64, pages), dtype=np.int32), "cuda")
    big.max_q_len, big.max_kv_len = 16, 1_048_584
    d["batch"] = big
    out = torch.full_like(d["out"], float("nan"))
    with pytest.raises(ba.BeamError) as e:
        _noalloc(d, out)
    assert e.value.status == ba.BEAM_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()    # nothing was launched
