"""The BEAMATTN_DEBUG build (libbeamattn_debug.so): its K/V-write, prefill and decode
entry points check the device-resident batch metadata on the GPU before launching
anything, and report the first broken beam_batch rule instead of reading or writing out
of bounds. On valid batches it computes exactly what the library computes.

The broken batches here are only ever passed to the debug build, whose check runs before
any kernel that would use the metadata; the check itself reads only inside the arrays'
host-validated bounds."""

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import run_attend, run_kvwrite, say, stage

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_lib(gpu_lib):
    from nope_gqa_attention_amd import beamattn as ba
    ba._lib = None
    lib = ba.load(ba.DEBUG_LIB_PATH)
    yield lib
    ba._lib = None
    ba.load()


def _outputs(call, mode):
    d = stage(call)
    run_kvwrite(d)
    run_attend(d, mode=mode)
    torch.cuda.synchronize()
    return d["out"].clone(), d["cache"].k.clone()


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_debug_build_matches_library_on_valid_batches(mode, gpu_lib):
    from nope_gqa_attention_amd import beamattn as ba
    say(f"case debug build == library, mode={mode}")
    q_lens = [5, 1, 9] if mode == "decode" else [40, 0, 130]
    call = synth.make_call(q_lens, [900, 77, 2000], "full", "bf16", [81, 1])
    out_rel, k_rel = _outputs(call, mode)
    ba._lib = None
    ba.load(ba.DEBUG_LIB_PATH)
    try:
        out_dbg, k_dbg = _outputs(call, mode)
    finally:
        ba._lib = None
        ba.load()
    assert torch.equal(out_rel.view(torch.int16), out_dbg.view(torch.int16))
    assert torch.equal(k_rel.view(torch.int16), k_dbg.view(torch.int16))


BROKEN = [
    ("page-past-pool", "block_table entry", 1),
    ("page-negative", "block_table entry", 1),
    ("q_start-decreases", "q_start decreases", 1),
    ("kv_len-below-new", "kv_len is below", 0),
    ("kv_len-above-bound", "kv_len exceeds max_kv_len", 2),
]


@pytest.mark.parametrize("what,message,seq", BROKEN, ids=[b[0] for b in BROKEN])
@pytest.mark.parametrize("entry", ["kvwrite", "prefill", "decode"])
def test_debug_build_reports_broken_metadata(debug_lib, what, message, seq, entry):
    from nope_gqa_attention_amd import beamattn as ba
    say(f"case debug check {what} via {entry}")
    # sequence 3 has the most new tokens, so that moving q_start[2] down breaks only the
    # ordering rule (sequence 2 then has 7 new tokens, still within max_q_len = 8)
    q_lens = [3, 4, 2, 8]
    call = synth.make_call(q_lens, [700, 300, 1500, 1000], "swa", "bf16", [82, 1])
    d = stage(call)
    b = d["batch"]
    num_pages = d["cache"].k.shape[0]
    if what == "page-past-pool":
        b.block_table[1, 300 // 64] = num_pages          # the page of sequence 1's new tokens
    elif what == "page-negative":
        b.block_table[1, 299 // 64] = -1
    elif what == "q_start-decreases":
        b.q_start[2] = int(call.q_start[1]) - 1
    elif what == "kv_len-below-new":
        b.kv_len[0] = q_lens[0] - 1
    elif what == "kv_len-above-bound":
        b.kv_len[2] = b.max_kv_len + 1
    torch.cuda.synchronize()
    d["out"].fill_(7.0)
    k_before = d["cache"].k.clone()
    with pytest.raises(ba.BeamError) as e:
        if entry == "kvwrite":
            run_kvwrite(d)
        else:
            run_attend(d, mode=entry)
    torch.cuda.synchronize()
    say(f"  -> {e.value}")
    assert e.value.status == ba.BEAM_ERR_INVALID_ARG
    assert message in str(e.value) and f"sequence {seq}" in str(e.value)
    # nothing was launched: no output written, no cache byte changed
    assert bool((d["out"] == 7.0).all())
    assert torch.equal(d["cache"].k.view(torch.int16), k_before.view(torch.int16))
