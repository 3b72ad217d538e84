"""One decode workspace shared by calls of different shapes, in sequence.

The workspace holds scratch partials only: its contents need no initialisation. Each
call here runs on a workspace filled with 0xFF bytes (NaN as fp32) and is checked
against the oracle; the calls cover the split merge for one 16-row block and for
48-row chunks, several and many splits, and one split (no workspace use). A repeated
call must reproduce its first output bit for bit."""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from nope_gqa_attention_amd import beamattn as ba
from tests.gpu_util import TOL, bits16, run_kvwrite, say, seq_host_inputs, stage

pytestmark = pytest.mark.gpu

# name, kind, cache dtype, new tokens per sequence, keys per sequence after the call
CALLS = [
    ("batch1-60k", "full", "bf16", [1], [60000]),
    ("verify8-2seq", "full", "fp8", [8, 3], [30000, 7000]),
    ("batch2-140k", "full", "bf16", [1, 1], [140000, 9000]),
    ("batch4-mixed", "full", "fp8", [1, 2, 1, 1], [3000, 12000, 700, 40000]),
    ("swa-one-split", "swa", "bf16", [1, 1], [9000, 300]),
]


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


def _run(call, ws):
    d = stage(call)
    run_kvwrite(d)
    ws.fill_(0xFF)
    ba.beam_attn_decode(d["layer"].desc, d["batch"], d["cache"], d["q_out"], d["gate"],
                        d["gate_bias"], d["out"], ws)
    torch.cuda.synchronize()
    return d


def _check_oracle(call, out, what):
    errs = []
    for b in range(call.num_seqs):
        s, e = int(call.q_start[b]), int(call.q_start[b + 1])
        if e == s:
            continue
        ref = O.layer_call(seq_host_inputs(call, b))["y"]
        got = O.bf16_bits_to_f64(bits16(out[s:e]))
        assert np.all(np.isfinite(got)), f"{what} seq {b}: non-finite output"
        errs.append(np.abs(got - ref).reshape(e - s, -1))
    err = np.concatenate(errs)
    tmax, tmean = TOL[call.kv_dtype]
    say(f"  {what}: max-abs {err.max():.3e} (tol {tmax}), mean-abs {err.mean():.3e} (tol {tmean})")
    assert err.max() <= tmax and err.mean() <= tmean


def test_shared_garbage_workspace_across_shapes():
    calls = [(name, synth.make_call(q, k, kind, dt, [41, i], cache_device="cuda"))
             for i, (name, kind, dt, q, k) in enumerate(CALLS)]
    need = 0
    for name, call in calls:
        layer = ba.layer_desc(call.kind)
        need = max(need, ba.beam_attn_decode_workspace_bytes(layer, call.num_seqs, call.max_q_len,
                                                             int(call.kv_len.max())))
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    first = None
    for name, call in calls + [calls[0]]:
        say(f"case shared workspace: {name} ({call.kind}, {call.kv_dtype}, q {list(call.q_lens)}, "
            f"kv {list(call.kv_len)})")
        d = _run(call, ws)
        if first is None:
            first = bits16(d["out"])
            _check_oracle(call, d["out"], name)
        elif name == calls[0][0]:
            assert np.array_equal(bits16(d["out"]), first), "repeated call changed its output bits"
        else:
            _check_oracle(call, d["out"], name)
        del d
    torch.cuda.empty_cache()
