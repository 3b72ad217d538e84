"""The fp8 store on the GPU over every bf16 input pattern.

All 65,536 bf16 bit patterns (NaN, +-inf, subnormals, values past +-448 and values whose
quotient lies on an e4m3 rounding midpoint included) go in as the V rows of one
64-token K/V write into an fp8 cache, once per V scale. Every stored code must equal the
oracle's: the e4m3 code nearest to the exact quotient value / scale (saturating at
+-448, NaN to 0x7F), formed there in fp64. At v_scale = 1 the quotient is the value
itself; at the scales of the form amax/448 some binary32 quotients land on a midpoint
that the exact quotient is not on, which the device encoder has to settle the exact way.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from tests.gpu_util import run_kvwrite, say, stage

pytestmark = pytest.mark.gpu

SCALES = [1.0, float(np.float32(5.0625 / 448)), float(np.float32(4.9375 / 448)),
          0.01018415205180645, 2.0 ** -7, 3.0]


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


def _all_patterns_call(v_scale):
    call = synth.make_call([64], [64], "full", "fp8", [61, 0])
    pats = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    return dataclasses.replace(call, v=pats.reshape(64, 8, 128).clone(), v_scale=v_scale)


@pytest.mark.parametrize("v_scale", SCALES)
def test_fp8_store_of_every_bf16_pattern_matches_oracle(v_scale):
    say(f"case fp8 codec v_scale={v_scale!r}")
    call = _all_patterns_call(v_scale)
    inp = call.oracle_inputs()
    seq, pos = O.new_token_positions(inp["q_start"], inp["kv_len"])
    ref = O.store_kv(inp["v_cache"], inp["block_table"], seq, pos, inp["v"], "fp8", v_scale)
    d = stage(call)
    run_kvwrite(d)
    torch.cuda.synchronize()
    got = d["cache"].v.cpu().numpy()
    page, slot = O.physical_slot(inp["block_table"], seq, pos)
    g, e = got[page, :, slot, :], ref[page, :, slot, :]
    bad = np.nonzero(g != e)
    say(f"  {g.size} codes, {len(bad[0])} differ")
    if len(bad[0]):
        i = tuple(b[0] for b in bad)
        raise AssertionError(f"bf16 0x{int(inp['v'][i]):04x}: GPU code 0x{int(g[i]):02x}, "
                             f"oracle 0x{int(e[i]):02x}")
    if v_scale == 1.0:
        # the quotient is the value itself: the codes are the oracle's encoder applied to
        # each pattern directly
        x = O.bf16_bits_to_f64(inp["v"])
        assert np.array_equal(g, O.f64_to_e4m3(x))
        assert np.all(g[np.isnan(x)] == 0x7F)
        assert np.all(g[np.isposinf(x)] == 0x7E) and np.all(g[np.isneginf(x)] == 0xFE)
