"""Pages beyond 4 GiB of cache: slot and element offsets that only int64 arithmetic holds.

A page of one layer's K (or V) cache holds 8 KV heads x 64 slots x 128 values, so the
element offset of a slot passes 2^31 from physical page 32,768 on (bf16: byte offsets
past 4 GiB). These calls draw about 100,000 spare pages, so the data pages scatter over
physical indices up to ~100,000 (the block table maps every logical page, "Reflection
Beam 1.0 on vLLM": paged KV cache of 64-token pages); the fused K/V store, prefill and
decode must read and write exactly the pages the oracle reads."""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from tests.gpu_util import TOL, bits16, run_layer, say, seq_host_inputs

pytestmark = pytest.mark.gpu

SPARE_PAGES = 100_000
LIMIT_PAGE = 2 ** 31 // (8 * 64 * 128)        # first page whose element offset needs 32+ bits


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("mode,q_lens,kv_lens", [("prefill", [5, 40, 1], [3000, 40, 700]),
                                                 ("decode", [1, 4, 1], [3000, 9, 700])],
                         ids=["prefill", "decode"])
def test_pages_past_int32_offsets(kind, kv_dtype, mode, q_lens, kv_lens):
    call = synth.make_call(q_lens, kv_lens, kind, kv_dtype, [81, len(mode)], spare_pages=SPARE_PAGES,
                           cache_device="cuda")
    used = {int(call.block_table[b][j]) for b in range(call.num_seqs)
            for j in range((int(call.kv_len[b]) + 63) // 64)}
    high = sum(1 for p in used if p >= LIMIT_PAGE)
    say(f"case large offsets {mode} kind={kind} dtype={kv_dtype}: {call.k_cache.shape[0]} pages, "
        f"{high} of {len(used)} used pages at or past page {LIMIT_PAGE}")
    assert high > 0
    d = run_layer(call, mode)
    errs = []
    for b in range(call.num_seqs):
        s, e = int(call.q_start[b]), int(call.q_start[b + 1])
        ref = O.layer_call(seq_host_inputs(call, b))["y"]
        got = O.bf16_bits_to_f64(bits16(d["out"][s:e]))
        assert np.all(np.isfinite(got)), f"seq {b}: non-finite output"
        errs.append(np.abs(got - ref).reshape(e - s, -1))
    err = np.concatenate(errs)
    tmax, tmean = TOL[kv_dtype]
    say(f"  max-abs {err.max():.3e} (tol {tmax}), mean-abs {err.mean():.3e} (tol {tmean})")
    assert err.max() <= tmax and err.mean() <= tmean
    del d, call
    torch.cuda.empty_cache()
