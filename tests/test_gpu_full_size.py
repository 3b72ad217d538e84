"""Parity at the workloads' real sizes, in the launch configuration bench.py times.

Each workload is staged exactly as bench.py stages it (same generator, seed, device-side
cache draw, page permutation and NaN-poisoned unused slots), run through the C ABI, and
compared with the fp64 oracle on sampled rows: the oracle reads the very pages the GPU
read (copied back per sequence), so every sampled output is checked at full context.
  long prefill   8 sequences x 2048 new tokens on 98,304 cached (bf16): 5 rows per sequence
  the same prefill over an fp8 cache (chunked prefill on fp8 KV): 5 rows per sequence
  batch-1 decode 1 token at p = 100,000 (bf16): the row
  batched decode 32 sequences, 8K..128K keys (fp8): every row
  1M verify      8 tokens on 1,048,576 cached (fp8): every row
  long prefill at the TP8 head share (6 query heads, 1 KV head), bf16 and fp8 caches:
                 7 tokens per sequence, two of them straddling a 256-row tile boundary
                 (row 8192 of 12,288 = token 1365, head 2)
Both layer kinds run each workload."""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from bench import Staged
from tests.gpu_util import TOL, bits16, say, seq_host_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


def _check(cfg, kind, mode, rows_of_seq, kv_dtype=None, heads=None):
    call = synth.make_config(cfg, kind, cache_device="cuda", kv_dtype=kv_dtype, heads=heads)
    say(f"case full-size config{cfg} kind={kind} mode={mode}: {call.num_seqs} seqs, "
        f"{call.num_tokens} tokens, {call.k_cache.shape[0]} pages, {call.kv_dtype}")
    s = Staged(call)
    s.kvwrite()
    s.attend(mode)
    torch.cuda.synchronize()
    out = s.out
    errs = []
    for b in range(call.num_seqs):
        rows = rows_of_seq(b, int(call.q_start[b + 1] - call.q_start[b]))
        if len(rows) == 0:
            continue
        inp = seq_host_inputs(call, b)
        ref = O.layer_call(inp, rows=np.asarray(rows))["y"]
        got = O.bf16_bits_to_f64(bits16(out[int(call.q_start[b]) + np.asarray(rows)]))
        assert np.all(np.isfinite(got)), f"seq {b}: non-finite output"
        errs.append(np.abs(got - ref).reshape(len(rows), -1))
    err = np.concatenate(errs)
    tmax, tmean = TOL[call.kv_dtype]
    say(f"  {err.shape[0]} rows: max-abs {err.max():.3e} (tol {tmax}), mean-abs {err.mean():.3e} (tol {tmean})")
    assert err.max() <= tmax and err.mean() <= tmean
    del s, call
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["swa", "full"])
def test_long_prefill_full_size_sampled_rows(kind):
    _check(1, kind, "prefill", lambda b, n: [0, 63, 64, 1000 + 37 * b, n - 1])


@pytest.mark.parametrize("kind", ["swa", "full"])
def test_long_prefill_fp8_cache_full_size_sampled_rows(kind):
    _check(1, kind, "prefill", lambda b, n: [0, 63, 64, 1000 + 37 * b, n - 1], kv_dtype="fp8")


@pytest.mark.parametrize("kind", ["swa", "full"])
def test_batch1_decode_full_size(kind):
    _check(2, kind, "decode", lambda b, n: list(range(n)))


@pytest.mark.parametrize("kind", ["swa", "full"])
def test_batched_fp8_decode_full_size(kind):
    _check(3, kind, "decode", lambda b, n: list(range(n)))


@pytest.mark.parametrize("kind", ["swa", "full"])
def test_1m_verify_full_size(kind):
    _check(4, kind, "decode", lambda b, n: list(range(n)))


@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_long_prefill_tp8_head_share_sampled_rows(kind, kv_dtype):
    _check(1, kind, "prefill", lambda b, n: [0, 63, 1364, 1365, 1366, 2000 + b, n - 1],
           kv_dtype=kv_dtype, heads=(6, 1))
