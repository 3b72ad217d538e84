"""Scores that keep growing along the key axis: the online softmax must raise its running
maximum again and again, and the split merge must weigh splits whose maxima lie hundreds
of binary orders of magnitude apart.

Every query row is the same direction u and key j is cos(t_j) u + sin(t_j) r (r orthogonal
to u), with t_j falling from pi to 0 along the sequence, so a query's score grows with
the key position. With both RMSNorm weights at 4 the normalised vectors have length
4 sqrt(128) and the scaled scores span about +-261 in log2 units: about 0.75 per key, so
the running maximum outgrows the kernels' 2^8 rescale slack every few tiles, and the
softmax weight sits on the last few visible keys. The oracle is the plain two-pass
softmax in fp64 on the same bits ("Reflection Beam 1.0 on vLLM", Attention section:
per-head Q/K normalisation before attention)."""

import math

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from tests.gpu_util import assert_close_to_oracle, bits16, run_layer, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


def _directions(seed):
    g = np.random.default_rng(seed)
    u = g.standard_normal(128)
    u /= np.sqrt(np.mean(u * u))
    r = g.standard_normal(128)
    r -= u * (r @ u) / (u @ u)
    r /= np.sqrt(np.mean(r * r))
    return u, r


def _key(u, r, j, n):
    t = math.pi * (1.0 - j / max(n - 1, 1))
    return math.cos(t) * u + math.sin(t) * r


def _growing_call(q_lens, kv_lens, kind, kv_dtype, seed):
    call = synth.make_call(q_lens, kv_lens, kind, kv_dtype, [71, seed])
    u, r = _directions(seed)
    four = torch.full((128,), 4.0, dtype=torch.bfloat16)
    call.q_norm_w.copy_(four)
    call.k_norm_w.copy_(four)
    call.q[:] = torch.tensor(u, dtype=torch.bfloat16)
    for b in range(call.num_seqs):
        s, e = int(call.q_start[b]), int(call.q_start[b + 1])
        kv = int(call.kv_len[b])
        first = kv - (e - s)
        for i in range(e - s):
            call.k[s + i, :] = torch.tensor(_key(u, r, first + i, kv), dtype=torch.bfloat16)
        # cached keys are stored as the fused store would leave them: normalised (length
        # 4 sqrt(128)), one bf16 rounding; bf16 caches only
        assert first == 0 or call.kv_dtype == "bf16"
        for j in range(first):
            page = int(call.block_table[b][j // 64])
            kj = _key(u, r, j, kv)
            kj = 4.0 * kj / np.sqrt(np.mean(kj * kj))
            call.k_cache[page, :, j % 64, :] = torch.tensor(kj, dtype=torch.bfloat16)
    return call


@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_prefill_growing_scores(kind, kv_dtype):
    say(f"case prefill growing scores kind={kind} dtype={kv_dtype}")
    call = _growing_call([700, 130], [700, 130], kind, kv_dtype, 1)
    ref = O.layer_call(call.oracle_inputs())["y"]
    d = run_layer(call, "prefill")
    assert_close_to_oracle(bits16(d["out"]), ref, kv_dtype, f"prefill growing {kind} {kv_dtype}")


@pytest.mark.parametrize("kind", ["swa", "full"])
def test_decode_growing_scores_across_splits(kind):
    say(f"case decode growing scores kind={kind}")
    call = _growing_call([1, 4], [9000, 3000], kind, "bf16", 2)
    ref = O.layer_call(call.oracle_inputs())["y"]
    d = run_layer(call, "decode")
    assert_close_to_oracle(bits16(d["out"]), ref, "bf16", f"decode growing {kind}")
