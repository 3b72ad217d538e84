"""Parity of the bf16 projection kernel (y = x W^T) with the fp64 oracle: small ragged
shapes spanning several tiles and tails, strided views, and the two projections of the
attention sublayer at the long-prefill token count (16,384 tokens) on sampled rows:
packed Q/K/V/gate 5120 -> 14336 and o_proj 6144 -> 5120.

Bound: the kernel sums exact bf16 products in fp32 and rounds once to bf16, so each
output is within one bf16 ulp of the exact sum plus k * 2^-24 times the sum of the
terms' magnitudes (fp32 accumulation); almost all outputs are the correctly rounded
value."""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from tests.gpu_util import bits16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


def _check(x, w, y_gpu, rows=None):
    xs = x if rows is None else x[rows]
    yg = y_gpu if rows is None else y_gpu[rows]
    xb, wb = bits16(xs), bits16(w)
    ref = O.linear(xb, wb)
    mass = np.matmul(np.abs(O.bf16_bits_to_f64(xb)), np.abs(O.bf16_bits_to_f64(wb)).T)
    g = O.bf16_bits_to_f64(bits16(yg))
    k = x.shape[1]
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    err = np.abs(g - ref)
    bound = ulp + k * 2.0 ** -24 * mass
    exact = np.mean(g == O.bf16_round(ref))
    say(f"  {g.shape}: max err/bound {np.max(err / bound):.3f}, correctly rounded {exact:.5f}")
    assert np.all(err <= bound)
    assert exact >= 0.99


@pytest.mark.parametrize("m,n,k", [(1, 256, 64), (300, 520, 192), (517, 1024, 5120), (256, 768, 6144)])
def test_linear_matches_oracle(m, n, k):
    from nope_gqa_attention_amd import beamattn as ba
    say(f"case linear m={m} n={n} k={k}")
    x, w = synth.make_linear(m, n, k, [81, m, n, k], device="cuda")
    y = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    ba.beam_linear_bf16(x, w, y)
    torch.cuda.synchronize()
    _check(x, w, y)


def test_linear_strided_views():
    """x, W and y as column ranges of wider tensors (token strides larger than k / n)."""
    from nope_gqa_attention_amd import beamattn as ba
    say("case linear strided")
    xa, wa = synth.make_linear(130, 200, 256, [82, 0], device="cuda")
    x = xa[:, 64:192]                       # k = 128, stride 256
    w = wa[8:136, 64:192]                   # n = 128
    yb = torch.full((130, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    y = yb[:, 128:256]
    ba.beam_linear_bf16(x, w, y)
    torch.cuda.synchronize()
    _check(x, w, y)
    assert torch.all(yb[:, :128] == 7.0) and torch.all(yb[:, 256:] == 7.0)


def test_linear_partial_last_chunk_leaves_neighbours_untouched():
    """n % 8 == 4: the last 16-byte chunk of each output row is half inside the matrix;
    the columns after it (a wider tensor's) must keep their values."""
    from nope_gqa_attention_amd import beamattn as ba
    say("case linear n % 8 == 4")
    x, w = synth.make_linear(260, 260, 128, [85, 0], device="cuda")
    yb = torch.full((260, 272), 7.0, dtype=torch.bfloat16, device="cuda")
    y = yb[:, :260]
    ba.beam_linear_bf16(x, w, y)
    torch.cuda.synchronize()
    _check(x, w, y)
    assert torch.all(yb[:, 260:] == 7.0)


@pytest.mark.parametrize("n,k", [(14336, 5120), (5120, 6144)], ids=["qkv_gate", "o_proj"])
def test_linear_projection_shapes_at_16k_tokens(n, k):
    from nope_gqa_attention_amd import beamattn as ba
    m = 16384
    say(f"case linear projection m={m} n={n} k={k}")
    x, w = synth.make_linear(m, n, k, [83, n, k], device="cuda")
    y = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    ba.beam_linear_bf16(x, w, y)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 255, 256, 4097, 8191, 12000, m - 1], device="cuda")
    _check(x, w, y, rows)


def test_linear_rejects_bad_shapes_and_overlap():
    from nope_gqa_attention_amd import beamattn as ba
    x, w = synth.make_linear(8, 64, 96, [84, 0], device="cuda")
    y = torch.empty(8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ba.BeamError) as e:
        ba.beam_linear_bf16(x, w, y)                     # k = 96 is not a multiple of 64
    assert e.value.status == ba.BEAM_ERR_INVALID_ARG and "64" in str(e.value)
    buf = torch.zeros(8, 128, dtype=torch.bfloat16, device="cuda")
    x2, w2 = synth.make_linear(8, 64, 64, [84, 1], device="cuda")
    buf[:, :64] = x2
    with pytest.raises(ba.BeamError) as e:
        ba.beam_linear_bf16(buf[:, :64], w2, buf[:, 64:])  # y overlaps x's rows
    assert e.value.status == ba.BEAM_ERR_INVALID_ARG
    ba.beam_linear_bf16(x2[:0], w2, y[:0])               # m = 0: nothing to do
