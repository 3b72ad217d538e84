"""Attention over q', gate and out that are column ranges of wider row-major tensors, as
when they are views into the packed QKV + gate projection output ("Reflection Beam 1.0
on vLLM", section "Agent-driven optimization made batch-1 decode 2.71x faster": one packed
GEMM feeds the fused norm kernel), against the same call on contiguous tensors.

The token stride only moves where each row is read or written, so the two calls must
agree bit for bit. Prefill moves these rows through LDS with 32-bit offsets from each row
tile's first token; the cases cover both layer kinds, both cache dtypes, a ragged batch
whose tiles start inside a token's heads, the largest token stride the entry point
accepts, and one past it (refused)."""

import pytest
import torch

import synth
from tests.gpu_util import run_attend, run_kvwrite, say, stage

pytestmark = pytest.mark.gpu

MAX_STRIDE = 4194303 // 8 * 8        # largest multiple of 8 within the documented bound


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


def _wide(n_tok, stride, col0, like):
    """A [n_tok][Hq][128] view at column col0 of a [n_tok][stride] bf16 tensor whose other
    columns hold NaN, so that a read outside the view shows in the output."""
    hq, d = like.shape[1], like.shape[2]
    base = torch.full((n_tok, stride), float("nan"), dtype=torch.bfloat16, device=like.device)
    v = base[:, col0:col0 + hq * d].view(n_tok, hq, d)
    v.copy_(like)
    return base, v


@pytest.mark.parametrize("kind", ["swa", "full"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_strided_rows_equal_contiguous_bit_for_bit(kind, kv_dtype, mode):
    say(f"case strided rows kind={kind} dtype={kv_dtype} mode={mode}")
    q_lens = [300, 77, 5] if mode == "prefill" else [1, 7, 16]
    call = synth.make_call(q_lens, [1500, 77, 700], kind, kv_dtype, [91, len(q_lens)])
    d = stage(call)
    run_kvwrite(d)
    run_attend(d, mode)
    torch.cuda.synchronize()
    ref = d["out"].clone()
    n = d["q_out"].shape[0]
    # the packed projection's layout: q' in columns [0, 6144), gate in [8192, 14336)
    _, qv = _wide(n, 14336, 0, d["q_out"])
    gbase, _ = _wide(n, 14336, 8192, d["gate"].view(n, 48, 128))
    obase, ov = _wide(n, 6144 + 64, 64, torch.zeros_like(d["out"]))
    d["layer"].attend(d["batch"], d["cache"], qv, gbase[:, 8192:], d["gate_bias"], ov, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(ov.contiguous().view(torch.int16), ref.view(torch.int16))
    # columns around the output view are untouched
    assert torch.isnan(obase[:, :64].float()).all()


@pytest.mark.parametrize("kind", ["swa", "full"])
def test_prefill_at_the_largest_token_stride(kind):
    # one query head per KV head: a full-layer row tile is 256 tokens, so its rows reach
    # 255 strides past its first token, the farthest the 32-bit offsets go
    say(f"case prefill largest stride kind={kind}")
    call = synth.make_call([300, 3], [300, 900], kind, "bf16", [92, 2], heads=(8, 8))
    d = stage(call)
    run_kvwrite(d)
    run_attend(d, "prefill")
    torch.cuda.synchronize()
    ref = d["out"].clone()
    n = d["q_out"].shape[0]
    # q' rows MAX_STRIDE elements apart (303 tokens: about 2.5 GB), out and gate contiguous
    _, qv = _wide(n, MAX_STRIDE, 0, d["q_out"])
    d["layer"].attend(d["batch"], d["cache"], qv, d["gate"], d["gate_bias"], d["out"], mode="prefill")
    torch.cuda.synchronize()
    assert torch.equal(d["out"].view(torch.int16), ref.view(torch.int16))
    del qv
    torch.cuda.empty_cache()


def test_prefill_refuses_a_token_stride_past_the_bound():
    from nope_gqa_attention_amd import beamattn as ba

    call = synth.make_call([4], [40], "full", "bf16", [93, 1])
    d = stage(call)
    n = d["q_out"].shape[0]
    base = torch.zeros((n, MAX_STRIDE + 8), dtype=torch.bfloat16, device="cuda")
    qv = base[:, :48 * 128].view(n, 48, 128)
    with pytest.raises(ba.BeamError, match="stride"):
        d["layer"].attend(d["batch"], d["cache"], qv, d["gate"], d["gate_bias"], d["out"], mode="prefill")
