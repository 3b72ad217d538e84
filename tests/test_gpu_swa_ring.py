"""Sliding-window layers over a window-only page pool: each sequence owns a ring of 9
pages (576 slots), and logical page p of the sequence maps to ring page p mod 9.

The kernels read only the pages that overlap the window of the new tokens, and the
fused K/V store writes each new token at its logical slot, so a ring works unchanged as
long as one call adds at most 9 * 64 - 511 = 65 tokens per sequence (the oldest key the
first new token needs must not be overwritten by the call's own stores). The test runs
two sequences through their rings in steps of 1..65 new tokens (prefill and decode
steps) and compares every output row with the oracle run on each whole sequence at once
over an ordinary cache ("Reflection Beam 1.0 on vLLM": sliding-window layers keep only
the window's KV; section on the two KV lifetimes)."""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from tests.gpu_util import TOL, bits16, say

pytestmark = pytest.mark.gpu

RING = 9
MAX_STEP = RING * synth.PAGE - synth.WINDOW + 1          # 65


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_swa_window_ring_matches_whole_sequence_oracle(kv_dtype):
    from nope_gqa_attention_amd import beamattn as ba
    from nope_gqa_attention_amd.layer import HybridAttention

    lens = [700, 333]
    say(f"case swa ring kv={kv_dtype} lens={lens} ring={RING} pages")
    whole = synth.make_call(lens, lens, "swa", kv_dtype, [41, 7])
    ref = O.layer_call(whole.oracle_inputs())["y"]

    dev = "cuda"
    B = len(lens)
    fill = synth.BF16_NAN if kv_dtype == "bf16" else synth.FP8_NAN
    shape = (B * RING, synth.HKV, synth.PAGE, synth.D)
    if kv_dtype == "bf16":
        kc = torch.full(shape, fill, dtype=torch.int16, device=dev).view(torch.bfloat16)
        vc = torch.full(shape, fill, dtype=torch.int16, device=dev).view(torch.bfloat16)
    else:
        kc = torch.full(shape, fill, dtype=torch.uint8, device=dev)
        vc = torch.full(shape, fill, dtype=torch.uint8, device=dev)
    cache = ba.DeviceCache(kc, vc, whole.k_scale, whole.v_scale)
    max_pages = (max(lens) + synth.PAGE - 1) // synth.PAGE
    bt = np.array([[b * RING + p % RING for p in range(max_pages)] for b in range(B)], dtype=np.int32)
    layer = HybridAttention("swa")
    t = {n: getattr(whole, n).to(dev) for n in ("q", "k", "v", "gate", "q_norm_w", "k_norm_w", "gate_bias")}
    out_all = torch.empty_like(t["q"])

    sizes = [64, 50, 1, 65, 16, 3, 64, 37, 1, 1, 65, 64, 64, 2, 64]
    done = [0] * B
    step = 0
    while any(done[b] < lens[b] for b in range(B)):
        want = sizes[step % len(sizes)]
        step += 1
        n = [min(want, lens[b] - done[b]) for b in range(B)]
        assert max(n) <= MAX_STEP
        idx = torch.cat([torch.arange(int(whole.q_start[b]) + done[b], int(whole.q_start[b]) + done[b] + n[b])
                         for b in range(B)]).to(dev)
        q_start = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        kv_len = np.array([done[b] + n[b] for b in range(B)], dtype=np.int32)
        batch = ba.DeviceBatch(q_start, kv_len, bt, dev)
        q_out = torch.empty(len(idx), synth.HQ, synth.D, dtype=torch.bfloat16, device=dev)
        out = torch.empty_like(q_out)
        mode = "decode" if 1 <= max(n) <= 16 else "prefill"
        layer.kvwrite(batch, cache, t["q"][idx].contiguous(), t["k"][idx].contiguous(),
                      t["v"][idx].contiguous(), t["q_norm_w"], t["k_norm_w"], q_out)
        layer.attend(batch, cache, q_out, t["gate"][idx].contiguous(), t["gate_bias"], out, mode=mode)
        out_all[idx] = out
        done = [done[b] + n[b] for b in range(B)]
    torch.cuda.synchronize()
    say(f"  {step} steps")
    g = O.bf16_bits_to_f64(bits16(out_all))
    assert np.all(np.isfinite(g))
    err = np.abs(g - ref)
    tmax, tmean = TOL[kv_dtype]
    say(f"  max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= tmax and err.mean() <= tmean
