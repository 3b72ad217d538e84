"""A chunked-prefill step recorded once as a HIP graph and replayed with other chunk
lengths and contexts.

The step is the fused Q/K norm + RoPE/SSMax + KV store followed by prefill attention
with the gate ("Reflection Beam 1.0 on vLLM", section "Attention: sliding-window layers
plus NoPE full-attention layers"; chunked prefill: new tokens attend to the cached prefix
and causally among themselves). It is recorded with host bounds that cover every step
(300 new tokens per sequence, 3,000 keys, all token rows), so that only device arrays
and tensor contents change between replays: row tiles past a sequence's new tokens exit,
and full layers keep the key-split plan the bounds chose. Every replay is compared bit
for bit with the same step run eagerly in between, and with the oracle."""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O
import synth
from tests.gpu_util import TOL, bits16, say

pytestmark = pytest.mark.gpu

NSEQ, MAXQ, MAXKV = 3, 300, 3000
STEPS = [([300, 77, 5], [1500, 77, 700]), ([1, 300, 120], [3000, 300, 2000]),
         ([64, 65, 1], [64, 2999, 2500])]


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


class StaticBatch:
    """beam_batch over fixed device arrays, with bounds that cover every step."""

    def __init__(self, max_pages, dev):
        self.q_start = torch.zeros(NSEQ + 1, dtype=torch.int32, device=dev)
        self.kv_len = torch.zeros(NSEQ, dtype=torch.int32, device=dev)
        self.block_table = torch.zeros(NSEQ, max_pages, dtype=torch.int32, device=dev)
        self.num_seqs, self.num_tokens = NSEQ, NSEQ * MAXQ
        self.max_q_len, self.max_kv_len, self.max_pages = MAXQ, MAXKV, max_pages

    def struct(self):
        from nope_gqa_attention_amd import beamattn as ba
        return ba.Batch(self.num_seqs, self.q_start.data_ptr(), self.kv_len.data_ptr(),
                        self.block_table.data_ptr(), self.max_pages, self.max_q_len,
                        self.max_kv_len, self.num_tokens)


@pytest.mark.parametrize("kind,kv_dtype", [("swa", "bf16"), ("full", "bf16"), ("full", "fp8")])
def test_prefill_step_graph_replays_match_eager_and_oracle(kind, kv_dtype):
    from nope_gqa_attention_amd import beamattn as ba
    from nope_gqa_attention_amd.layer import HybridAttention

    say(f"case prefill graph kind={kind} dtype={kv_dtype} steps={len(STEPS)}")
    dev = "cuda"
    scales = (0.0125, 0.0125) if kv_dtype == "fp8" else None
    calls = [synth.make_call(q, k, kind, kv_dtype, [64, i], fp8_scales=scales)
             for i, (q, k) in enumerate(STEPS)]
    refs = [O.layer_call(c.oracle_inputs())["y"] for c in calls]
    max_pages = (MAXKV + synth.PAGE - 1) // synth.PAGE
    pool = max(c.k_cache.shape[0] for c in calls)
    N = NSEQ * MAXQ
    cdt = torch.uint8 if kv_dtype == "fp8" else torch.bfloat16
    st = {
        "kc": torch.zeros(pool, synth.HKV, synth.PAGE, synth.D, dtype=cdt, device=dev),
        "vc": torch.zeros(pool, synth.HKV, synth.PAGE, synth.D, dtype=cdt, device=dev),
        "q": torch.zeros(N, synth.HQ, synth.D, dtype=torch.bfloat16, device=dev),
        "k": torch.zeros(N, synth.HKV, synth.D, dtype=torch.bfloat16, device=dev),
        "v": torch.zeros(N, synth.HKV, synth.D, dtype=torch.bfloat16, device=dev),
        "gate": torch.zeros(N, synth.HQ * synth.D, dtype=torch.bfloat16, device=dev),
        "qnw": torch.zeros(synth.D, dtype=torch.bfloat16, device=dev),
        "knw": torch.zeros(synth.D, dtype=torch.bfloat16, device=dev),
        "bias": torch.zeros(synth.HQ, dtype=torch.bfloat16, device=dev),
        "q_out": torch.zeros(N, synth.HQ, synth.D, dtype=torch.bfloat16, device=dev),
        "out": torch.zeros(N, synth.HQ, synth.D, dtype=torch.bfloat16, device=dev),
    }
    batch = StaticBatch(max_pages, dev)
    # one scale pair for every step (the graph records the cache descriptor by value)
    ks, vs = calls[0].k_scale, calls[0].v_scale
    cache = ba.DeviceCache(st["kc"], st["vc"], ks, vs)
    layer = HybridAttention(kind)

    def load(i):
        c = calls[i]
        n = c.num_tokens
        P = c.k_cache.shape[0]
        st["kc"][:P].copy_(c.k_cache)
        st["vc"][:P].copy_(c.v_cache)
        for name, src in (("q", c.q), ("k", c.k), ("v", c.v), ("gate", c.gate)):
            st[name].zero_()
            st[name][:n].copy_(src)
        st["qnw"].copy_(c.q_norm_w); st["knw"].copy_(c.k_norm_w); st["bias"].copy_(c.gate_bias)
        batch.q_start.copy_(torch.from_numpy(c.q_start))
        batch.kv_len.copy_(torch.from_numpy(c.kv_len))
        bt = np.zeros((NSEQ, max_pages), dtype=np.int32)
        bt[:, :c.block_table.shape[1]] = c.block_table
        batch.block_table.copy_(torch.from_numpy(bt))

    def step():
        layer.kvwrite(batch, cache, st["q"], st["k"], st["v"], st["qnw"], st["knw"], st["q_out"])
        layer.attend(batch, cache, st["q_out"], st["gate"], st["bias"], st["out"], mode="prefill")

    load(0)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(2):
        for i, c in enumerate(calls):
            assert c.k_scale == ks and c.v_scale == vs
            load(i)
            g.replay()
            torch.cuda.synchronize()
            n = c.num_tokens
            got = st["out"][:n].clone()
            load(i)
            step()                                    # eager, same bounds
            torch.cuda.synchronize()
            eager = st["out"][:n].clone()
            assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"step {i} rep {rep}"
            y = O.bf16_bits_to_f64(bits16(got))
            err = np.abs(y - refs[i])
            tmax, tmean = TOL[kv_dtype]
            say(f"  rep {rep} step {i} q={STEPS[i][0]} kv={STEPS[i][1]}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
            assert np.all(np.isfinite(y)) and err.max() <= tmax and err.mean() <= tmean
