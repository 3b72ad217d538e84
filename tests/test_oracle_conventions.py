"""Pins of the oracle's conventions against the routines of the `transformers` library
that implement the same model components.

The pages fix the components (a 512-token sliding window, rotary embeddings on the
sliding layers, per-head Q/K RMS normalisation, 48 query heads over 8 KV heads: "Reflection
Beam 1.0 on vLLM", section "Attention: sliding-window layers plus NoPE full-attention
layers") but not every convention inside them: whether the window counts the query's
own key, which dimensions RoPE pairs, how query heads map to KV heads, whether one norm
weight serves all heads. The oracle takes the reading of the common open
implementations; these tests check it against those implementations' own code, run
here on CPU:
  * the window and causal masks against `transformers.masking_utils`;
  * the query-head -> KV-head mapping against Llama's `repeat_kv`;
  * the rotary embedding (pairing, direction, frequencies) against Llama's
    `LlamaRotaryEmbedding` and `apply_rotary_pos_emb`;
  * the per-head RMSNorm with one [head_dim] weight against Qwen3's `q_norm`.
"""

import numpy as np
import pytest
import torch

import oracle.beam_oracle as O

transformers = pytest.importorskip("transformers")


def test_sliding_window_and_causal_visibility_match_transformers_masks():
    from transformers import masking_utils as mu

    q = torch.arange(0, 1200)[:, None]
    kv = torch.arange(0, 1200)[None, :]
    swa = mu.sliding_window_causal_mask_function(O.WINDOW)(0, 0, q, kv).numpy()
    full = mu.causal_mask_function(0, 0, q, kv).numpy()
    qn, kn = np.arange(1200)[:, None], np.arange(1200)[None, :]
    lo_s = np.array([O.visible_range(int(p), O.KIND_SWA)[0] for p in range(1200)])[:, None]
    lo_f = np.array([O.visible_range(int(p), O.KIND_FULL)[0] for p in range(1200)])[:, None]
    ours_swa = (kn >= lo_s) & (kn <= qn)
    ours_full = (kn >= lo_f) & (kn <= qn)
    assert np.array_equal(ours_swa, swa)
    assert np.array_equal(ours_full, full)
    # 512 keys per row once the window is full, the query's own key among them
    assert swa[600].sum() == 512 and swa[600, 600] and not swa[600, 88]
    # other window lengths (the layer descriptor's window is a parameter)
    for w in (1, 64, 200, 1000):
        ref = mu.sliding_window_causal_mask_function(w)(0, 0, q, kv).numpy()
        lo_w = np.array([O.visible_range(int(p), O.KIND_SWA, w)[0] for p in range(1200)])[:, None]
        assert np.array_equal((kn >= lo_w) & (kn <= qn), ref), w


def test_query_heads_read_kv_heads_as_repeat_kv_maps_them():
    from transformers.models.llama.modeling_llama import repeat_kv

    rng = np.random.default_rng(5)
    R, L, Hq, Hkv, D = 7, 40, O.NUM_Q_HEADS, O.NUM_KV_HEADS, O.HEAD_DIM
    q = rng.standard_normal((R, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    ours = O.attend(q, k, v)
    # Llama's layout: [batch, heads, seq, dim]; repeat_kv expands KV heads to query heads
    kr = repeat_kv(torch.from_numpy(k).permute(1, 0, 2)[None], Hq // Hkv)[0]   # [Hq, L, D]
    vr = repeat_kv(torch.from_numpy(v).permute(1, 0, 2)[None], Hq // Hkv)[0]
    qt = torch.from_numpy(q).permute(1, 0, 2)                                  # [Hq, R, D]
    p = torch.softmax(O.SM_SCALE * (qt @ kr.transpose(1, 2)), dim=-1)
    ref = (p @ vr).permute(1, 0, 2).numpy()
    assert np.max(np.abs(ours - ref)) < 1e-12


def _llama_rotary(positions, dtype):
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding

    cfg = LlamaConfig(hidden_size=O.NUM_Q_HEADS * O.HEAD_DIM, num_attention_heads=O.NUM_Q_HEADS,
                      num_key_value_heads=O.NUM_KV_HEADS, head_dim=O.HEAD_DIM,
                      rope_theta=O.ROPE_THETA, max_position_embeddings=1 << 21)
    emb = LlamaRotaryEmbedding(cfg)
    x = torch.zeros(1, 1, O.HEAD_DIM, dtype=dtype)
    cos, sin = emb(x, torch.as_tensor(positions)[None])
    return emb, cos[0], sin[0]


def test_rope_frequencies_match_llama_rotary_embedding():
    emb, _, _ = _llama_rotary([0], torch.float32)
    inv = emb.inv_freq.double().numpy()
    assert inv.shape == (O.HEAD_DIM // 2,)
    assert np.allclose(O.rope_inv_freq(), inv, rtol=1e-6, atol=0)


def test_rope_rotation_matches_llama_apply_rotary_pos_emb():
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb

    rng = np.random.default_rng(6)
    pos = np.array([0, 1, 2, 63, 64, 511, 512, 1000])
    y = rng.standard_normal((len(pos), O.HEAD_DIM))
    ours = O.rope(y, pos)
    # exact check of the pairing and direction: Llama's rotation fed fp64 angles laid
    # out as it lays them out (the frequencies repeated over both halves)
    ang = pos[:, None].astype(np.float64) * np.concatenate([O.rope_inv_freq()] * 2)[None, :]
    yt = torch.from_numpy(y)[:, None, :]                    # [N, 1 head, D]
    cos = torch.from_numpy(np.cos(ang))
    sin = torch.from_numpy(np.sin(ang))
    q_rot, _ = apply_rotary_pos_emb(yt, yt, cos, sin, unsqueeze_dim=1)
    assert np.max(np.abs(ours - q_rot[:, 0].numpy())) < 1e-12
    # end to end with the library's own (fp32) cos/sin at these positions
    _, c32, s32 = _llama_rotary(pos.tolist(), torch.float32)
    q32, _ = apply_rotary_pos_emb(yt.float(), yt.float(), c32, s32, unsqueeze_dim=1)
    assert np.max(np.abs(ours - q32[:, 0].double().numpy())) < 1e-3


def test_per_head_rms_norm_with_one_weight_matches_qwen3_q_norm():
    from transformers.models.qwen3.modeling_qwen3 import Qwen3RMSNorm

    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, O.NUM_Q_HEADS, O.HEAD_DIM))
    w = 1.0 + 0.1 * rng.standard_normal(O.HEAD_DIM)
    ours = O.rms_norm(x, w[None, None, :])
    norm = Qwen3RMSNorm(O.HEAD_DIM, eps=O.RMS_EPS)
    with torch.no_grad():
        norm.weight.copy_(torch.from_numpy(w).float())
        ref = norm(torch.from_numpy(x).float()).double().numpy()    # computes in fp32
    assert np.max(np.abs(ours - ref) / (np.abs(ours) + 1e-3)) < 1e-5
