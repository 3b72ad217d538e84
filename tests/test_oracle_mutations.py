"""Plants plausible mistakes in the oracle (on the CPU) and checks that a pin catches
each one: a pin that passes for a wrong oracle would pin nothing."""

import numpy as np
import pytest

import oracle.beam_oracle as B
import tests.test_oracle_pins as pins

try:  # the convention pins need the transformers library; the other pins do not
    import tests.test_oracle_conventions as conv
except pytest.skip.Exception:
    conv = None


def _window_off_by_one(pos, kind, window=B.WINDOW):
    if kind == B.KIND_FULL:
        return 0, int(pos)
    return max(0, int(pos) - window), int(pos)


def _attend_wrong_group(q_hat, k, v, sm_scale=B.SM_SCALE):
    R, Hq, D = q_hat.shape
    Hkv = k.shape[1]
    o = np.empty((R, Hq, D))
    for h in range(Hq):
        g = h % Hkv
        z = sm_scale * (q_hat[:, h, :] @ k[:, g, :].T)
        o[:, h, :] = B.softmax(z) @ v[:, g, :]
    return o


def _rope_wrong_sign(y, pos, theta=B.ROPE_THETA):
    y = np.asarray(y, dtype=np.float64)
    half = y.shape[-1] // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * B.rope_inv_freq(y.shape[-1], theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = y[..., :half], y[..., half:]
    return np.concatenate([a * c + b * s, b * c - a * s], axis=-1)


def _rope_wrong_freq(y, pos, theta=B.ROPE_THETA):
    y = np.asarray(y, dtype=np.float64)
    half = y.shape[-1] // 2
    i = np.arange(half, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * np.power(theta, -i / half / 2)
    c, s = np.cos(ang), np.sin(ang)
    a, b = y[..., :half], y[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _ssmax_zero_based(p, base=B.SSMAX_BASE, exponent=B.SSMAX_EXPONENT):
    return np.power(1.0 + (np.asarray(p, dtype=np.float64) - 1) / base, exponent)


def _rms_no_eps(x, w, eps=B.RMS_EPS):
    x = np.asarray(x, dtype=np.float64)
    return np.asarray(w, dtype=np.float64) * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))


def _gate_minus_bias(o, gate_bits, bias_bits):
    o = np.asarray(o, dtype=np.float64)
    N, Hq, D = o.shape
    gate = B.bf16_bits_to_f64(gate_bits).reshape(N, Hq, D)
    bias = B.bf16_bits_to_f64(bias_bits).reshape(1, Hq, 1)
    return o * B.sigmoid(gate - bias)


def _e4m3_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), B.E4M3_MAX)
    vals = B._E4M3_POS_VALUES
    hi = np.clip(np.searchsorted(vals, ax, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    pick_lo = (ax - vals[lo]) < (vals[hi] - ax)
    mag = np.where(pick_lo, lo, hi).astype(np.uint8)
    return (mag | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def _bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def _store_binary32_quotient(cache, block_table, seq, pos, values_bits, kv_dtype, scale=1.0):
    out = np.array(cache, copy=True)
    page, slot = B.physical_slot(block_table, seq, pos)
    if kv_dtype == "bf16":
        out[page, :, slot, :] = np.asarray(values_bits, dtype=np.uint16)
    else:
        q = B.bf16_bits_to_f64(values_bits).astype(np.float32) / np.float32(scale)
        out[page, :, slot, :] = B.f64_to_e4m3(q.astype(np.float64))
    return out


def _prepare(x_bits, w_bits, pos, kind, is_query, order):
    """prepare_qk with the sliding-layer steps in a wrong order: 'rotate-first' applies
    RoPE before the norm, 'round-between' rounds to bf16 after the norm and again after
    the rotation."""
    x = B.bf16_bits_to_f64(x_bits)
    w = B.bf16_bits_to_f64(w_bits)
    w = w[None, None, :] if w.ndim == 1 else w[None, :, :]
    pos = np.asarray(pos, dtype=np.int64)
    if kind != B.KIND_SWA:
        y = B.rms_norm(x, w)
        if is_query:
            y = y * B.ssmax_scale(pos + 1)[:, None, None]
        return B.f64_to_bf16_bits(y)
    if order == "rotate-first":
        y = B.rms_norm(B.rope(x, pos[:, None]), w)
    else:
        y = B.rope(B.bf16_round(B.rms_norm(x, w)), pos[:, None])
    return B.f64_to_bf16_bits(y)


_ORIG_BF16_ROUND = B.bf16_round


def _bf16_round_via_binary32(x):
    return _ORIG_BF16_ROUND(np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64))


def _rope_interleaved_pairs(y, pos, theta=B.ROPE_THETA):
    # pairs (2i, 2i + 1) instead of (i, i + D/2)
    y = np.asarray(y, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * B.rope_inv_freq(y.shape[-1], theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = y[..., 0::2], y[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def _inv_freq_over_half_dim(head_dim=B.HEAD_DIM, theta=B.ROPE_THETA):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(theta, -i / head_dim)


def _rms_over_all_heads(x, w, eps=B.RMS_EPS):
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=(-2, -1), keepdims=True)
    return np.asarray(w, dtype=np.float64) * x / np.sqrt(ms + eps)


MUTATIONS = [
    ("store_kv", _store_binary32_quotient, pins.test_fp8_store_is_nearest_e4m3_of_exact_quotient),
    ("prepare_qk", lambda *a, **k: _prepare(*a, order="rotate-first"),
     pins.test_prepare_k_sliding_layer_is_norm_then_rotation_then_one_rounding),
    ("prepare_qk", lambda *a, **k: _prepare(*a, order="round-between"),
     pins.test_prepare_k_sliding_layer_is_norm_then_rotation_then_one_rounding),
    ("bf16_round", _bf16_round_via_binary32, pins.test_bf16_round_of_f64_is_one_rounding),
    ("visible_range", _window_off_by_one, pins.test_window_equals_full_up_to_512_keys_and_differs_after),
    ("attend", _attend_wrong_group, pins.test_attention_matches_sdpa_textbook_routine),
    ("rope", _rope_wrong_sign, lambda: pins.test_rope_frequencies_and_direction(16, 0.1)),
    ("rope", _rope_wrong_freq, lambda: pins.test_rope_frequencies_and_direction(16, 0.1)),
    ("ssmax_scale", _ssmax_zero_based, pins.test_prepare_q_full_layer_scales_by_ssmax_of_one_based_position),
    ("rms_norm", _rms_no_eps, pins.test_rms_norm_matches_torch),
    ("head_gate", _gate_minus_bias, pins.test_gate_bias_switches_heads_off_and_on),
    ("f64_to_e4m3", _e4m3_ties_away, pins.test_e4m3_encode_all_bf16_inputs_match_torch_after_clamp),
    ("bf16_round", _bf16_truncate, pins.test_bf16_round_matches_torch_cast),
    ("SM_SCALE", 1.0 / 128.0, pins.test_attention_matches_sdpa_textbook_routine),
]
if conv is not None:
    MUTATIONS += [
        ("visible_range", _window_off_by_one, conv.test_sliding_window_and_causal_visibility_match_transformers_masks),
        ("attend", _attend_wrong_group, conv.test_query_heads_read_kv_heads_as_repeat_kv_maps_them),
        ("rope", _rope_wrong_sign, conv.test_rope_rotation_matches_llama_apply_rotary_pos_emb),
        ("rope", _rope_interleaved_pairs, conv.test_rope_rotation_matches_llama_apply_rotary_pos_emb),
        ("rope_inv_freq", _inv_freq_over_half_dim, conv.test_rope_frequencies_match_llama_rotary_embedding),
        ("rms_norm", _rms_over_all_heads, conv.test_per_head_rms_norm_with_one_weight_matches_qwen3_q_norm),
    ]


@pytest.mark.parametrize("name,bad,pin", MUTATIONS, ids=[f"{m[0]}-{i}" for i, m in enumerate(MUTATIONS)])
def test_pin_catches_planted_mistake(monkeypatch, name, bad, pin):
    if name == "SM_SCALE":
        # default arguments captured the constant: patch the functions' defaults
        monkeypatch.setattr(B.attend, "__defaults__", (bad,))
        monkeypatch.setattr(B.attention_rows, "__defaults__", (1.0, 1.0, bad, B.WINDOW))
    else:
        monkeypatch.setattr(B, name, bad)
    with pytest.raises(AssertionError):
        pin()
